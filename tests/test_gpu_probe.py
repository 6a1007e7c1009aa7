"""The MFMA probe on the GPU (MI355X only): it runs, its clock readings are
consistent, and the rate it implies lies between a third of the published
2.5 PFLOP/s bf16 peak and that peak (plus a margin for the published figure's
rounding)."""
import pytest

pytestmark = pytest.mark.gpu


def test_probe_rate_and_clock_are_plausible():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import headwise_chunked_context_amd as lib

    g = torch.Generator(device="cuda:0").manual_seed(7)
    ops = torch.randn(8 << 20, generator=g, device="cuda:0").to(torch.bfloat16)   # 16 MiB
    wg, iters = 512, 2000
    lib.probe_mfma(ops, 10, wg)                                                   # warm-up
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    sink, clocks = lib.probe_mfma(ops, iters, wg)
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1)
    tflops = wg * 4 * iters * lib.binding.PROBE_FLOP_PER_ROUND / (ms * 1e-3) / 1e12
    ck = clocks.view(-1, 2).double()
    assert bool((ck > 0).all())
    ghz = float((ck[:, 0] / ck[:, 1]).mean()) * 0.1
    print(f"probe: {tflops:.0f} TFLOP/s at {ghz:.2f} GHz ({ms:.2f} ms)", flush=True)
    assert bool(torch.isfinite(sink).all())
    assert 800.0 < tflops < 2600.0
    assert 0.8 < ghz < 2.6
