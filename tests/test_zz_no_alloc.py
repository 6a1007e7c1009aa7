"""The allocation-free forward (upipe_attn_fwd_static, the library's static
device scratch in place of a workspace) against upipe_attn_fwd, through the
C ABI, on two calls in a row, the second with a smaller input."""
import numpy as np
import pytest

import oracle
import synthetic
from _helpers import f64, from_dev_bf16, from_dev_f32, max_abs, rel_l2, to_dev

pytestmark = pytest.mark.gpu

FWD_MAX_ABS, FWD_REL = 2e-2, 1e-2
LSE_ABS, LSE_REL = 2e-2, 2e-3


def test_static_scratch_forward_equals_workspace_forward():
    import torch

    import headwise_chunked_context_amd as lib

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    base = synthetic.WORKLOADS[1]
    shapes = [
        base.with_(L=1500, hidden=1024, n_q=8, n_kv=2, head_chunk=4),   # first call
        base.with_(L=333, hidden=1024, n_q=8, n_kv=2, head_chunk=4),    # smaller input
        base.with_(L=700, hidden=0, n_q=4, n_kv=1, head_chunk=1),       # q/k/v given
    ]
    for w in shapes:
        inp = synthetic.make_inputs(w, with_grad=False)
        x, wq, wo = (to_dev(inp[k]) for k in ("x", "w_qkv", "w_o"))
        ref = lib.attn_fwd(x, wq, wo, w.n_q, w.n_kv, w.head_chunk, w.theta)
        got = lib.attn_fwd_static(x, wq, wo, w.n_q, w.n_kv, w.head_chunk, w.theta)
        torch.cuda.synchronize()
        for name, a, b in zip(("y", "o", "lse"), ref, got):
            if a is None:
                assert b is None
                continue
            bits = (lambda t: t.view(torch.int16)) if a.dtype == torch.bfloat16 else (
                lambda t: t.view(torch.int32))
            same = torch.equal(bits(a), bits(b))
            print(f"static scratch L={w.L} hidden={w.hidden} hc={w.head_chunk}: {name} "
                  f"bitwise equal = {same}", flush=True)
            assert same, name
        # and the oracle's bar on the static call's own result
        ry, ro, rl = oracle.layer_fwd(f64(inp["x"]), f64(inp["w_qkv"]), f64(inp["w_o"]), w.n_q,
                                      w.n_kv, w.head_dim, w.theta, w.head_chunk)
        out = from_dev_bf16(got[0]) if w.hidden else from_dev_bf16(got[1])
        want = ry if w.hidden else ro
        lse_x = float(np.max(np.abs(from_dev_f32(got[2]) - rl) / (LSE_ABS + LSE_REL * np.abs(rl))))
        print(f"  vs oracle: out max {max_abs(out, want):.3e} rel {rel_l2(out, want):.3e} "
              f"lse gate {lse_x:.2f}", flush=True)
        assert max_abs(out, want) <= FWD_MAX_ABS and rel_l2(out, want) <= FWD_REL
        assert lse_x <= 1.0


def test_static_scratch_refuses_oversized_shapes():
    """Beyond the 256 MiB scratch the call returns UPIPE_ESCRATCH before any
    GPU work, and the workspace entry point still runs those shapes."""
    import torch

    import headwise_chunked_context_amd as lib

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    L, D, nq, nkv = 32768, 4096, 32, 8
    need = lib.workspace_bytes(L, D, nq, nkv, 128, 16, lib.PASS_FWD)
    assert need > lib.STATIC_SCRATCH_BYTES
    x = torch.zeros(L, D, dtype=torch.bfloat16, device="cuda:0")
    wq = torch.zeros((nq + 2 * nkv) * 128, D, dtype=torch.bfloat16, device="cuda:0")
    wo = torch.zeros(D, nq * 128, dtype=torch.bfloat16, device="cuda:0")
    with pytest.raises(lib.UpipeError) as e:
        lib.attn_fwd_static(x, wq, wo, nq, nkv, 16, 5e5)
    assert e.value.status == lib.UPIPE_ESCRATCH
    torch.cuda.synchronize()
