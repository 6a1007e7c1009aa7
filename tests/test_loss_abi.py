"""Host-side tests of the sequence-tiled loss's C ABI (no GPU): the
workspace planner holds one tile of [T, vocab] buffers and the weight-sized
accumulator, and every argument check returns its status before any HIP
call."""
import ctypes

import pytest

import headwise_chunked_context_amd as hc_amd
from headwise_chunked_context_amd import binding as B

P = 0x7F0000000000
WS = 0x7F1000000000


def _ws(L, D, V, T, pss):
    out = ctypes.c_size_t(0)
    rc = hc_amd.lib().upipe_loss_workspace_bytes(L, D, V, T, pss, ctypes.byref(out))
    return rc, out.value


def test_workspace_holds_no_fp32_logits():
    """Forward: per row of the tile, one (max, sum) fp32 pair per 256-column
    tile of the vocabulary and the target's logit, plus 4 bytes per position
    (the per-row loss): the logits themselves stay in the GEMM's registers.
    Backward: one tile of bf16 dlogits [T, V], s fp32 [T, D] slices when the
    dh GEMM (output [T, D], reduction over V) has fewer than 256 output
    tiles of 256 x 256 (s = min(ceil(256 / tiles), V / 512)), the fp32 dW
    accumulator (4 V D bytes) and one fp32 scale.  Nothing of size L x V."""
    up = lambda v: (v + 255) // 256 * 256
    L, D, V = 32768, 4096, 128256
    nct = -(-V // 256)

    def slices(T):
        tiles = -(-T // 256) * -(-D // 256)
        return 0 if tiles >= 256 else max(1, min(-(-256 // tiles), V // 512))

    for T in (1, 100, 2048, 4096, 32768):
        fwd = up(T * nct * 8) + up(T * 4) + up(L * 4)
        s = slices(T)
        bwd = up(T * V * 2) + (up(s * T * D * 4) if s > 1 else 0) + up(V * D * 4) + 256
        assert _ws(L, D, V, T, B.PASS_FWD) == (B.UPIPE_OK, fwd), T
        assert _ws(L, D, V, T, B.PASS_BWD) == (B.UPIPE_OK, bwd), T
        # the fused pass holds both (its [T, V] 2-byte tile serves as fp16
        # logits, then bf16 dlogits)
        fused = fwd + bwd
        assert _ws(L, D, V, T, B.PASS_FWD_BWD) == (B.UPIPE_OK, fused), T
    assert _ws(1000, D, V, 5000, B.PASS_FWD) == _ws(1000, D, V, 1000, B.PASS_FWD)
    # against the whole sequence's fp32 logits (16.8 GB at L 32768): the
    # forward at tile 4096 keeps under 0.1% of that, the backward's bf16 tile
    # an eighth
    assert _ws(L, D, V, 4096, B.PASS_FWD)[1] < L * V * 4 / 1000
    assert up(4096 * V * 2) <= L * V * 4 / 16


@pytest.mark.parametrize("args,code", [
    ((1000, 256, 1024, 256, 0), B.UPIPE_OK),
    ((1000, 256, 1024, 256, 1), B.UPIPE_OK),
    ((0, 256, 1024, 256, 0), B.UPIPE_EINVAL),
    ((1000, 256, 1024, 0, 0), B.UPIPE_EINVAL),
    ((1000, 0, 1024, 256, 0), B.UPIPE_EINVAL),
    ((1000, 256, 0, 256, 0), B.UPIPE_EINVAL),
    ((1000, 256, 1024, 256, 2), B.UPIPE_EINVAL),          # no recompute pass here
    ((1000, 200, 1024, 256, 0), B.UPIPE_EUNSUPPORTED),    # hidden % 128
    ((1000, 256, 50257, 256, 0), B.UPIPE_EUNSUPPORTED),   # vocab % 128 (pad it)
    (((1 << 24) + 1, 256, 1024, 256, 0), B.UPIPE_EUNSUPPORTED),
    ((1000, 1 << 16, 1 << 17, 256, 0), B.UPIPE_EUNSUPPORTED),  # hidden * vocab >= 2^33
])
def test_workspace_query_status(args, code):
    assert _ws(*args)[0] == code


def _fwd(**kw):
    a = dict(L=1000, D=256, V=1024, T=256, h=P, w=P, t=P, ign=-100, loss=P, lse=P, ws=WS,
             wsb=1 << 40)
    a.update(kw)
    return hc_amd.lib().upipe_loss_fwd(a["L"], a["D"], a["V"], a["T"], a["h"], a["w"], a["t"],
                                       a["ign"], a["loss"], a["lse"], a["ws"], a["wsb"], None)


def _bwd(**kw):
    a = dict(L=1000, D=256, V=1024, T=256, h=P, w=P, t=P, ign=-100, lse=P, dloss=1.0, dh=P, dw=P,
             ws=WS, wsb=1 << 40)
    a.update(kw)
    return hc_amd.lib().upipe_loss_bwd(a["L"], a["D"], a["V"], a["T"], a["h"], a["w"], a["t"],
                                       a["ign"], a["lse"], a["dloss"], a["dh"], a["dw"], a["ws"],
                                       a["wsb"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(h=None), B.UPIPE_EINVAL),
    (dict(w=None), B.UPIPE_EINVAL),
    (dict(t=None), B.UPIPE_EINVAL),
    (dict(loss=None), B.UPIPE_EINVAL),
    (dict(lse=None), B.UPIPE_EINVAL),
    (dict(h=P + 2), B.UPIPE_EINVAL),              # bf16 data not 16-byte aligned
    (dict(t=P + 2), B.UPIPE_EINVAL),              # int32 data not 4-byte aligned
    (dict(lse=P + 1), B.UPIPE_EINVAL),
    (dict(ws=None), B.UPIPE_EWORKSPACE),
    (dict(ws=WS + 64), B.UPIPE_EWORKSPACE),
    (dict(wsb=1000), B.UPIPE_EWORKSPACE),
    (dict(V=1000), B.UPIPE_EUNSUPPORTED),
    (dict(T=0), B.UPIPE_EINVAL),
])
def test_forward_checks_before_any_gpu_work(kw, code):
    assert _fwd(**kw) == code


@pytest.mark.parametrize("kw,code", [
    (dict(lse=None), B.UPIPE_EINVAL),
    (dict(dh=None), B.UPIPE_EINVAL),
    (dict(dw=None), B.UPIPE_EINVAL),
    (dict(dw=P + 8), B.UPIPE_EINVAL),
    (dict(wsb=_ws(1000, 256, 1024, 256, B.PASS_FWD)[1]), B.UPIPE_EWORKSPACE),  # forward size
    (dict(D=100), B.UPIPE_EUNSUPPORTED),
])
def test_backward_checks_before_any_gpu_work(kw, code):
    assert _bwd(**kw) == code


def _fused(**kw):
    a = dict(L=1000, D=256, V=1024, T=256, h=P, w=P, t=P, ign=-100, dloss=1.0, loss=P, lse=P, dh=P,
             dw=P, ws=WS, wsb=1 << 40)
    a.update(kw)
    return hc_amd.lib().upipe_loss_fwd_bwd(a["L"], a["D"], a["V"], a["T"], a["h"], a["w"], a["t"],
                                           a["ign"], a["dloss"], a["loss"], a["lse"], a["dh"],
                                           a["dw"], a["ws"], a["wsb"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(h=None), B.UPIPE_EINVAL),
    (dict(loss=None), B.UPIPE_EINVAL),
    (dict(lse=None), B.UPIPE_EINVAL),
    (dict(dh=None), B.UPIPE_EINVAL),
    (dict(dw=None), B.UPIPE_EINVAL),
    (dict(dh=P + 8), B.UPIPE_EINVAL),
    (dict(lse=P + 2), B.UPIPE_EINVAL),
    (dict(wsb=_ws(1000, 256, 1024, 256, B.PASS_BWD)[1]), B.UPIPE_EWORKSPACE),  # backward size
    (dict(ws=WS + 64), B.UPIPE_EWORKSPACE),
    (dict(V=1000), B.UPIPE_EUNSUPPORTED),
    (dict(T=0), B.UPIPE_EINVAL),
])
def test_fused_checks_before_any_gpu_work(kw, code):
    assert _fused(**kw) == code


def test_binding_checks_shapes_before_the_library():
    import torch

    h = torch.zeros(10, 128, dtype=torch.bfloat16)
    w = torch.zeros(256, 128, dtype=torch.bfloat16)
    t = torch.zeros(10, dtype=torch.int32)
    with pytest.raises(ValueError):
        hc_amd.loss_fwd(h, w, t, 4)                   # host tensors
    with pytest.raises(ValueError):
        hc_amd.loss_fwd(h, w, t[:-1], 4)              # one target per row


def test_choose_tile_takes_the_longest_tile_that_fits():
    L, D, V = 32768, 4096, 128256
    for budget, pss in ((8 << 20, B.PASS_FWD), (64 << 20, B.PASS_FWD), (3 << 30, B.PASS_BWD),
                        (64 << 30, B.PASS_BWD)):
        t, b = hc_amd.loss_choose_tile(L, D, V, budget, pss)
        assert b <= budget and _ws(L, D, V, t, pss) == (B.UPIPE_OK, b)
        assert t % 256 == 0 or t == L
        for t2 in range(t + 256, L + 256, 256):
            assert _ws(L, D, V, min(t2, L), pss)[1] > budget
    with pytest.raises(B.UpipeError):
        hc_amd.loss_choose_tile(L, D, V, 64 << 10, B.PASS_FWD)      # nothing fits
