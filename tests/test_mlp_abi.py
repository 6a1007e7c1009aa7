"""Host-side tests of the sequence-tiled SwiGLU MLP's C ABI (no GPU): the
workspace planner is affine in the tile and every argument check returns its
status before any HIP call."""
import ctypes

import pytest

import headwise_chunked_context_amd as hc_amd
from headwise_chunked_context_amd import binding as B

P = 0x7F0000000000
WS = 0x7F1000000000


def _ws(L, D, F, T, pss):
    out = ctypes.c_size_t(0)
    rc = hc_amd.lib().upipe_mlp_workspace_bytes(L, D, F, T, pss, ctypes.byref(out))
    return rc, out.value


def test_workspace_is_one_tile_of_intermediates_plus_weight_accumulators():
    """Forward: [T, 2F] (h | u) and [T, F] (a) bf16, plus s fp32 [T, D]
    slices when the tile is too short for the hidden-wide GEMMs (output
    [T, D], reduction K = F forward, 2F backward) to fill 256 CUs with
    256 x 256 output tiles: their reduction is split in s = min(ceil(256 /
    tiles), K / 512) parts.  The backward adds the fp32 gradient
    accumulators of both weights (12 D F bytes), independent of L and T.  A
    tile longer than the sequence is the sequence."""
    up = lambda v: (v + 255) // 256 * 256
    L, D, F = 32768, 4096, 14336

    def slices(T, K):
        tiles = -(-T // 256) * -(-D // 256)
        return 0 if tiles >= 256 else max(1, min(-(-256 // tiles), K // 512))

    for T in (1, 100, 2048, 8192, 32768):
        base = up(T * 2 * F * 2) + up(T * F * 2)
        sf, sb = slices(T, F), slices(T, 2 * F)
        fwd = base + (up(sf * T * D * 4) if sf > 1 else 0)
        bwd = base + (up(sb * T * D * 4) if sb > 1 else 0) + 12 * D * F
        assert _ws(L, D, F, T, B.PASS_FWD) == (B.UPIPE_OK, fwd), T
        assert _ws(L, D, F, T, B.PASS_BWD) == (B.UPIPE_OK, bwd), T
    assert _ws(1000, D, F, 5000, B.PASS_FWD) == _ws(1000, D, F, 1000, B.PASS_FWD)
    # the whole-sequence intermediates a tile avoids: at L 32768, tile 8192
    # keeps a quarter of them
    q = _ws(L, D, F, 8192, B.PASS_FWD)[1] / _ws(L, D, F, L, B.PASS_FWD)[1]
    assert abs(q - 0.25) < 1e-6


@pytest.mark.parametrize("args,code", [
    ((1000, 512, 1536, 256, 0), B.UPIPE_OK),
    ((1000, 512, 1536, 256, 1), B.UPIPE_OK),
    ((0, 512, 1536, 256, 0), B.UPIPE_EINVAL),
    ((1000, 512, 1536, 0, 0), B.UPIPE_EINVAL),
    ((1000, 0, 1536, 256, 0), B.UPIPE_EINVAL),
    ((1000, 512, 1536, 256, 2), B.UPIPE_EINVAL),          # no recompute pass here
    ((1000, 500, 1536, 256, 0), B.UPIPE_EUNSUPPORTED),    # hidden % 128
    ((1000, 512, 1000, 256, 0), B.UPIPE_EUNSUPPORTED),    # ffn % 128
    (((1 << 24) + 1, 512, 1536, 256, 0), B.UPIPE_EUNSUPPORTED),
    ((1000, 1 << 17, 1 << 16, 256, 0), B.UPIPE_EUNSUPPORTED),  # hidden * ffn >= 2^33
])
def test_workspace_query_status(args, code):
    assert _ws(*args)[0] == code


def _fwd(**kw):
    a = dict(L=1000, D=512, F=1536, T=256, x=P, wgu=P, wd=P, y=P, ws=WS, wsb=1 << 40)
    a.update(kw)
    return hc_amd.lib().upipe_mlp_fwd(a["L"], a["D"], a["F"], a["T"], a["x"], a["wgu"], a["wd"],
                                      a["y"], a["ws"], a["wsb"], None)


def _bwd(**kw):
    a = dict(L=1000, D=512, F=1536, T=256, x=P, wgu=P, wd=P, dy=P, dx=P, dwgu=P, dwd=P,
             ws=WS, wsb=1 << 40)
    a.update(kw)
    return hc_amd.lib().upipe_mlp_bwd(a["L"], a["D"], a["F"], a["T"], a["x"], a["wgu"], a["wd"],
                                      a["dy"], a["dx"], a["dwgu"], a["dwd"], a["ws"], a["wsb"],
                                      None)


@pytest.mark.parametrize("kw,code", [
    (dict(x=None), B.UPIPE_EINVAL),
    (dict(wgu=None), B.UPIPE_EINVAL),
    (dict(wd=None), B.UPIPE_EINVAL),
    (dict(y=None), B.UPIPE_EINVAL),
    (dict(x=P + 2), B.UPIPE_EINVAL),              # misaligned
    (dict(ws=None), B.UPIPE_EWORKSPACE),
    (dict(ws=WS + 64), B.UPIPE_EWORKSPACE),       # not 256-byte aligned
    (dict(wsb=1000), B.UPIPE_EWORKSPACE),
    (dict(D=500), B.UPIPE_EUNSUPPORTED),
    (dict(T=0), B.UPIPE_EINVAL),
])
def test_forward_checks_before_any_gpu_work(kw, code):
    assert _fwd(**kw) == code


@pytest.mark.parametrize("kw,code", [
    (dict(dy=None), B.UPIPE_EINVAL),
    (dict(dx=None), B.UPIPE_EINVAL),
    (dict(dwgu=None), B.UPIPE_EINVAL),
    (dict(dwd=None), B.UPIPE_EINVAL),
    (dict(dwd=P + 8), B.UPIPE_EINVAL),
    (dict(wsb=_ws(1000, 512, 1536, 256, B.PASS_FWD)[1]), B.UPIPE_EWORKSPACE),  # forward size
    (dict(F=1000), B.UPIPE_EUNSUPPORTED),
])
def test_backward_checks_before_any_gpu_work(kw, code):
    assert _bwd(**kw) == code


def test_binding_checks_shapes_before_the_library():
    import torch

    x = torch.zeros(10, 128, dtype=torch.bfloat16)
    wgu = torch.zeros(256, 128, dtype=torch.bfloat16)
    wd = torch.zeros(128, 128, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        hc_amd.mlp_fwd(x, wgu, wd, 4)                 # host tensors
    with pytest.raises(ValueError):
        hc_amd.mlp_fwd(x, wgu[:-1], wd, 4)            # gate/up rows != 2 ffn


def test_choose_tile_takes_the_longest_tile_that_fits():
    L, D, F = 32768, 4096, 14336
    for budget in (100 << 20, 500 << 20, 2 << 30, 64 << 30):
        t, b = hc_amd.mlp_choose_tile(L, D, F, budget, B.PASS_BWD if budget > (2 << 30) else B.PASS_FWD)
        pss = B.PASS_BWD if budget > (2 << 30) else B.PASS_FWD
        assert b <= budget and _ws(L, D, F, t, pss) == (B.UPIPE_OK, b)
        assert t % 256 == 0 or t == L
        # no longer candidate fits
        for t2 in range(t + 256, L + 256, 256):
            assert _ws(L, D, F, min(t2, L), pss)[1] > budget
    with pytest.raises(B.UpipeError):
        hc_amd.mlp_choose_tile(L, D, F, 1 << 20, B.PASS_FWD)       # nothing fits
