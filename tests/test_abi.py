"""Host-side tests of the C ABI (no GPU): the library loads, exports every
declared entry point, and every argument check returns its status before any
HIP call; the workspace planner is affine in the head chunk."""
import ctypes
import json
import os
import re

import pytest

import headwise_chunked_context_amd as hc_amd
from headwise_chunked_context_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", h) for h in sorted(os.listdir(os.path.join(ROOT, "include")))
           if h.endswith(".h")]

# fake, 256-byte aligned device addresses: never dereferenced by the host
P = 0x7F0000000000
WS = 0x7F1000000000


def _declared_functions():
    names = set()
    for h in HEADERS:
        text = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names |= set(re.findall(r"\b(upipe_\w+)\s*\(", text))
    return sorted(names)


def test_library_exports_every_declared_function():
    lib = hc_amd.lib()
    names = _declared_functions()
    assert set(names) == set(B.EXPORTS), names
    for n in names:
        assert hasattr(lib, n), n
    assert lib.upipe_version() >= 100


def test_strerror_covers_every_status():
    seen = set()
    for code in (0, -1, -2, -3, -4, -5, -6):
        msg = hc_amd.strerror(code)
        assert msg and msg not in seen
        seen.add(msg)
    assert hc_amd.strerror(12345) == "unknown status"


def _ws(L, D, nq, nkv, d, hc, pss):
    out = ctypes.c_size_t(0)
    rc = hc_amd.lib().upipe_attn_workspace_bytes(L, D, nq, nkv, d, hc, pss, ctypes.byref(out))
    return rc, out.value


@pytest.mark.parametrize("args,code", [
    ((1024, 1024, 8, 2, 128, 2, 0), B.UPIPE_OK),
    ((0, 1024, 8, 2, 128, 2, 0), B.UPIPE_EINVAL),            # L = 0
    ((-5, 1024, 8, 2, 128, 2, 0), B.UPIPE_EINVAL),
    ((1024, -128, 8, 2, 128, 2, 0), B.UPIPE_EINVAL),
    ((1024, 1024, 8, 3, 128, 2, 0), B.UPIPE_EINVAL),         # Hq % Hkv
    ((1024, 1024, 0, 1, 128, 1, 0), B.UPIPE_EINVAL),
    ((1024, 1024, 8, 2, 64, 2, 0), B.UPIPE_EUNSUPPORTED),    # head_dim
    ((1024, 1000, 8, 2, 128, 2, 0), B.UPIPE_EUNSUPPORTED),   # hidden % 128
    (((1 << 24) + 1, 0, 4, 1, 128, 1, 0), B.UPIPE_EUNSUPPORTED),
    ((1024, 1024, 8, 2, 128, 3, 0), B.UPIPE_ECHUNK),         # does not divide Hq
    ((1024, 1536, 12, 3, 128, 6, 1), B.UPIPE_ECHUNK),        # G = 4, chunk 6 straddles
    ((1024, 1024, 8, 2, 128, 0, 0), B.UPIPE_EINVAL),
    ((1024, 1024, 8, 2, 128, 2, 7), B.UPIPE_EINVAL),         # bad pass
    # launch grids of 2^32 threads or more are refused on the host
    ((1 << 24, 16384, 32, 32, 128, 32, 1), B.UPIPE_OK),      # the documented sufficient bound
    ((1 << 24, 0, 32, 32, 128, 32, 0), B.UPIPE_OK),
    ((1 << 24, 0, 128, 128, 128, 128, 0), B.UPIPE_EUNSUPPORTED),  # L_256 * chunk = 2^31
    ((1 << 24, 0, 64, 64, 128, 64, 0), B.UPIPE_EUNSUPPORTED),     # L_256 * kc = 2^30
    ((1 << 24, 32768, 8, 8, 128, 1, 0), B.UPIPE_EUNSUPPORTED),    # L_256 * hidden = 2^39
    ((4096, 1 << 22, 64, 64, 128, 64, 1), B.UPIPE_EUNSUPPORTED),  # hidden * w > 2^34
    ((1024, 1024, 8, 2, 128, 2, 5), B.UPIPE_EINVAL),
    ((1024, 1024, 8, 2, 128, 2, -1), B.UPIPE_EINVAL),
    ((1024, 1024, 8, 2, 128, 2, 4), B.UPIPE_OK),             # pipelined backward
    ((1024, 0, 8, 2, 128, 2, 4), B.UPIPE_OK),
    ((1024, 0, 8, 2, 128, 2, 3), B.UPIPE_OK),                # pipelined forward
    ((1024, 1024, 8, 2, 128, 2, 2), B.UPIPE_OK),             # recompute backward
    ((1024, 0, 8, 2, 128, 2, 2), B.UPIPE_EINVAL),            # ... needs projection mode
])
def test_workspace_query_status(args, code):
    rc, _ = _ws(*args)
    assert rc == code


def test_workspace_query_null_output():
    rc = hc_amd.lib().upipe_attn_workspace_bytes(1024, 1024, 8, 2, 128, 2, 0, None)
    assert rc == B.UPIPE_EINVAL


@pytest.mark.parametrize("pss", [B.PASS_FWD, B.PASS_BWD, B.PASS_BWD_RECOMPUTE, B.PASS_FWD_PIPELINED,
                                 B.PASS_BWD_PIPELINED])
@pytest.mark.parametrize("shape", [(262144, 5120, 8, 1), (524288, 0, 4, 1), (32768, 4096, 32, 8)])
def test_workspace_affine_and_shrinking_in_chunk(shape, pss):
    L, D, nq, nkv = shape
    if pss == B.PASS_BWD_RECOMPUTE and D == 0:
        pytest.skip("the recompute backward exists in projection mode only")
    G = nq // nkv
    chunks = [c for c in (1, 2, 4, 8, 16, 32) if nq % c == 0 and (c % G == 0 or G % c == 0)]
    sizes = {c: _ws(L, D, nq, nkv, 128, c, pss)[1] for c in chunks}
    for a, b in zip(chunks, chunks[1:]):
        assert sizes[a] < sizes[b]
    # affine within each regime: chunks below the group size touch one KV head,
    # chunks of whole groups touch c/G KV heads (still linear in c)
    lo = [c for c in chunks if c <= G]
    hi = [c for c in chunks if c >= G]
    for grp in (lo, hi):
        if len(grp) >= 3:
            slopes = [(sizes[b] - sizes[a]) / (b - a) for a, b in zip(grp, grp[1:])]
            assert max(slopes) == min(slopes), slopes


def _per_q_head_bytes(L, D, pss):
    """Bytes of the workspace buffers that exist once per query head of a
    chunk, counted buffer by buffer from what each pass holds per q head
    (Lp = L rounded up to 256, d = 128):
      forward:  rotated q [Lp, d] bf16; the projection's q columns of the
                staging block [L, d] bf16 (projection mode)
      backward: rotated q and dO [Lp, d] bf16 each; the base-2 LSE and
                D = dO . O rows [Lp] fp32 each; the dq columns of the
                staging block [L, d] bf16 and the chunk's dW_qkv rows of the
                fp32 weight-gradient accumulator [d, D] (projection mode)."""
    Lp, d = -(-L // 256) * 256, 128
    if pss == B.PASS_FWD:
        return 2 * Lp * d + (2 * L * d if D else 0)
    return 2 * (2 * Lp * d) + 2 * (4 * Lp) + ((2 * L * d + 4 * d * D) if D else 0)


def test_query_side_reduction_matches_page_figure():
    """The 32B-share shape (8 q heads, 1 KV head per GPU): the planner's
    growth from chunk 1 to chunk 8 is exactly seven sets of the per-q-head
    buffers counted one by one, so chunk 1 keeps 1/8 of the q-side
    intermediates of chunk 8 (the page's 87.5%), while the resident KV
    group, which chunking cannot shrink, keeps the whole workspace's cut
    below that figure."""
    fig = json.load(open(os.path.join(ROOT, "tests", "golden", "page_figures.json")))
    want = fig["attention_intermediate_reduction_32b"]["value"]
    L, D = 262144, 5120
    for pss in (B.PASS_FWD, B.PASS_BWD):
        s = {c: _ws(L, D, 8, 1, 128, c, pss)[1] for c in (1, 2, 4, 8)}
        per_head = _per_q_head_bytes(L, D, pss)
        for c in (2, 4, 8):
            assert s[c] - s[1] == (c - 1) * per_head, (pss, c)
        q1, q8 = 1 * per_head, 8 * per_head
        assert abs((1 - q1 / q8) - want) < 1e-12
        whole = 1 - s[1] / s[8]
        assert 0 < whole < want, whole
    lo, hi = fig["chunk_sizes_ablated"]["value"]
    assert _ws(L, D, 32, 1, 128, lo, 0)[1] < _ws(L, D, 32, 1, 128, hi, 0)[1]


def _fwd(**kw):
    a = dict(L=1024, D=1024, nq=8, nkv=2, d=128, theta=5e5, hc=2,
             x=P, wqkv=P, wo=P, y=P, o=P, lse=P, ws=WS, wsb=1 << 40)
    a.update(kw)
    return hc_amd.lib().upipe_attn_fwd(a["L"], a["D"], a["nq"], a["nkv"], a["d"], a["theta"],
                                       a["hc"], a["x"], a["wqkv"], a["wo"], a["y"], a["o"],
                                       a["lse"], a["ws"], a["wsb"], None)


def _bwd(**kw):
    a = dict(L=1024, D=1024, nq=8, nkv=2, d=128, theta=5e5, hc=2, x=P, wqkv=P, wo=P, o=P,
             lse=P, dy=P, dx=P, dwqkv=P, dwo=P, ws=WS, wsb=1 << 40)
    a.update(kw)
    return hc_amd.lib().upipe_attn_bwd(a["L"], a["D"], a["nq"], a["nkv"], a["d"], a["theta"],
                                       a["hc"], a["x"], a["wqkv"], a["wo"], a["o"], a["lse"],
                                       a["dy"], a["dx"], a["dwqkv"], a["dwo"], a["ws"], a["wsb"],
                                       None)


@pytest.mark.parametrize("kw,code", [
    (dict(x=None), B.UPIPE_EINVAL),
    (dict(wo=None), B.UPIPE_EINVAL),                 # projection mode needs both weights
    (dict(y=None), B.UPIPE_EINVAL),
    (dict(o=None), B.UPIPE_EINVAL),
    (dict(lse=None), B.UPIPE_EINVAL),
    (dict(x=P + 2), B.UPIPE_EINVAL),                 # misaligned
    (dict(theta=0.0), B.UPIPE_EINVAL),
    (dict(theta=float("nan")), B.UPIPE_EINVAL),
    (dict(ws=None), B.UPIPE_EWORKSPACE),
    (dict(ws=WS + 16), B.UPIPE_EWORKSPACE),          # not 256-byte aligned
    (dict(wsb=1024), B.UPIPE_EWORKSPACE),            # too small
    (dict(hc=3), B.UPIPE_ECHUNK),
    (dict(d=96), B.UPIPE_EUNSUPPORTED),
    (dict(D=0, wqkv=None, wo=None), B.UPIPE_EINVAL),  # q/k/v-given mode must not get y
    (dict(L=0), B.UPIPE_EINVAL),
])
def test_fwd_rejects_before_launch(kw, code):
    assert _fwd(**kw) == code


@pytest.mark.parametrize("kw,code", [
    (dict(dy=None), B.UPIPE_EINVAL),
    (dict(dx=None), B.UPIPE_EINVAL),
    (dict(dwo=None), B.UPIPE_EINVAL),
    (dict(D=0, wqkv=None, wo=None), B.UPIPE_EINVAL),   # weight grads must be NULL then
    (dict(lse=P + 4), B.UPIPE_EINVAL),
    (dict(wsb=0), B.UPIPE_EWORKSPACE),
    (dict(nkv=3), B.UPIPE_EINVAL),
    (dict(hc=16), B.UPIPE_ECHUNK),
])
def test_bwd_rejects_before_launch(kw, code):
    assert _bwd(**kw) == code


def test_exact_workspace_size_is_accepted_by_the_check():
    # one byte short of the query is rejected; the check runs before any launch
    rc, need = _ws(1024, 1024, 8, 2, 128, 2, B.PASS_BWD)
    assert rc == 0 and need > 0
    assert _bwd(wsb=need - 1) == B.UPIPE_EWORKSPACE


@pytest.mark.parametrize("L,hc", [(1000, 1), (1024, 2), (4097, 8)])
def test_recompute_workspace_adds_chunk_output_and_v_tiles(L, hc):
    """The recompute backward needs the chunk's attention output [L][hc*128]
    bf16 and the V tiles of the KV heads it touches [kc][Lp][128] fp16 on top
    of the ordinary backward's workspace (each buffer 256-byte aligned)."""
    nq, nkv = 8, 2
    G = nq // nkv
    kc = hc // G if hc >= G else 1
    Lp = (L + 255) // 256 * 256
    up = lambda v: (v + 255) // 256 * 256
    _, base = _ws(L, 1024, nq, nkv, 128, hc, B.PASS_BWD)
    _, rec = _ws(L, 1024, nq, nkv, 128, hc, B.PASS_BWD_RECOMPUTE)
    assert rec - base == up(L * hc * 128 * 2) + up(kc * Lp * 128 * 2)


def test_bwd_recompute_argument_checks():
    # o_saved = NULL selects the recompute backward: projection mode only
    assert _bwd(o=None, D=0, wqkv=None, wo=None, dwqkv=None, dwo=None) == B.UPIPE_EINVAL
    # ... and it needs the larger workspace
    _, base = _ws(1024, 1024, 8, 2, 128, 2, B.PASS_BWD)
    _, rec = _ws(1024, 1024, 8, 2, 128, 2, B.PASS_BWD_RECOMPUTE)
    assert _bwd(o=None, wsb=base) == B.UPIPE_EWORKSPACE
    assert _bwd(o=None, wsb=rec - 1) == B.UPIPE_EWORKSPACE
    assert _bwd(o=None, lse=None, wsb=rec) == B.UPIPE_EINVAL   # the saved LSE is still needed
    # with o_saved given, the ordinary workspace suffices
    assert _bwd(wsb=base - 1) == B.UPIPE_EWORKSPACE


def test_pipelined_forward_workspace_and_check():
    """Pipelining adds a second slot of q [hc][Lp][128] and k, v [kc][Lp][128]
    (bf16/fp16) to the forward workspace, and while it is enabled the forward
    rejects a workspace of the one-slot size before any launch."""
    L, hc, nq, nkv = 1000, 2, 8, 2
    Lp = 1024
    up = lambda v: (v + 255) // 256 * 256
    _, one = _ws(L, 1024, nq, nkv, 128, hc, B.PASS_FWD)
    _, two = _ws(L, 1024, nq, nkv, 128, hc, B.PASS_FWD_PIPELINED)
    assert two - one == up(hc * Lp * 256) + 2 * up(1 * Lp * 256)
    try:
        hc_amd.pipeline_enable(True)
        assert hc_amd.fwd_pass() == B.PASS_FWD_PIPELINED
        assert _fwd(L=L, wsb=one) == B.UPIPE_EWORKSPACE
        assert _fwd(L=L, wsb=two, o=None) == B.UPIPE_EINVAL
    finally:
        hc_amd.pipeline_enable(False)
    assert hc_amd.fwd_pass() == B.PASS_FWD
    assert _fwd(L=L, wsb=one - 1) == B.UPIPE_EWORKSPACE


def test_pipelined_backward_workspace_and_check():
    """The pipelined backward's second slot holds q [hc][Lp][128], k and v
    [kc][Lp][128], dO [hc][Lp][128] (bf16), the LSE2 and D rows [hc][Lp]
    (fp32), the staging block [L][(hc+2kc)128] (bf16) and the weight-gradient
    accumulator [(hc+2kc)128][hidden] (fp32); while pipelining is enabled the
    saved-output backward needs it and the recompute backward does not."""
    L, D, hc, nq, nkv = 1000, 1024, 2, 8, 2
    Lp, kc, w = 1024, 1, (2 + 2) * 128
    up = lambda v: (v + 255) // 256 * 256
    _, one = _ws(L, D, nq, nkv, 128, hc, B.PASS_BWD)
    _, two = _ws(L, D, nq, nkv, 128, hc, B.PASS_BWD_PIPELINED)
    assert two - one == (up(hc * Lp * 256) + 2 * up(kc * Lp * 256) + up(hc * Lp * 256)
                         + 2 * up(hc * Lp * 4) + up(L * w * 2) + up(w * D * 4))
    try:
        hc_amd.pipeline_enable(True)
        assert hc_amd.bwd_pass() == B.PASS_BWD_PIPELINED
        assert hc_amd.bwd_pass(recompute=True) == B.PASS_BWD_RECOMPUTE
        assert _bwd(L=L, wsb=one) == B.UPIPE_EWORKSPACE
        assert _bwd(L=L, wsb=two, dx=None) == B.UPIPE_EINVAL
        _, rec = _ws(L, D, nq, nkv, 128, hc, B.PASS_BWD_RECOMPUTE)
        assert _bwd(L=L, wsb=rec - 1, o=None) == B.UPIPE_EWORKSPACE
    finally:
        hc_amd.pipeline_enable(False)
    assert hc_amd.bwd_pass() == B.PASS_BWD
    assert _bwd(L=L, wsb=one - 1) == B.UPIPE_EWORKSPACE


def test_binding_refuses_host_tensors_before_any_call():
    """The binding validates tensors before it reaches the library: host
    tensors are refused (no pointer of them ever reaches a kernel)."""
    import torch

    x = torch.zeros(16, 128, dtype=torch.bfloat16)
    wq = torch.zeros(3 * 128, 128, dtype=torch.bfloat16)
    wo = torch.zeros(128, 128, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        hc_amd.attn_fwd(x, wq, wo, 1, 1, 1, 5e5)
    with pytest.raises(ValueError):
        hc_amd.attn_fwd(x, wq, None, 1, 1, 1, 5e5)   # weights come together


def test_profile_mask_bounds():
    """upipe_profile_enable takes a class mask in 0 .. UPIPE_PROFILE_ALL and
    refuses anything else; reading a class outside the eight is refused too
    (host-side state only, no GPU needed)."""
    L = B.lib()
    assert L.upipe_profile_enable(-1) == B.UPIPE_EINVAL
    assert L.upipe_profile_enable(B.PROFILE_ALL + 1) == B.UPIPE_EINVAL
    assert L.upipe_profile_enable(1 << B.KERNEL_KINDS["attn_bwd_dkdv"]) == B.UPIPE_OK
    ms, n = ctypes.c_double(-1), ctypes.c_int64(-1)
    assert L.upipe_profile_read(len(B.KERNEL_KINDS), ctypes.byref(ms), ctypes.byref(n)) == B.UPIPE_EINVAL
    assert L.upipe_profile_read(-1, ctypes.byref(ms), ctypes.byref(n)) == B.UPIPE_EINVAL
    assert L.upipe_profile_read(1, ctypes.byref(ms), ctypes.byref(n)) == B.UPIPE_OK
    assert (ms.value, n.value) == (0.0, 0)
    assert L.upipe_profile_enable(0) == B.UPIPE_OK


def test_bench_refuses_more_than_one_gpu():
    """bench.py measures one GPU's share only: --gpus N > 1 exits non-zero
    with a message (before touching a GPU)."""
    import subprocess
    import sys

    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    res = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=120)
    assert res.returncode != 0
    assert "one GPU" in (res.stdout + res.stderr)


def _fwd_static(**kw):
    a = dict(L=1024, D=1024, nq=8, nkv=2, d=128, theta=5e5, hc=2,
             x=P, wqkv=P, wo=P, y=P, o=P, lse=P)
    a.update(kw)
    return hc_amd.lib().upipe_attn_fwd_static(a["L"], a["D"], a["nq"], a["nkv"], a["d"],
                                              a["theta"], a["hc"], a["x"], a["wqkv"], a["wo"],
                                              a["y"], a["o"], a["lse"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(L=32768, D=4096, nq=32, nkv=8, hc=16), B.UPIPE_ESCRATCH),   # 384 MiB > 256 MiB
    (dict(L=524288, D=0, nq=4, nkv=1, hc=1, wqkv=None, wo=None, y=None), B.UPIPE_ESCRATCH),
    (dict(hc=3), B.UPIPE_ECHUNK),
    (dict(o=None), B.UPIPE_EINVAL),
    (dict(lse=None), B.UPIPE_EINVAL),
    (dict(y=None), B.UPIPE_EINVAL),                     # projection mode needs y
    (dict(wo=None), B.UPIPE_EINVAL),
    (dict(theta=-1.0), B.UPIPE_EINVAL),
    (dict(x=P + 8), B.UPIPE_EINVAL),                    # misaligned
])
def test_static_forward_checks_before_any_gpu_work(kw, code):
    """The allocation-free forward refuses bad arguments, and shapes whose
    workspace exceeds its static scratch, on the host (no GPU here)."""
    assert _fwd_static(**kw) == code


def test_static_scratch_limit_covers_the_benchmarked_forward():
    """L 32768, hidden 4096, 32 q / 8 KV heads: chunk 8 fits the scratch,
    chunk 16 does not."""
    assert _ws(32768, 4096, 32, 8, 128, 8, B.PASS_FWD)[1] <= B.STATIC_SCRATCH_BYTES
    assert _ws(32768, 4096, 32, 8, 128, 16, B.PASS_FWD)[1] > B.STATIC_SCRATCH_BYTES


def test_debug_mode_switch_is_host_only():
    """upipe_debug_enable only sets host state (no GPU here)."""
    L = B.lib()
    assert L.upipe_debug_enable(1) == B.UPIPE_OK
    assert L.upipe_debug_enable(0) == B.UPIPE_OK


@pytest.mark.parametrize("shape", [(262144, 5120, 8, 1), (32768, 4096, 32, 8), (524288, 0, 4, 1)])
def test_choose_chunk_takes_the_largest_chunk_that_fits(shape):
    """The chunk that fits a memory budget (chunk-size ablation paragraph):
    the largest valid chunk whose workspace is within the budget."""
    L, D, nq, nkv = shape
    G = nq // nkv
    valid = [c for c in range(1, nq + 1) if nq % c == 0 and (c % G == 0 or G % c == 0)]
    sizes = {c: _ws(L, D, nq, nkv, 128, c, B.PASS_BWD)[1] for c in valid}
    for c in valid:
        got = hc_amd.choose_chunk(L, D, nq, nkv, sizes[c], B.PASS_BWD)
        assert got == (c, sizes[c])
        if c > 1:
            assert hc_amd.choose_chunk(L, D, nq, nkv, sizes[c] - 1, B.PASS_BWD)[0] < c
    with pytest.raises(B.UpipeError) as e:
        hc_amd.choose_chunk(L, D, nq, nkv, sizes[valid[0]] - 1, B.PASS_BWD)
    assert e.value.status == B.UPIPE_EWORKSPACE
    with pytest.raises(B.UpipeError) as e:
        hc_amd.choose_chunk(L, D, nq, nkv, 1 << 40, 7)
    assert e.value.status == B.UPIPE_EINVAL


def test_autograd_wrappers_import_without_gpu():
    """The autograd module imports on a host without a GPU and exposes one
    torch.autograd.Function per forward / backward pair."""
    import torch

    from headwise_chunked_context_amd import autograd as ag

    for f in (ag._Attention, ag._SwiGluMlp, ag._CrossEntropy):
        assert issubclass(f, torch.autograd.Function)
    for fn in (ag.attention, ag.swiglu_mlp, ag.cross_entropy):
        assert callable(fn)
