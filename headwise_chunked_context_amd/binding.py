"""ctypes binding of libupipe_attn.so (argument marshalling only).

Every step of the layer runs in the HIP library; this module only turns torch
tensors into device pointers, allocates outputs and the workspace with torch,
and raises on a non-zero status.  If the library is missing it fails loudly:
there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libupipe_attn.so")

UPIPE_OK = 0
UPIPE_EINVAL = -1
UPIPE_EUNSUPPORTED = -2
UPIPE_ECHUNK = -3
UPIPE_EWORKSPACE = -4
UPIPE_EHIP = -5
UPIPE_ESCRATCH = -6
STATIC_SCRATCH_BYTES = 256 << 20
PASS_FWD = 0
PASS_BWD = 1
PASS_BWD_RECOMPUTE = 2
PASS_FWD_PIPELINED = 3
PASS_BWD_PIPELINED = 4
PASS_FWD_BWD = 5   # the loss's fused forward-backward
_pipeline = False

# names declared in include/upipe_attn.h, include/upipe_mlp.h,
# include/upipe_loss.h and include/upipe_probe.h
EXPORTS = (
    "upipe_attn_workspace_bytes",
    "upipe_attn_fwd",
    "upipe_attn_fwd_static",
    "upipe_attn_bwd",
    "upipe_attn_choose_chunk",
    "upipe_mlp_workspace_bytes",
    "upipe_mlp_choose_tile",
    "upipe_mlp_fwd",
    "upipe_mlp_bwd",
    "upipe_loss_workspace_bytes",
    "upipe_loss_choose_tile",
    "upipe_loss_fwd",
    "upipe_loss_bwd",
    "upipe_loss_fwd_bwd",
    "upipe_probe_mfma",
    "upipe_profile_enable",
    "upipe_profile_read",
    "upipe_pipeline_enable",
    "upipe_debug_enable",
    "upipe_last_hip_error",
    "upipe_last_hip_error_string",
    "upipe_strerror",
    "upipe_version",
)

KERNEL_KINDS = {"attn_fwd": 0, "attn_bwd_dkdv": 1, "attn_bwd_dq": 2, "gemm": 3, "prep": 4,
                "finalize": 5, "gemm_accum": 6, "prep_dout": 7}


class UpipeError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = f"{where}: status {status}: {strerror(status)}"
        if status == UPIPE_EHIP:
            self.hip_error = lib().upipe_last_hip_error()
            msg += f" (HIP error {self.hip_error}: {lib().upipe_last_hip_error_string().decode()})"
        super().__init__(msg)


_lib = None


def lib() -> ctypes.CDLL:
    """Load the in-tree HIP library (raises if it was not built).

    torch is imported first.  A process holds one HIP runtime per soname:
    torch ships its own libamdhip64.so.7, and the library, linked against
    the system ROCm's, must bind to that same copy.  Loaded the other way
    round, the system copy comes up next to torch's as a second runtime that
    may not see the GPU (measured: "no ROCm-capable device", while torch's
    copy works), and every launch of the library fails."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is missing: build it with `python -m headwise_chunked_context_amd.build`"
        )
    import torch  # noqa: F401  (its HIP runtime first; see above)

    L = ctypes.CDLL(LIB_PATH)
    i64, i32, f64, sz = ctypes.c_int64, ctypes.c_int32, ctypes.c_double, ctypes.c_size_t
    vp = ctypes.c_void_p
    L.upipe_attn_workspace_bytes.argtypes = [i64, i32, i32, i32, i32, i32, i32, ctypes.POINTER(sz)]
    L.upipe_attn_workspace_bytes.restype = ctypes.c_int
    L.upipe_attn_fwd.argtypes = [i64, i32, i32, i32, i32, f64, i32,
                                 vp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.upipe_attn_fwd.restype = ctypes.c_int
    L.upipe_attn_fwd_static.argtypes = [i64, i32, i32, i32, i32, f64, i32,
                                        vp, vp, vp, vp, vp, vp, vp]
    L.upipe_attn_fwd_static.restype = ctypes.c_int
    L.upipe_attn_bwd.argtypes = [i64, i32, i32, i32, i32, f64, i32,
                                 vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.upipe_attn_bwd.restype = ctypes.c_int
    L.upipe_attn_choose_chunk.argtypes = [i64, i32, i32, i32, i32, i32, sz, ctypes.POINTER(i32),
                                          ctypes.POINTER(sz)]
    L.upipe_attn_choose_chunk.restype = ctypes.c_int
    L.upipe_mlp_choose_tile.argtypes = [i64, i32, i32, i32, sz, ctypes.POINTER(i32), ctypes.POINTER(sz)]
    L.upipe_mlp_choose_tile.restype = ctypes.c_int
    L.upipe_mlp_workspace_bytes.argtypes = [i64, i32, i32, i32, i32, ctypes.POINTER(sz)]
    L.upipe_mlp_workspace_bytes.restype = ctypes.c_int
    L.upipe_mlp_fwd.argtypes = [i64, i32, i32, i32, vp, vp, vp, vp, vp, sz, vp]
    L.upipe_mlp_fwd.restype = ctypes.c_int
    L.upipe_mlp_bwd.argtypes = [i64, i32, i32, i32, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.upipe_mlp_bwd.restype = ctypes.c_int
    L.upipe_loss_choose_tile.argtypes = [i64, i32, i32, i32, sz, ctypes.POINTER(i32), ctypes.POINTER(sz)]
    L.upipe_loss_choose_tile.restype = ctypes.c_int
    L.upipe_loss_workspace_bytes.argtypes = [i64, i32, i32, i32, i32, ctypes.POINTER(sz)]
    L.upipe_loss_workspace_bytes.restype = ctypes.c_int
    L.upipe_loss_fwd.argtypes = [i64, i32, i32, i32, vp, vp, vp, i32, vp, vp, vp, sz, vp]
    L.upipe_loss_fwd.restype = ctypes.c_int
    L.upipe_loss_bwd.argtypes = [i64, i32, i32, i32, vp, vp, vp, i32, vp, ctypes.c_float, vp, vp,
                                 vp, sz, vp]
    L.upipe_loss_bwd.restype = ctypes.c_int
    L.upipe_loss_fwd_bwd.argtypes = [i64, i32, i32, i32, vp, vp, vp, i32, ctypes.c_float, vp, vp,
                                     vp, vp, vp, sz, vp]
    L.upipe_loss_fwd_bwd.restype = ctypes.c_int
    L.upipe_probe_mfma.argtypes = [vp, sz, i32, i32, vp, vp, vp]
    L.upipe_probe_mfma.restype = ctypes.c_int
    L.upipe_strerror.argtypes = [ctypes.c_int]
    L.upipe_strerror.restype = ctypes.c_char_p
    L.upipe_version.argtypes = []
    L.upipe_version.restype = ctypes.c_int
    L.upipe_profile_enable.argtypes = [ctypes.c_int]
    L.upipe_profile_enable.restype = ctypes.c_int
    L.upipe_profile_read.argtypes = [ctypes.c_int, ctypes.POINTER(ctypes.c_double),
                                     ctypes.POINTER(ctypes.c_int64)]
    L.upipe_profile_read.restype = ctypes.c_int
    L.upipe_pipeline_enable.argtypes = [ctypes.c_int]
    L.upipe_pipeline_enable.restype = ctypes.c_int
    L.upipe_debug_enable.argtypes = [ctypes.c_int]
    L.upipe_debug_enable.restype = ctypes.c_int
    L.upipe_last_hip_error.argtypes = []
    L.upipe_last_hip_error.restype = ctypes.c_int
    L.upipe_last_hip_error_string.argtypes = []
    L.upipe_last_hip_error_string.restype = ctypes.c_char_p
    _lib = L
    return L


def strerror(status: int) -> str:
    return lib().upipe_strerror(int(status)).decode()


def workspace_bytes(L: int, hidden: int, n_q: int, n_kv: int, head_dim: int, head_chunk: int,
                    pass_: int) -> int:
    out = ctypes.c_size_t(0)
    rc = lib().upipe_attn_workspace_bytes(L, hidden, n_q, n_kv, head_dim, head_chunk, pass_,
                                          ctypes.byref(out))
    if rc != UPIPE_OK:
        raise UpipeError(rc, "upipe_attn_workspace_bytes")
    return out.value


def pipeline_enable(on: bool) -> None:
    """Two-slot pipelining of the forward and the saved-output backward on a
    second stream (default off; needs the PASS_*_PIPELINED workspaces while
    on)."""
    global _pipeline
    rc = lib().upipe_pipeline_enable(1 if on else 0)
    if rc != UPIPE_OK:
        raise UpipeError(rc, "upipe_pipeline_enable")
    _pipeline = bool(on)


def choose_chunk(L: int, hidden: int, n_q: int, n_kv: int, budget_bytes: int, pass_: int,
                 head_dim: int = 128):
    """(head_chunk, workspace bytes): the largest chunk whose workspace fits."""
    c, b = ctypes.c_int32(0), ctypes.c_size_t(0)
    rc = lib().upipe_attn_choose_chunk(L, hidden, n_q, n_kv, head_dim, pass_, budget_bytes,
                                       ctypes.byref(c), ctypes.byref(b))
    if rc != UPIPE_OK:
        raise UpipeError(rc, "upipe_attn_choose_chunk")
    return c.value, b.value


def debug_enable(on: bool) -> None:
    """Debug mode: the library NaN-fills each chunk's (or MLP tile's)
    workspace buffers before writing them, so stale reads show as NaN."""
    rc = lib().upipe_debug_enable(1 if on else 0)
    if rc != UPIPE_OK:
        raise UpipeError(rc, "upipe_debug_enable")


def pipeline_enabled() -> bool:
    """Whether two-slot pipelining is on (as set through pipeline_enable)."""
    return _pipeline


def fwd_pass() -> int:
    """Workspace pass of upipe_attn_fwd under the current pipelining setting."""
    return PASS_FWD_PIPELINED if _pipeline else PASS_FWD


def bwd_pass(recompute: bool = False) -> int:
    """Workspace pass of upipe_attn_bwd under the current pipelining setting
    (the full-recompute backward is never pipelined)."""
    if recompute:
        return PASS_BWD_RECOMPUTE
    return PASS_BWD_PIPELINED if _pipeline else PASS_BWD


PROFILE_ALL = 0xFF


def profile_enable(on: bool, kinds=None) -> None:
    """Start (clearing old records) or stop per-kernel-class event timing.
    kinds: the KERNEL_KINDS names whose launches are bracketed (default: all)."""
    if not on:
        mask = 0
    elif kinds is None:
        mask = PROFILE_ALL
    else:
        mask = 0
        for k in kinds:
            mask |= 1 << KERNEL_KINDS[k]
    rc = lib().upipe_profile_enable(mask)
    if rc != UPIPE_OK:
        raise UpipeError(rc, "upipe_profile_enable")


def profile_read() -> dict:
    """{kind: (total_ms, launches)} since the last profile_enable(True)."""
    out = {}
    for name, kind in KERNEL_KINDS.items():
        ms, n = ctypes.c_double(0), ctypes.c_int64(0)
        rc = lib().upipe_profile_read(kind, ctypes.byref(ms), ctypes.byref(n))
        if rc != UPIPE_OK:
            raise UpipeError(rc, "upipe_profile_read")
        out[name] = (ms.value, n.value)
    return out


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _check(t, name: str, shape: tuple, dtype, device=None):
    """The library sees only a pointer: the tensor must be a contiguous
    device tensor of exactly this shape and dtype (a wrong extent would make
    the kernels read or write outside it)."""
    if t is None:
        raise ValueError(f"{name} is required")
    if not t.is_cuda or (device is not None and t.device != device):
        raise ValueError(f"{name} must be on the GPU device of x")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _check_inputs(x, w_qkv, w_o, n_q: int, n_kv: int, head_dim: int):
    import torch

    bf = torch.bfloat16
    if x is None or x.dim() != 2:
        raise ValueError("x must be a 2-D tensor")
    L = x.shape[0]
    if (w_qkv is None) != (w_o is None):
        raise ValueError("w_qkv and w_o are given together (projection mode) or not at all")
    if w_qkv is not None:
        hidden = x.shape[1]
        _check(x, "x", (L, hidden), bf)
        _check(w_qkv, "w_qkv", ((n_q + 2 * n_kv) * head_dim, hidden), bf, x.device)
        _check(w_o, "w_o", (hidden, n_q * head_dim), bf, x.device)
    else:
        _check(x, "x (packed q|k|v)", (L, (n_q + 2 * n_kv) * head_dim), bf)
    return L


def _stream(stream):
    import torch

    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _workspace(nbytes: int, device, workspace):
    import torch

    if workspace is not None:
        if not workspace.is_cuda or workspace.device != device or not workspace.is_contiguous():
            raise ValueError("workspace must be a contiguous tensor on the device of x")
        return workspace
    # 256-byte aligned by the caching allocator
    return torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)


def attn_fwd(x, w_qkv, w_o, n_q: int, n_kv: int, head_chunk: int, theta: float,
             head_dim: int = 128, workspace=None, stream=None):
    """Forward of the chunked layer.  Returns (y or None, o_saved, lse).

    x: bf16 [L, hidden] (projection mode) or packed q|k|v [L, (Hq+2Hkv)d]
    when w_qkv is None.
    """
    import torch

    L = _check_inputs(x, w_qkv, w_o, n_q, n_kv, head_dim)
    proj = w_qkv is not None
    hidden = x.shape[1] if proj else 0
    dev = x.device
    y = torch.empty(L, hidden, dtype=torch.bfloat16, device=dev) if proj else None
    o_saved = torch.empty(L, n_q * head_dim, dtype=torch.bfloat16, device=dev)
    lse = torch.empty(n_q, L, dtype=torch.float32, device=dev)
    ws_n = workspace_bytes(L, hidden, n_q, n_kv, head_dim, head_chunk, fwd_pass())
    ws = _workspace(ws_n, dev, workspace)
    rc = lib().upipe_attn_fwd(L, hidden, n_q, n_kv, head_dim, float(theta), head_chunk,
                              _ptr(x), _ptr(w_qkv), _ptr(w_o), _ptr(y), _ptr(o_saved), _ptr(lse),
                              _ptr(ws), ws.numel() * ws.element_size(), _stream(stream))
    if rc != UPIPE_OK:
        raise UpipeError(rc, "upipe_attn_fwd")
    return y, o_saved, lse


def attn_fwd_static(x, w_qkv, w_o, n_q: int, n_kv: int, head_chunk: int, theta: float,
                    head_dim: int = 128, out=None, stream=None):
    """Forward through the allocation-free entry point (the library's static
    scratch instead of a workspace).  Returns (y or None, o_saved, lse);
    out=(y, o_saved, lse) reuses caller-allocated outputs, so a call then
    allocates nothing at all."""
    import torch

    L = _check_inputs(x, w_qkv, w_o, n_q, n_kv, head_dim)
    proj = w_qkv is not None
    hidden = x.shape[1] if proj else 0
    dev = x.device
    if out is None:
        y = torch.empty(L, hidden, dtype=torch.bfloat16, device=dev) if proj else None
        o_saved = torch.empty(L, n_q * head_dim, dtype=torch.bfloat16, device=dev)
        lse = torch.empty(n_q, L, dtype=torch.float32, device=dev)
    else:
        y, o_saved, lse = out
        if proj:
            _check(y, "y", (L, hidden), torch.bfloat16, dev)
        _check(o_saved, "o_saved", (L, n_q * head_dim), torch.bfloat16, dev)
        _check(lse, "lse", (n_q, L), torch.float32, dev)
    rc = lib().upipe_attn_fwd_static(L, hidden, n_q, n_kv, head_dim, float(theta), head_chunk,
                                     _ptr(x), _ptr(w_qkv), _ptr(w_o), _ptr(y), _ptr(o_saved),
                                     _ptr(lse), _stream(stream))
    if rc != UPIPE_OK:
        raise UpipeError(rc, "upipe_attn_fwd_static")
    return y, o_saved, lse


def attn_bwd(x, w_qkv, w_o, o_saved, lse, dy, n_q: int, n_kv: int, head_chunk: int,
             theta: float, head_dim: int = 128, workspace=None, stream=None):
    """Backward of the chunked layer.  Returns (dx, dw_qkv, dw_o); in q/k/v-given
    mode dx is dqkv and the weight gradients are None.  With o_saved=None
    (projection mode only) each chunk's attention output is recomputed."""
    import torch

    L = _check_inputs(x, w_qkv, w_o, n_q, n_kv, head_dim)
    proj = w_qkv is not None
    hidden = x.shape[1] if proj else 0
    dev = x.device
    if o_saved is not None:
        _check(o_saved, "o_saved", (L, n_q * head_dim), torch.bfloat16, dev)
    _check(lse, "lse", (n_q, L), torch.float32, dev)
    _check(dy, "dy", (L, hidden if proj else n_q * head_dim), torch.bfloat16, dev)
    dx = torch.empty_like(x)
    dw_qkv = torch.empty_like(w_qkv) if proj else None
    dw_o = torch.empty_like(w_o) if proj else None
    pass_ = bwd_pass(recompute=o_saved is None)
    ws_n = workspace_bytes(L, hidden, n_q, n_kv, head_dim, head_chunk, pass_)
    ws = _workspace(ws_n, dev, workspace)
    rc = lib().upipe_attn_bwd(L, hidden, n_q, n_kv, head_dim, float(theta), head_chunk,
                              _ptr(x), _ptr(w_qkv), _ptr(w_o), _ptr(o_saved), _ptr(lse), _ptr(dy),
                              _ptr(dx), _ptr(dw_qkv), _ptr(dw_o),
                              _ptr(ws), ws.numel() * ws.element_size(), _stream(stream))
    if rc != UPIPE_OK:
        raise UpipeError(rc, "upipe_attn_bwd")
    return dx, dw_qkv, dw_o


# ---------------------------------------------------------------- SwiGLU MLP
def mlp_choose_tile(L: int, hidden: int, ffn: int, budget_bytes: int, pass_: int):
    """(tile_rows, workspace bytes): the longest tile whose workspace fits."""
    t, b = ctypes.c_int32(0), ctypes.c_size_t(0)
    rc = lib().upipe_mlp_choose_tile(L, hidden, ffn, pass_, budget_bytes, ctypes.byref(t),
                                     ctypes.byref(b))
    if rc != UPIPE_OK:
        raise UpipeError(rc, "upipe_mlp_choose_tile")
    return t.value, b.value


def mlp_workspace_bytes(L: int, hidden: int, ffn: int, tile_rows: int, pass_: int) -> int:
    out = ctypes.c_size_t(0)
    rc = lib().upipe_mlp_workspace_bytes(L, hidden, ffn, tile_rows, pass_, ctypes.byref(out))
    if rc != UPIPE_OK:
        raise UpipeError(rc, "upipe_mlp_workspace_bytes")
    return out.value


def _check_mlp(x, w_gate_up, w_down):
    import torch

    bf = torch.bfloat16
    if x is None or x.dim() != 2:
        raise ValueError("x must be a 2-D tensor")
    L, hidden = x.shape
    if w_down is None or w_down.dim() != 2:
        raise ValueError("w_down must be a 2-D tensor")
    ffn = w_down.shape[1]
    _check(x, "x", (L, hidden), bf)
    _check(w_gate_up, "w_gate_up", (2 * ffn, hidden), bf, x.device)
    _check(w_down, "w_down", (hidden, ffn), bf, x.device)
    return L, hidden, ffn


def mlp_fwd(x, w_gate_up, w_down, tile_rows: int, workspace=None, stream=None):
    """Sequence-tiled SwiGLU MLP forward: y = (silu(x Wg^T) * x Wu^T) Wd^T,
    w_gate_up = [Wg; Wu] (gate rows first).  Returns y."""
    import torch

    L, hidden, ffn = _check_mlp(x, w_gate_up, w_down)
    y = torch.empty(L, hidden, dtype=torch.bfloat16, device=x.device)
    ws = _workspace(mlp_workspace_bytes(L, hidden, ffn, tile_rows, PASS_FWD), x.device, workspace)
    rc = lib().upipe_mlp_fwd(L, hidden, ffn, tile_rows, _ptr(x), _ptr(w_gate_up), _ptr(w_down),
                             _ptr(y), _ptr(ws), ws.numel() * ws.element_size(), _stream(stream))
    if rc != UPIPE_OK:
        raise UpipeError(rc, "upipe_mlp_fwd")
    return y


def mlp_bwd(x, w_gate_up, w_down, dy, tile_rows: int, workspace=None, stream=None):
    """Backward of mlp_fwd.  Returns (dx, dw_gate_up, dw_down)."""
    import torch

    L, hidden, ffn = _check_mlp(x, w_gate_up, w_down)
    _check(dy, "dy", (L, hidden), torch.bfloat16, x.device)
    dx = torch.empty_like(x)
    dwgu = torch.empty_like(w_gate_up)
    dwd = torch.empty_like(w_down)
    ws = _workspace(mlp_workspace_bytes(L, hidden, ffn, tile_rows, PASS_BWD), x.device, workspace)
    rc = lib().upipe_mlp_bwd(L, hidden, ffn, tile_rows, _ptr(x), _ptr(w_gate_up), _ptr(w_down),
                             _ptr(dy), _ptr(dx), _ptr(dwgu), _ptr(dwd), _ptr(ws),
                             ws.numel() * ws.element_size(), _stream(stream))
    if rc != UPIPE_OK:
        raise UpipeError(rc, "upipe_mlp_bwd")
    return dx, dwgu, dwd


# ---------------------------------------------------------------- tiled loss
def loss_choose_tile(L: int, hidden: int, vocab: int, budget_bytes: int, pass_: int):
    """(tile_rows, workspace bytes): the longest tile whose workspace fits."""
    t, b = ctypes.c_int32(0), ctypes.c_size_t(0)
    rc = lib().upipe_loss_choose_tile(L, hidden, vocab, pass_, budget_bytes, ctypes.byref(t),
                                      ctypes.byref(b))
    if rc != UPIPE_OK:
        raise UpipeError(rc, "upipe_loss_choose_tile")
    return t.value, b.value


def loss_workspace_bytes(L: int, hidden: int, vocab: int, tile_rows: int, pass_: int) -> int:
    out = ctypes.c_size_t(0)
    rc = lib().upipe_loss_workspace_bytes(L, hidden, vocab, tile_rows, pass_, ctypes.byref(out))
    if rc != UPIPE_OK:
        raise UpipeError(rc, "upipe_loss_workspace_bytes")
    return out.value


def _check_loss(h, w, targets):
    import torch

    if h is None or h.dim() != 2:
        raise ValueError("h must be a 2-D tensor")
    L, hidden = h.shape
    if w is None or w.dim() != 2:
        raise ValueError("w must be a 2-D tensor")
    vocab = w.shape[0]
    _check(h, "h", (L, hidden), torch.bfloat16)
    _check(w, "w", (vocab, hidden), torch.bfloat16, h.device)
    _check(targets, "targets", (L,), torch.int32, h.device)
    return L, hidden, vocab


def loss_fwd(h, w, targets, tile_rows: int, ignore_index: int = -100, workspace=None, stream=None):
    """Sequence-tiled mean cross-entropy of logits = h w^T against targets
    (rows with ignore_index do not count).  Returns (loss [1] fp32, lse [L]
    fp32)."""
    import torch

    L, hidden, vocab = _check_loss(h, w, targets)
    loss = torch.empty(1, dtype=torch.float32, device=h.device)
    lse = torch.empty(L, dtype=torch.float32, device=h.device)
    ws = _workspace(loss_workspace_bytes(L, hidden, vocab, tile_rows, PASS_FWD), h.device, workspace)
    rc = lib().upipe_loss_fwd(L, hidden, vocab, tile_rows, _ptr(h), _ptr(w), _ptr(targets),
                              ignore_index, _ptr(loss), _ptr(lse), _ptr(ws),
                              ws.numel() * ws.element_size(), _stream(stream))
    if rc != UPIPE_OK:
        raise UpipeError(rc, "upipe_loss_fwd")
    return loss, lse


def loss_bwd(h, w, targets, lse, dloss: float, tile_rows: int, ignore_index: int = -100,
             workspace=None, stream=None):
    """Backward of loss_fwd with upstream gradient dloss.  Returns (dh, dw)."""
    import torch

    L, hidden, vocab = _check_loss(h, w, targets)
    _check(lse, "lse", (L,), torch.float32, h.device)
    dh = torch.empty_like(h)
    dw = torch.empty_like(w)
    ws = _workspace(loss_workspace_bytes(L, hidden, vocab, tile_rows, PASS_BWD), h.device, workspace)
    rc = lib().upipe_loss_bwd(L, hidden, vocab, tile_rows, _ptr(h), _ptr(w), _ptr(targets),
                              ignore_index, _ptr(lse), float(dloss), _ptr(dh), _ptr(dw), _ptr(ws),
                              ws.numel() * ws.element_size(), _stream(stream))
    if rc != UPIPE_OK:
        raise UpipeError(rc, "upipe_loss_bwd")
    return dh, dw


def loss_fwd_bwd(h, w, targets, dloss: float, tile_rows: int, ignore_index: int = -100,
                 workspace=None, stream=None):
    """Forward and backward of the tiled loss in one pass (dloss known up
    front).  Returns (loss [1] fp32, lse [L] fp32, dh, dw)."""
    import torch

    L, hidden, vocab = _check_loss(h, w, targets)
    loss = torch.empty(1, dtype=torch.float32, device=h.device)
    lse = torch.empty(L, dtype=torch.float32, device=h.device)
    dh = torch.empty_like(h)
    dw = torch.empty_like(w)
    ws = _workspace(loss_workspace_bytes(L, hidden, vocab, tile_rows, PASS_FWD_BWD), h.device,
                    workspace)
    rc = lib().upipe_loss_fwd_bwd(L, hidden, vocab, tile_rows, _ptr(h), _ptr(w), _ptr(targets),
                                  ignore_index, float(dloss), _ptr(loss), _ptr(lse), _ptr(dh),
                                  _ptr(dw), _ptr(ws), ws.numel() * ws.element_size(), _stream(stream))
    if rc != UPIPE_OK:
        raise UpipeError(rc, "upipe_loss_fwd_bwd")
    return loss, lse, dh, dw


# ---------------------------------------------------------------- MFMA probe
PROBE_FLOP_PER_ROUND = 32 * 32 * 32 * 16 * 2   # 32 MFMAs 32x32x16 per wave and round


def probe_mfma(operands, iters: int, workgroups: int, stream=None):
    """Launch the sustained bf16 MFMA probe over `operands` (a bf16 device
    tensor of at least 16 MiB).  Returns (sink, clocks) device tensors; the
    caller times the launch.  FLOPs = workgroups * 4 * iters *
    PROBE_FLOP_PER_ROUND; clock = clocks[0::2] / clocks[1::2] * 100 MHz."""
    import torch

    if not operands.is_cuda or operands.dtype != torch.bfloat16 or not operands.is_contiguous():
        raise ValueError("operands must be a contiguous bf16 device tensor")
    sink = torch.empty(workgroups * 256, dtype=torch.float32, device=operands.device)
    clocks = torch.empty(workgroups * 4 * 2, dtype=torch.int64, device=operands.device)
    rc = lib().upipe_probe_mfma(_ptr(operands), operands.numel() * 2, iters, workgroups, _ptr(sink),
                                _ptr(clocks), _stream(stream))
    if rc != UPIPE_OK:
        raise UpipeError(rc, "upipe_probe_mfma")
    return sink, clocks
