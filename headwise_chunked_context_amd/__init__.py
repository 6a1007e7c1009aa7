"""Headwise-chunked causal GQA attention (UPipe) for MI355X / gfx950, with the
sequence-tiled SwiGLU MLP and language-model loss of the same long-context
training stack.

All run in the HIP library libupipe_attn.so (C ABI in include/upipe_attn.h,
include/upipe_mlp.h and include/upipe_loss.h); this package is its thin
ctypes binding.
"""
from .binding import (  # noqa: F401
    EXPORTS,
    KERNEL_KINDS,
    PASS_BWD,
    PASS_BWD_RECOMPUTE,
    PASS_FWD,
    PASS_FWD_PIPELINED,
    PASS_BWD_PIPELINED,
    UPIPE_ECHUNK,
    UPIPE_EHIP,
    UPIPE_ESCRATCH,
    STATIC_SCRATCH_BYTES,
    UPIPE_EINVAL,
    UPIPE_EUNSUPPORTED,
    UPIPE_EWORKSPACE,
    UPIPE_OK,
    UpipeError,
    attn_bwd,
    attn_fwd,
    attn_fwd_static,
    fwd_pass,
    bwd_pass,
    choose_chunk,
    debug_enable,
    lib,
    loss_bwd,
    loss_choose_tile,
    loss_fwd,
    loss_workspace_bytes,
    mlp_bwd,
    mlp_choose_tile,
    mlp_fwd,
    mlp_workspace_bytes,
    pipeline_enable,
    probe_mfma,
    pipeline_enabled,
    profile_enable,
    profile_read,
    strerror,
    workspace_bytes,
)
