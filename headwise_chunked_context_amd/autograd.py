"""torch.autograd wrappers of the library's forward / backward pairs, so a
PyTorch model can call them and get gradients from loss.backward().

Each Function's forward calls the library's forward entry point and keeps
what the matching backward entry point needs; its backward calls that entry
point.  Every step runs in the HIP library; these classes only pass
tensors between the two calls.  Inputs must be what the binding accepts
(bfloat16, contiguous, on the GPU, with the shape rules of the C headers);
gradients arriving from autograd are made contiguous first.

- attention(): the headwise-chunked causal GQA attention layer
  (upipe_attn_fwd / upipe_attn_bwd).  With recompute=True the forward keeps
  only x, the weights and the log-sum-exp, and the backward recomputes the
  attention output per chunk (o_saved = NULL).
- swiglu_mlp(): the sequence-tiled SwiGLU MLP (upipe_mlp_fwd / _bwd).
- cross_entropy(): the sequence-tiled mean cross-entropy over the
  vocabulary projection (upipe_loss_fwd / _bwd).  The library takes the
  upstream gradient as a host value, so its backward reads the incoming
  gradient to the host (one synchronization per backward).
"""
from __future__ import annotations

import torch

from . import binding


class _Attention(torch.autograd.Function):
    @staticmethod
    def forward(ctx, x, w_qkv, w_o, n_q, n_kv, head_chunk, theta, recompute):
        y, o, lse = binding.attn_fwd(x, w_qkv, w_o, n_q, n_kv, head_chunk, theta)
        projection = w_qkv is not None
        keep_o = o if (not recompute or not projection) else None
        ctx.save_for_backward(x, w_qkv, w_o, keep_o, lse)
        ctx.cfg = (n_q, n_kv, head_chunk, theta)
        return y if projection else o

    @staticmethod
    def backward(ctx, dout):
        x, w_qkv, w_o, o, lse = ctx.saved_tensors
        n_q, n_kv, head_chunk, theta = ctx.cfg
        dx, dw_qkv, dw_o = binding.attn_bwd(x, w_qkv, w_o, o, lse, dout.contiguous(), n_q, n_kv,
                                            head_chunk, theta)
        return dx, dw_qkv, dw_o, None, None, None, None, None


def attention(x, w_qkv, w_o, n_q: int, n_kv: int, head_chunk: int, theta: float,
              recompute: bool = False):
    """y = the layer's output (x [L, hidden], w_qkv [(Hq+2Hkv)*128, hidden],
    w_o [hidden, Hq*128]); or, with w_qkv = w_o = None, the attention output
    O [L, Hq*128] of the packed q|k|v rows in x.  recompute=True (projection
    mode only) keeps no attention output for the backward."""
    return _Attention.apply(x, w_qkv, w_o, n_q, n_kv, head_chunk, theta, recompute)


class _SwiGluMlp(torch.autograd.Function):
    @staticmethod
    def forward(ctx, x, w_gate_up, w_down, tile_rows):
        y = binding.mlp_fwd(x, w_gate_up, w_down, tile_rows)
        ctx.save_for_backward(x, w_gate_up, w_down)
        ctx.tile_rows = tile_rows
        return y

    @staticmethod
    def backward(ctx, dy):
        x, w_gate_up, w_down = ctx.saved_tensors
        dx, dwgu, dwd = binding.mlp_bwd(x, w_gate_up, w_down, dy.contiguous(), ctx.tile_rows)
        return dx, dwgu, dwd, None


def swiglu_mlp(x, w_gate_up, w_down, tile_rows: int):
    """y = (silu(x W_gate^T) * (x W_up^T)) W_down^T, tile_rows rows at a time
    (w_gate_up packs W_gate and W_up, gate rows first)."""
    return _SwiGluMlp.apply(x, w_gate_up, w_down, tile_rows)


class _CrossEntropy(torch.autograd.Function):
    @staticmethod
    def forward(ctx, h, w, targets, tile_rows, ignore_index):
        loss, lse = binding.loss_fwd(h, w, targets, tile_rows, ignore_index)
        ctx.save_for_backward(h, w, targets, lse)
        ctx.cfg = (tile_rows, ignore_index)
        return loss.reshape(())

    @staticmethod
    def backward(ctx, dloss):
        h, w, targets, lse = ctx.saved_tensors
        tile_rows, ignore_index = ctx.cfg
        dh, dw = binding.loss_bwd(h, w, targets, lse, float(dloss.item()), tile_rows,
                                  ignore_index)
        return dh, dw, None, None, None


def cross_entropy(h, w, targets, tile_rows: int, ignore_index: int = -100):
    """Mean cross-entropy of logits = h W^T against int32 targets, rows whose
    target is ignore_index left out; a 0-dimensional fp32 tensor."""
    return _CrossEntropy.apply(h, w, targets, tile_rows, ignore_index)
