"""Plain fp64 oracle of the sequence-tiled SwiGLU MLP.

TEST INFRASTRUCTURE ONLY: imported by tests/ and by bench.py's cpu_baseline
leg, never by the library.  Nothing here is shared with the HIP path.

What is computed, and where it comes from
-----------------------------------------
* The MLP is the gated one of "GLU Variants Improve Transformer" (Builds-on
  list of "Untied Ulysses: Memory-Efficient Context Parallelism via Headwise
  Chunking"): the input is projected twice, one projection goes through the
  Swish (SiLU) activation, z * sigmoid(z), and gates the other elementwise;
  the product is projected back.  With nn.Linear [out, in] weights and no
  bias:  h = x W_gate^T,  u = x W_up^T,  a = silu(h) * u,  y = a W_down^T.
* Sequence tiling is the Arctic Long Sequence Training step of the memory
  progression in "Untied Ulysses Pushes Llama-3-8B Training to 5 Million
  Tokens": computations that act on each position separately are run a tile
  of positions at a time, so that no intermediate spans the whole sequence.
  Every output row depends on its own input row only, and the weight
  gradients are sums over rows, so tiling changes the memory schedule, not
  the result.  The functions below take the tile size and loop over tiles in
  order; no other blocking, fusion or reordering is applied.
* The backward pass is the chain rule of the same definition:
    dW_down = dy^T a,  da = dy W_down,  du = da * silu(h),
    dh = da * u * silu'(h),  silu'(z) = s(z) (1 + z (1 - s(z))),
    dx = dh W_gate + du W_up,  dW_gate = dh^T x,  dW_up = du^T x.

Readings where the pages are silent (listed with their reasons in the design
notes): the MLP is the SwiGLU one of the Llama models the pages train; the
gate and up weights are packed as one [2F, D] matrix, gate rows first; no
bias; tiles are consecutive rows, the last one ragged.
"""
from __future__ import annotations

import numpy as np


def sigmoid(z: np.ndarray) -> np.ndarray:
    """1 / (1 + exp(-z)), as e / (1 + e) with e = exp(-|z|) on the negative
    side, so no exponential overflows and the far tails keep full relative
    precision."""
    z = np.asarray(z, dtype=np.float64)
    e = np.exp(-np.abs(z))
    return np.where(z >= 0, 1.0 / (1.0 + e), e / (1.0 + e))


def silu(z: np.ndarray) -> np.ndarray:
    """Swish with beta = 1: z * sigmoid(z)."""
    z = np.asarray(z, dtype=np.float64)
    return z * sigmoid(z)


def silu_grad(z: np.ndarray) -> np.ndarray:
    """d silu / dz = sigmoid(z) (1 + z (1 - sigmoid(z)))."""
    z = np.asarray(z, dtype=np.float64)
    s = sigmoid(z)
    return s * (1.0 + z * (1.0 - s))


def _split(w_gate_up):
    F = w_gate_up.shape[0] // 2
    return w_gate_up[:F], w_gate_up[F:]


def _tiles(L: int, tile_rows: int):
    assert tile_rows >= 1
    for t0 in range(0, L, tile_rows):
        yield slice(t0, min(L, t0 + tile_rows))


def mlp_fwd(x, w_gate_up, w_down, tile_rows):
    """y [L, D] of the SwiGLU MLP, one tile of rows at a time."""
    wg, wu = _split(w_gate_up)
    y = np.zeros((x.shape[0], w_down.shape[0]))
    for t in _tiles(x.shape[0], tile_rows):
        h = x[t] @ wg.T
        u = x[t] @ wu.T
        y[t] = (silu(h) * u) @ w_down.T
    return y


def mlp_bwd(x, w_gate_up, w_down, dy, tile_rows):
    """(dx, dw_gate_up, dw_down), one tile of rows at a time; the tile's
    intermediates are recomputed from x and the weight gradients summed over
    tiles."""
    wg, wu = _split(w_gate_up)
    F = wg.shape[0]
    dx = np.zeros_like(x, dtype=np.float64)
    dw_gate_up = np.zeros_like(w_gate_up, dtype=np.float64)
    dw_down = np.zeros_like(w_down, dtype=np.float64)
    for t in _tiles(x.shape[0], tile_rows):
        h = x[t] @ wg.T
        u = x[t] @ wu.T
        a = silu(h) * u
        dw_down += dy[t].T @ a
        da = dy[t] @ w_down
        du = da * silu(h)
        dh = da * u * silu_grad(h)
        dx[t] = dh @ wg + du @ wu
        dw_gate_up[:F] += dh.T @ x[t]
        dw_gate_up[F:] += du.T @ x[t]
    return dx, dw_gate_up, dw_down
