"""Plain fp64 oracle of the sequence-tiled language-model loss.

TEST INFRASTRUCTURE ONLY: imported by tests/ and by bench.py's cpu_baseline
leg, never by the library.  Nothing here is shared with the HIP path.

What is computed, and where it comes from
-----------------------------------------
* The loss of next-token training: the final hidden states h [L, D] are
  projected onto the vocabulary by the output weight W [V, D] (nn.Linear
  [out, in], no bias), logits = h W^T, and each position's loss is the
  cross-entropy of the softmax over its logits against its target token,
      loss_r = log sum_j exp(logits_rj) - logits_r,t(r),
  averaged over the positions whose target is not the ignore index.
* Sequence tiling is the Arctic Long Sequence Training step of the memory
  progression in "Untied Ulysses Pushes Llama-3-8B Training to 5 Million
  Tokens": the loss, like the MLP, acts on each position separately, so it
  can be computed a tile of positions at a time and the [L, V] logits never
  exist at once.  The functions below take the tile size and loop over tiles
  in order; no other blocking, fusion or reordering is applied.
* The backward pass is the chain rule of the same definition, with the
  upstream gradient dloss of the mean:
      dlogits_rj = (softmax_rj - [j == t(r)]) * dloss / count   (valid rows),
      dlogits_r  = 0                                              (ignored rows),
      dh = dlogits W,   dW = dlogits^T h,
  where softmax_rj = exp(logits_rj - lse_r) with lse_r the row's log-sum-exp
  (the forward returns it, so the backward needs no second reduction).

Readings where the pages are silent (listed with their reasons in the design
notes): the loss is the mean cross-entropy of the Llama models the pages
train; positions whose target equals ignore_index are left out of the mean;
when every position is ignored the loss and the gradients are 0 (a mean over
no terms, taken as 0 rather than 0/0); a target outside [0, V) that is not
the ignore index makes that row's loss, the total and that row's gradients
NaN; tiles are consecutive rows, the last one ragged.
"""
from __future__ import annotations

import numpy as np


def _tiles(L: int, tile_rows: int):
    assert tile_rows >= 1
    for t0 in range(0, L, tile_rows):
        yield slice(t0, min(L, t0 + tile_rows))


def logsumexp_rows(z: np.ndarray) -> np.ndarray:
    """log sum_j exp(z_rj) per row, shifted by the row maximum so that no
    exponential overflows."""
    z = np.asarray(z, dtype=np.float64)
    m = z.max(axis=1)
    return m + np.log(np.exp(z - m[:, None]).sum(axis=1))


def _valid(targets, V, ignore_index):
    t = np.asarray(targets, dtype=np.int64)
    ignored = t == ignore_index
    in_range = (t >= 0) & (t < V)
    return ignored, in_range


def loss_fwd(h, w, targets, ignore_index, tile_rows):
    """(loss, lse [L]) of the mean cross-entropy, one tile of rows at a time."""
    h = np.asarray(h, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    L, V = h.shape[0], w.shape[0]
    ignored, in_range = _valid(targets, V, ignore_index)
    t = np.asarray(targets, dtype=np.int64)
    lse = np.zeros(L)
    loss_rows = np.zeros(L)
    for s in _tiles(L, tile_rows):
        logits = h[s] @ w.T
        lse[s] = logsumexp_rows(logits)
        rows = np.arange(s.start, s.stop)
        for r in rows:
            if ignored[r]:
                continue
            loss_rows[r] = lse[r] - logits[r - s.start, t[r]] if in_range[r] else np.nan
    count = int((~ignored).sum())
    loss = loss_rows.sum() / count if count > 0 else 0.0
    return loss, lse


def loss_bwd(h, w, targets, ignore_index, lse, dloss, tile_rows):
    """(dh [L, D], dw [V, D]) of the mean cross-entropy scaled by dloss, one
    tile of rows at a time: each tile's logits are recomputed from h, and the
    weight gradient is summed over tiles."""
    h = np.asarray(h, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    L, V = h.shape[0], w.shape[0]
    ignored, in_range = _valid(targets, V, ignore_index)
    t = np.asarray(targets, dtype=np.int64)
    count = int((~ignored).sum())
    scale = dloss / count if count > 0 else 0.0
    dh = np.zeros_like(h)
    dw = np.zeros_like(w)
    for s in _tiles(L, tile_rows):
        logits = h[s] @ w.T
        d = np.exp(logits - np.asarray(lse, dtype=np.float64)[s][:, None])
        for r in range(s.start, s.stop):
            i = r - s.start
            if ignored[r]:
                d[i] = 0.0
            elif in_range[r]:
                d[i, t[r]] -= 1.0
            else:
                d[i] = np.nan
        d *= scale
        dh[s] = d @ w
        dw += d.T @ h[s]
    return dh, dw
