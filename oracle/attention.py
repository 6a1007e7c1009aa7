"""Plain fp64 oracle of the headwise-chunked causal GQA attention layer.

TEST INFRASTRUCTURE ONLY: imported by tests/, by __graft_entry__.smoke() and by
the cpu_baseline leg of bench.py, never by the library.  Nothing here is shared
with the HIP path.

What is computed, and where it comes from
-----------------------------------------
* The layer is ordinary causal softmax attention.  The headwise-chunking method
  changes only the memory schedule, not the attention formula ("Untied Ulysses
  Pushes Llama-3-8B Training to 5 Million Tokens", the Untied Ulysses section),
  and FlashAttention, which the method runs per head group, is exact attention
  ("Untied Ulysses: Memory-Efficient Context Parallelism via Headwise
  Chunking", Builds-on list: FlashAttention).  So every function below is the
  plain definition written out: S = q k^T / sqrt(d) over keys j <= i,
  softmax, O = P v (Builds-on list: Attention Is All You Need).
* The head loop follows the method: heads are processed one chunk at a time; a
  chunk's q/k/v are projected with only that chunk's rows of W_qkv, attention
  is run, the partial result is stored and the output projection of that chunk
  is accumulated into y (same section: compute one group of heads, store a
  partial result, move to the next group reusing the buffers).
* Grouped-query attention (same page, same section: the method is built for
  layers where several query heads share one key/value head): q head h reads KV head h // G,
  G = Hq / Hkv.
* Rotary position embedding (Builds-on list: RoFormer): consecutive pairs
  (2i, 2i+1) are rotated by angle p * theta^(-2i/d) at position p.
* The backward pass is the chain rule of the same definition.

Readings where the pages are silent (each is listed with its reason in the
design notes): scale 1/sqrt(d); key j visible to query i iff j <= i; no bias;
nn.Linear weight layout with W_qkv rows packed Q heads | K heads | V heads; the
RoPE pair convention above with absolute positions 0..L-1 and no frequency
scaling; batch 1.

Evaluation order: a causal softmax row depends only on its own scores, so rows
are evaluated in blocks of ROW_BLOCK to bound memory.  No other blocking,
fusion or reordering is applied.
"""
from __future__ import annotations

import math

import numpy as np

ROW_BLOCK = 256


# --------------------------------------------------------------------------
# Rotary position embedding (RoFormer, cited in the Builds-on list)
# --------------------------------------------------------------------------
def rope_angles(positions, d: int, theta: float) -> np.ndarray:
    """Angle p * theta^(-2i/d) for every position p and pair i < d/2, in fp64."""
    i = np.arange(d // 2, dtype=np.float64)
    inv_freq = np.power(float(theta), -2.0 * i / d)
    return np.asarray(positions, dtype=np.float64)[:, None] * inv_freq[None, :]


def rope(u: np.ndarray, positions, theta: float, inverse: bool = False) -> np.ndarray:
    """Rotate pairs (u[2i], u[2i+1]) of each row by +angle (or -angle if inverse)."""
    u = np.asarray(u, dtype=np.float64)
    a = rope_angles(positions, u.shape[-1], theta)
    c, s = np.cos(a), np.sin(a)
    if inverse:
        s = -s
    ev, od = u[:, 0::2], u[:, 1::2]
    out = np.empty_like(u)
    out[:, 0::2] = ev * c - od * s
    out[:, 1::2] = ev * s + od * c
    return out


# --------------------------------------------------------------------------
# Causal softmax attention, one head (Attention Is All You Need; exact
# attention as in FlashAttention)
# --------------------------------------------------------------------------
def _masked_scores(q_blk, rows, k, scale):
    """Scores of query rows `rows` against keys 0..max(rows); masked keys -> -inf."""
    kmax = int(rows[-1]) + 1
    s = (q_blk @ k[:kmax].T) * scale
    visible = np.arange(kmax)[None, :] <= np.asarray(rows)[:, None]
    return np.where(visible, s, -np.inf), visible


def attention_rows(q_rows: np.ndarray, rows, k: np.ndarray, v: np.ndarray):
    """O_i and natural-log LSE_i for the listed query positions.

    q_rows[n] is the (already rotated) query at position rows[n]; rows must be
    sorted ascending.  LSE_i = log sum_{j<=i} exp(S_ij).
    """
    rows = np.asarray(rows, dtype=np.int64)
    d = q_rows.shape[1]
    scale = 1.0 / math.sqrt(d)
    out = np.empty((len(rows), v.shape[1]))
    lse = np.empty(len(rows))
    for b0 in range(0, len(rows), ROW_BLOCK):
        b1 = min(len(rows), b0 + ROW_BLOCK)
        s, _ = _masked_scores(q_rows[b0:b1], rows[b0:b1], k, scale)
        m = s.max(axis=1, keepdims=True)
        e = np.exp(s - m)
        z = e.sum(axis=1, keepdims=True)
        lse[b0:b1] = (m + np.log(z))[:, 0]
        out[b0:b1] = (e / z) @ v[: s.shape[1]]
    return out, lse


def attention_fwd_head(q: np.ndarray, k: np.ndarray, v: np.ndarray):
    """O [L, dv] and LSE [L] of causal attention for one head (q, k rotated)."""
    return attention_rows(q, np.arange(q.shape[0]), k, v)


def attention_bwd_head(q, k, v, dO):
    """Gradients (dq, dk, dv) of causal attention for one head, in rotated space.

    With P = softmax(S), D_i = dO_i . O_i:  dV = P^T dO, dP = dO v^T,
    dS = P o (dP - D), dq = dS k / sqrt(d), dk = dS^T q / sqrt(d).
    """
    L, d = q.shape
    scale = 1.0 / math.sqrt(d)
    O, lse = attention_fwd_head(q, k, v)
    D = np.sum(dO * O, axis=1)
    dq = np.zeros_like(q, dtype=np.float64)
    dk = np.zeros_like(k, dtype=np.float64)
    dv = np.zeros_like(v, dtype=np.float64)
    for r0 in range(0, L, ROW_BLOCK):
        r1 = min(L, r0 + ROW_BLOCK)
        rows = np.arange(r0, r1)
        s, visible = _masked_scores(q[r0:r1], rows, k, scale)
        P = np.where(visible, np.exp(s - lse[r0:r1, None]), 0.0)
        dv[:r1] += P.T @ dO[r0:r1]
        dP = dO[r0:r1] @ v[:r1].T
        dS = P * (dP - D[r0:r1, None])
        dq[r0:r1] = (dS @ k[:r1]) * scale
        dk[:r1] += (dS.T @ q[r0:r1]) * scale
    return dq, dk, dv


# --------------------------------------------------------------------------
# The layer, one head chunk at a time
# --------------------------------------------------------------------------
def _check(n_q, n_kv, head_chunk):
    assert n_q % n_kv == 0, "Hq must be a multiple of Hkv"
    assert n_q % head_chunk == 0, "head chunk must divide Hq"
    G = n_q // n_kv
    assert head_chunk % G == 0 or G % head_chunk == 0, "chunk straddles a KV group"
    return G


def _q_part(x, w_qkv, h, d):
    """Pre-rotation query of head h: x W_q,h^T, or the given q columns."""
    if w_qkv is None:
        return x[:, h * d:(h + 1) * d]
    return x @ w_qkv[h * d:(h + 1) * d].T


def _kv_part(x, w_qkv, g, n_q, n_kv, d):
    """Pre-rotation key and value of KV head g."""
    k0 = (n_q + g) * d
    v0 = (n_q + n_kv + g) * d
    if w_qkv is None:
        return x[:, k0:k0 + d], x[:, v0:v0 + d]
    return x @ w_qkv[k0:k0 + d].T, x @ w_qkv[v0:v0 + d].T


def layer_fwd(x, w_qkv, w_o, n_q, n_kv, head_dim, theta, head_chunk):
    """Forward of the chunked layer.

    Projection mode (w_qkv, w_o given): x [L, hidden] -> y [L, hidden].
    q/k/v-given mode (w_qkv is None): x is packed q|k|v [L, (Hq+2Hkv)d], y None.
    Also returns o_saved [L, Hq d] (per-head attention output) and lse [Hq, L].
    """
    G = _check(n_q, n_kv, head_chunk)
    d = head_dim
    L = x.shape[0]
    pos = np.arange(L)
    proj = w_qkv is not None
    o_saved = np.zeros((L, n_q * d))
    lse = np.zeros((n_q, L))
    y = np.zeros((L, w_o.shape[0])) if proj else None
    resident = {}
    for c in range(n_q // head_chunk):
        heads = range(c * head_chunk, (c + 1) * head_chunk)
        for h in heads:
            g = h // G
            if g not in resident:       # a KV group is projected once, when first touched
                k_g, v_g = _kv_part(x, w_qkv, g, n_q, n_kv, d)
                resident = {g: (rope(k_g, pos, theta), v_g)}
            k_rot, v_g = resident[g]
            q_rot = rope(_q_part(x, w_qkv, h, d), pos, theta)
            O, l = attention_fwd_head(q_rot, k_rot, v_g)
            o_saved[:, h * d:(h + 1) * d] = O
            lse[h] = l
        if proj:                        # accumulate this chunk's share of the output projection
            cols = slice(c * head_chunk * d, (c + 1) * head_chunk * d)
            y += o_saved[:, cols] @ w_o[:, cols].T
    return y, o_saved, lse


def layer_bwd(x, w_qkv, w_o, dy, n_q, n_kv, head_dim, theta, head_chunk):
    """Backward of the chunked layer (recomputes the forward itself).

    Projection mode returns (dx, dw_qkv, dw_o); q/k/v-given mode returns
    (dqkv, None, None) with dy read as dO [L, Hq d].
    """
    G = _check(n_q, n_kv, head_chunk)
    d = head_dim
    L = x.shape[0]
    pos = np.arange(L)
    proj = w_qkv is not None
    _, o_saved, _ = layer_fwd(x, w_qkv, w_o, n_q, n_kv, head_dim, theta, head_chunk)
    if proj:
        dx = np.zeros_like(x, dtype=np.float64)
        dw_qkv = np.zeros_like(w_qkv, dtype=np.float64)
        dw_o = np.zeros_like(w_o, dtype=np.float64)
    else:
        dqkv = np.zeros((L, (n_q + 2 * n_kv) * d))
    dk_acc, dv_acc, resident = {}, {}, {}
    for c in range(n_q // head_chunk):
        heads = range(c * head_chunk, (c + 1) * head_chunk)
        cols = slice(c * head_chunk * d, (c + 1) * head_chunk * d)
        if proj:
            dO_c = dy @ w_o[:, cols]
            dw_o[:, cols] = dy.T @ o_saved[:, cols]
        else:
            dO_c = dy[:, cols]
        for j, h in enumerate(heads):
            g = h // G
            if g not in resident:
                k_g, v_g = _kv_part(x, w_qkv, g, n_q, n_kv, d)
                resident = {g: (rope(k_g, pos, theta), v_g)}
                dk_acc[g] = np.zeros((L, d))
                dv_acc[g] = np.zeros((L, d))
            k_rot, v_g = resident[g]
            q_rot = rope(_q_part(x, w_qkv, h, d), pos, theta)
            dq_rot, dk_rot, dv = attention_bwd_head(q_rot, k_rot, v_g, dO_c[:, j * d:(j + 1) * d])
            dq = rope(dq_rot, pos, theta, inverse=True)
            dk_acc[g] += dk_rot
            dv_acc[g] += dv
            rq = slice(h * d, (h + 1) * d)
            if proj:
                dx += dq @ w_qkv[rq]
                dw_qkv[rq] = dq.T @ x
            else:
                dqkv[:, rq] = dq
            if h == (g + 1) * G - 1:   # last q head of the group: its K/V gradient is complete
                dk = rope(dk_acc.pop(g), pos, theta, inverse=True)
                dv_g = dv_acc.pop(g)
                rk = slice((n_q + g) * d, (n_q + g + 1) * d)
                rv = slice((n_q + n_kv + g) * d, (n_q + n_kv + g + 1) * d)
                if proj:
                    dx += dk @ w_qkv[rk] + dv_g @ w_qkv[rv]
                    dw_qkv[rk] = dk.T @ x
                    dw_qkv[rv] = dv_g.T @ x
                else:
                    dqkv[:, rk] = dk
                    dqkv[:, rv] = dv_g
    if proj:
        return dx, dw_qkv, dw_o
    return dqkv, None, None


# --------------------------------------------------------------------------
# Row-sampled forms for sequence lengths where the full oracle is too slow.
# Each output row is the same definition evaluated for that row alone.
# --------------------------------------------------------------------------
def _kv_rotated(x, w_qkv, g, n_q, n_kv, d, theta, upto):
    k_g, v_g = _kv_part(x[:upto], w_qkv, g, n_q, n_kv, d)
    return rope(k_g, np.arange(upto), theta), np.asarray(v_g, dtype=np.float64)


def layer_rows(x, w_qkv, w_o, n_q, n_kv, head_dim, theta, rows):
    """y_i (projection mode, else None), O_i [n, Hq d] and LSE [Hq, n] for rows i."""
    rows = np.sort(np.asarray(rows, dtype=np.int64))
    d = head_dim
    G = n_q // n_kv
    upto = int(rows[-1]) + 1
    o = np.zeros((len(rows), n_q * d))
    lse = np.zeros((n_q, len(rows)))
    xr = x[rows]
    for g in range(n_kv):
        k_rot, v_g = _kv_rotated(x, w_qkv, g, n_q, n_kv, d, theta, upto)
        for h in range(g * G, (g + 1) * G):
            q_rot = rope(_q_part(xr, w_qkv, h, d), rows, theta)
            O, l = attention_rows(q_rot, rows, k_rot, v_g)
            o[:, h * d:(h + 1) * d] = O
            lse[h] = l
    y = o @ w_o.T if w_qkv is not None else None
    return y, o, lse


def _dO_rows(dy_rows, w_o, h, d):
    if w_o is None:
        return dy_rows[:, h * d:(h + 1) * d]
    return dy_rows @ w_o[:, h * d:(h + 1) * d]


def dq_rows(x, w_qkv, w_o, dy, n_q, n_kv, head_dim, theta, rows):
    """Un-rotated query gradient dq_i [n, Hq d] for the listed rows.

    dq_i = (1/sqrt d) sum_{j<=i} P_ij (dO_i.v_j - D_i) k_j, rotated back by -p_i.
    """
    rows = np.sort(np.asarray(rows, dtype=np.int64))
    d = head_dim
    G = n_q // n_kv
    scale = 1.0 / math.sqrt(d)
    upto = int(rows[-1]) + 1
    xr, dyr = x[rows], dy[rows]
    out = np.zeros((len(rows), n_q * d))
    for g in range(n_kv):
        k_rot, v_g = _kv_rotated(x, w_qkv, g, n_q, n_kv, d, theta, upto)
        for h in range(g * G, (g + 1) * G):
            q_rot = rope(_q_part(xr, w_qkv, h, d), rows, theta)
            O, lse = attention_rows(q_rot, rows, k_rot, v_g)
            dO = _dO_rows(dyr, w_o, h, d)
            D = np.sum(dO * O, axis=1)
            for b0 in range(0, len(rows), ROW_BLOCK):
                b1 = min(len(rows), b0 + ROW_BLOCK)
                s, visible = _masked_scores(q_rot[b0:b1], rows[b0:b1], k_rot, scale)
                P = np.where(visible, np.exp(s - lse[b0:b1, None]), 0.0)
                dP = dO[b0:b1] @ v_g[: s.shape[1]].T
                dS = P * (dP - D[b0:b1, None])
                out[b0:b1, h * d:(h + 1) * d] = rope(
                    (dS @ k_rot[: s.shape[1]]) * scale, rows[b0:b1], theta, inverse=True)
    return out


def kv_grad_tail(x, w_qkv, w_o, dy, n_q, n_kv, head_dim, theta, tail):
    """Un-rotated dk_j, dv_j for the last `tail` key positions of every KV head.

    Keys j >= L - tail are seen only by queries i >= j, so only the last `tail`
    query rows are needed.  Returns (dk [tail, Hkv d], dv [tail, Hkv d]).
    """
    L = x.shape[0]
    d = head_dim
    G = n_q // n_kv
    scale = 1.0 / math.sqrt(d)
    rows = np.arange(L - tail, L)
    xr, dyr = x[rows], dy[rows]
    dk = np.zeros((tail, n_kv * d))
    dv = np.zeros((tail, n_kv * d))
    for g in range(n_kv):
        k_rot, v_g = _kv_rotated(x, w_qkv, g, n_q, n_kv, d, theta, L)
        for h in range(g * G, (g + 1) * G):
            q_rot = rope(_q_part(xr, w_qkv, h, d), rows, theta)
            O, lse = attention_rows(q_rot, rows, k_rot, v_g)
            dO = _dO_rows(dyr, w_o, h, d)
            D = np.sum(dO * O, axis=1)
            s = (q_rot @ k_rot[L - tail:].T) * scale
            visible = rows[None, :] <= rows[:, None]          # key j <= query i
            P = np.where(visible, np.exp(s - lse[:, None]), 0.0)
            dv[:, g * d:(g + 1) * d] += P.T @ dO
            dS = P * (dO @ v_g[L - tail:].T - D[:, None])
            dk[:, g * d:(g + 1) * d] += (dS.T @ q_rot) * scale
        dk[:, g * d:(g + 1) * d] = rope(dk[:, g * d:(g + 1) * d], rows, theta, inverse=True)
    return dk, dv
