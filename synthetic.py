"""Seeded synthetic inputs for the headwise-chunked attention layer.

This module is the only code shared by the fp64 oracle side and the HIP side of
the tests and of bench.py.  It draws seeded normal samples and rounds them to
bfloat16; it contains none of the layer's arithmetic.

Workloads stand in for the attention shapes the pages train (Llama-3-8B and a
Qwen2-32B-class model, "Untied Ulysses Pushes Llama-3-8B Training to 5 Million
Tokens", benchmark paragraphs); no dataset or trained weight is involved.

Recipe: numpy Generator(PCG64(seed)), float32 standard normal times sigma,
rounded to bfloat16 with round-to-nearest-even.  Seed = 1000 * workload_id +
tensor_id with tensor ids x|qkv = 1, W_qkv = 2, W_o = 3, dy|dO = 4.
"""
from __future__ import annotations

import dataclasses

import numpy as np

TENSOR_IDS = {"x": 1, "w_qkv": 2, "w_o": 3, "dy": 4, "targets": 5}


@dataclasses.dataclass(frozen=True)
class Workload:
    """One layer shape.  hidden == 0 means q/k/v are given (no projections)."""

    wid: int
    name: str
    L: int
    hidden: int
    n_q: int
    n_kv: int
    head_dim: int
    head_chunk: int
    theta: float
    x_sigma: float = 1.0
    w_sigma: float = 0.02

    @property
    def projection(self) -> bool:
        return self.hidden > 0

    @property
    def qkv_width(self) -> int:
        return (self.n_q + 2 * self.n_kv) * self.head_dim

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The five layer shapes the metric is quoted on (sizes spelled out in the names).
WORKLOADS = {
    1: Workload(1, "gqa8q2kv_hidden1024_L1024_chunk2", 1024, 1024, 8, 2, 128, 2, 5e5),
    2: Workload(2, "llama3_8b_layer_hidden4096_32q8kv_L32768_chunk8", 32768, 4096, 32, 8, 128, 8, 5e5),
    3: Workload(3, "llama3_8b_cp8_share_4q1kv_L524288_chunk1", 524288, 0, 4, 1, 128, 1, 5e5),
    4: Workload(4, "qwen32b_cp8_share_hidden5120_8q1kv_L262144", 262144, 5120, 8, 1, 128, 1, 1e6),
    5: Workload(5, "llama3_8b_cp8_share_4q1kv_L1048576_chunk1", 1048576, 0, 4, 1, 128, 1, 5e5),
}


@dataclasses.dataclass(frozen=True)
class MlpWorkload:
    """A sequence-tiled SwiGLU MLP shape: L rows of width hidden, ffn the
    intermediate width, tile_rows the rows processed at a time."""

    wid: int
    name: str
    L: int
    hidden: int
    ffn: int
    tile_rows: int
    x_sigma: float = 1.0
    w_sigma: float = 0.02

    def with_(self, **kw) -> "MlpWorkload":
        return dataclasses.replace(self, **kw)


# The Llama-3-8B MLP (hidden 4096, intermediate 14336) over the benchmarked
# layer's sequence, and a small one for parity tests.
MLP_WORKLOADS = {
    11: MlpWorkload(11, "mlp_hidden512_ffn1536_L1000_tile256", 1000, 512, 1536, 256),
    12: MlpWorkload(12, "llama3_8b_mlp_hidden4096_ffn14336_L32768_tile8192", 32768, 4096, 14336, 8192),
}


def make_mlp_inputs(w: MlpWorkload, with_grad: bool = True, seed_base: int | None = None) -> dict:
    """bf16 bit arrays (uint16): x [L, hidden], w_gate_up [2 ffn, hidden] (gate
    rows first), w_down [hidden, ffn], dy [L, hidden].  Seeds as for the
    attention workloads (1000 * wid + tensor id)."""
    base = 1000 * w.wid if seed_base is None else seed_base
    out = {
        "x": draw_bf16(base + TENSOR_IDS["x"], (w.L, w.hidden), w.x_sigma),
        "w_gate_up": draw_bf16(base + TENSOR_IDS["w_qkv"], (2 * w.ffn, w.hidden), w.w_sigma),
        "w_down": draw_bf16(base + TENSOR_IDS["w_o"], (w.hidden, w.ffn), w.w_sigma),
    }
    if with_grad:
        out["dy"] = draw_bf16(base + TENSOR_IDS["dy"], (w.L, w.hidden), 1.0)
    return out


@dataclasses.dataclass(frozen=True)
class LossWorkload:
    """A sequence-tiled language-model loss: L positions of width hidden
    projected onto a vocabulary of `vocab` tokens, tile_rows positions at a
    time; one position in `ignore_every` has the ignore index as target."""

    wid: int
    name: str
    L: int
    hidden: int
    vocab: int
    tile_rows: int
    ignore_every: int = 16
    h_sigma: float = 1.0
    w_sigma: float = 0.02

    def with_(self, **kw) -> "LossWorkload":
        return dataclasses.replace(self, **kw)


IGNORE_INDEX = -100

# The Llama-3-8B output projection (hidden 4096, vocabulary 128256) over the
# benchmarked layer's sequence, and a small one for parity tests.
LOSS_WORKLOADS = {
    21: LossWorkload(21, "loss_hidden256_vocab1024_L1000_tile256", 1000, 256, 1024, 256),
    22: LossWorkload(22, "llama3_8b_loss_hidden4096_vocab128256_L32768_tile4096", 32768, 4096, 128256, 4096),
}


def make_loss_inputs(w: LossWorkload, seed_base: int | None = None) -> dict:
    """h [L, hidden] and w [vocab, hidden] as bf16 bits (uint16), targets [L]
    int32 uniform over the vocabulary with every `ignore_every`-th position
    (from a seeded random offset) set to IGNORE_INDEX.  Seeds as for the
    attention workloads (1000 * wid + tensor id)."""
    base = 1000 * w.wid if seed_base is None else seed_base
    rng = np.random.Generator(np.random.PCG64(base + TENSOR_IDS["targets"]))
    targets = rng.integers(0, w.vocab, size=w.L, dtype=np.int64).astype(np.int32)
    if w.ignore_every > 0:
        targets[int(rng.integers(0, w.ignore_every))::w.ignore_every] = IGNORE_INDEX
    return {
        "h": draw_bf16(base + TENSOR_IDS["x"], (w.L, w.hidden), w.h_sigma),
        "w": draw_bf16(base + TENSOR_IDS["w_qkv"], (w.vocab, w.hidden), w.w_sigma),
        "targets": targets,
    }


def make_loss_inputs_device(w: LossWorkload, device="cuda:0") -> dict:
    """The same distributions drawn on the device by torch's generator
    (seeded 1000 * wid), for sizes whose host draw takes minutes: h, w as
    torch bfloat16 and targets as int32 tensors on `device`, every
    `ignore_every`-th position set to IGNORE_INDEX.  Not the host recipe's
    values."""
    import torch

    g = torch.Generator(device=device).manual_seed(1000 * w.wid)
    h = torch.randn(w.L, w.hidden, generator=g, device=device, dtype=torch.float32)
    if w.h_sigma != 1.0:
        h.mul_(w.h_sigma)
    wt = torch.randn(w.vocab, w.hidden, generator=g, device=device, dtype=torch.float32)
    wt.mul_(w.w_sigma)
    t = torch.randint(0, w.vocab, (w.L,), generator=g, device=device, dtype=torch.int32)
    if w.ignore_every > 0:
        t[::w.ignore_every] = IGNORE_INDEX
    return {"h": h.to(torch.bfloat16), "w": wt.to(torch.bfloat16), "targets": t}


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); returns uint16 bits."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    rounded = u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return (rounded >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def bf16_bits_to_f64(b: np.ndarray) -> np.ndarray:
    return bf16_bits_to_f32(b).astype(np.float64)


def draw_bf16(seed: int, shape, sigma: float, chunk_rows: int = 1 << 16) -> np.ndarray:
    """Seeded N(0, sigma^2) draw, rounded to bfloat16 bits (uint16).

    Rows are drawn in slabs so that very long sequences do not need a float32
    copy of the whole tensor at once; the stream of normals is the same as one
    single draw because the generator is consumed in row order.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    shape = tuple(int(s) for s in shape)
    out = np.empty(shape, dtype=np.uint16)
    if len(shape) == 2 and shape[0] > chunk_rows:
        for r0 in range(0, shape[0], chunk_rows):
            r1 = min(shape[0], r0 + chunk_rows)
            z = rng.standard_normal((r1 - r0, shape[1]), dtype=np.float32)
            if sigma != 1.0:
                z *= np.float32(sigma)
            out[r0:r1] = f32_to_bf16_bits(z)
        return out
    z = rng.standard_normal(shape, dtype=np.float32)
    if sigma != 1.0:
        z *= np.float32(sigma)
    out[...] = f32_to_bf16_bits(z)
    return out


def make_inputs(w: Workload, with_grad: bool = True, seed_base: int | None = None) -> dict:
    """bf16 bit arrays (uint16) for one workload.

    Projection mode: x [L, hidden], w_qkv [(Hq+2Hkv)d, hidden], w_o [hidden, Hq d],
    dy [L, hidden].  q/k/v-given mode: x is packed q|k|v [L, (Hq+2Hkv)d] and dy is
    dO [L, Hq d].
    """
    base = 1000 * w.wid if seed_base is None else seed_base
    d = w.head_dim
    out = {}
    if w.projection:
        out["x"] = draw_bf16(base + TENSOR_IDS["x"], (w.L, w.hidden), w.x_sigma)
        out["w_qkv"] = draw_bf16(base + TENSOR_IDS["w_qkv"], (w.qkv_width, w.hidden), w.w_sigma)
        out["w_o"] = draw_bf16(base + TENSOR_IDS["w_o"], (w.hidden, w.n_q * d), w.w_sigma)
        if with_grad:
            out["dy"] = draw_bf16(base + TENSOR_IDS["dy"], (w.L, w.hidden), 1.0)
    else:
        out["x"] = draw_bf16(base + TENSOR_IDS["x"], (w.L, w.qkv_width), w.x_sigma)
        out["w_qkv"] = None
        out["w_o"] = None
        if with_grad:
            out["dy"] = draw_bf16(base + TENSOR_IDS["dy"], (w.L, w.n_q * d), 1.0)
    return out
