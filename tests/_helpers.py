"""Shared test helpers: bf16 bit conversion between numpy and torch, and the
error metrics the parity gates use."""
import numpy as np

import synthetic


def to_dev(bits):
    """uint16 bf16 bits (numpy) -> torch bfloat16 on cuda:0."""
    import torch

    if bits is None:
        return None
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(torch.bfloat16).to("cuda:0")


def from_dev_bf16(t):
    """torch bfloat16 -> float64 numpy (exact)."""
    import torch

    bits = t.detach().view(torch.int16).cpu().numpy().view(np.uint16)
    return synthetic.bf16_bits_to_f64(bits)


def from_dev_bf16_f32(t):
    """torch bfloat16 -> float32 numpy (exact; half the host memory of fp64)."""
    import torch

    bits = t.detach().view(torch.int16).cpu().numpy().view(np.uint16)
    return synthetic.bf16_bits_to_f32(bits)


def from_dev_f32(t):
    return t.detach().cpu().numpy().astype(np.float64)


def f64(bits):
    return None if bits is None else synthetic.bf16_bits_to_f64(bits)


def max_abs(a, b):
    return float(np.max(np.abs(np.asarray(a) - np.asarray(b)))) if np.size(a) else 0.0


def rel_l2(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    den = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / den) if den > 0 else float(np.linalg.norm(a - b))
