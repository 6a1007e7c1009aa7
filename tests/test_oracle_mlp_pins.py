"""Pins of the sequence-tiled SwiGLU MLP oracle (CPU only) against things
other than itself: torch's own SiLU with autograd, central differences,
closed forms of the activation and of a zero gate, and invariance under the
tile size."""
import math

import numpy as np
import pytest
import torch

import oracle

RNG = np.random.default_rng(2024)


def _rand(*shape, scale=1.0):
    return RNG.standard_normal(shape) * scale


def _problem(L=13, D=8, F=6):
    return (_rand(L, D), _rand(2 * F, D, scale=0.5), _rand(D, F, scale=0.5), _rand(L, D))


def test_silu_known_values():
    z = np.array([0.0, 1.0, -1.0, 40.0, -40.0, 800.0, -800.0])
    s = 1.0 / (1.0 + np.exp(-np.clip(z, -700, 700)))
    np.testing.assert_allclose(oracle.silu(z), z * s, rtol=1e-14, atol=1e-300)
    assert oracle.silu(np.array([0.0]))[0] == 0.0
    assert abs(oracle.silu(np.array([1.0]))[0] - 1.0 / (1.0 + math.exp(-1.0))) < 1e-15
    # the derivative: 1/2 at 0, 1 far right, 0 far left, and central differences
    np.testing.assert_allclose(oracle.silu_grad(np.array([0.0, 40.0, -40.0])), [0.5, 1.0, 0.0],
                               atol=1e-15)
    zz = np.linspace(-6, 6, 25)
    num = (oracle.silu(zz + 1e-6) - oracle.silu(zz - 1e-6)) / 2e-6
    np.testing.assert_allclose(oracle.silu_grad(zz), num, rtol=0, atol=1e-9)


@pytest.mark.parametrize("tile", [1, 4, 13, 100])
def test_mlp_matches_torch_autograd(tile):
    """torch's F.silu and autograd in float64 on the CPU (one untiled pass)."""
    x, wgu, wd, dy = _problem()
    tx, tg, td = (torch.tensor(a, requires_grad=True) for a in (x, wgu, wd))
    F = wgu.shape[0] // 2
    ty = (torch.nn.functional.silu(tx @ tg[:F].T) * (tx @ tg[F:].T)) @ td.T
    (ty * torch.tensor(dy)).sum().backward()
    y = oracle.mlp_fwd(x, wgu, wd, tile)
    dx, dgu, dwd = oracle.mlp_bwd(x, wgu, wd, dy, tile)
    np.testing.assert_allclose(y, ty.detach().numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(dx, tx.grad.numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(dgu, tg.grad.numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(dwd, td.grad.numpy(), rtol=0, atol=1e-12)


def test_mlp_backward_matches_central_differences():
    """<y, dy> differentiated numerically in every element of x and both
    weights."""
    x, wgu, wd, dy = _problem(L=5, D=4, F=3)

    def f(x_, g_, d_):
        return float(np.sum(oracle.mlp_fwd(x_, g_, d_, 2) * dy))

    grads = oracle.mlp_bwd(x, wgu, wd, dy, 2)
    eps = 1e-6
    for which, base in enumerate((x, wgu, wd)):
        num = np.zeros_like(base)
        for idx in np.ndindex(base.shape):
            args_p = [x.copy(), wgu.copy(), wd.copy()]
            args_m = [x.copy(), wgu.copy(), wd.copy()]
            args_p[which][idx] += eps
            args_m[which][idx] -= eps
            num[idx] = (f(*args_p) - f(*args_m)) / (2 * eps)
        rel = np.linalg.norm(num - grads[which]) / np.linalg.norm(num)
        assert rel < 1e-7, (which, rel)


def test_zero_gate_closed_form():
    """W_gate = 0: h = 0, silu(0) = 0, so y = 0, dW_down = 0, dW_up = 0, dx = 0
    (dh is multiplied by W_gate = 0) and, with silu'(0) = 1/2,
    dW_gate = 1/2 ((dy W_down) * u)^T x."""
    x, wgu, wd, dy = _problem()
    F = wgu.shape[0] // 2
    wgu[:F] = 0.0
    y = oracle.mlp_fwd(x, wgu, wd, 5)
    dx, dgu, dwd = oracle.mlp_bwd(x, wgu, wd, dy, 5)
    assert np.abs(y).max() == 0.0 and np.abs(dwd).max() == 0.0
    assert np.abs(dgu[F:]).max() == 0.0 and np.abs(dx).max() == 0.0
    u = x @ wgu[F:].T
    np.testing.assert_allclose(dgu[:F], 0.5 * ((dy @ wd) * u).T @ x, rtol=0, atol=1e-12)


def test_tile_size_does_not_change_the_result():
    x, wgu, wd, dy = _problem(L=37)
    ref_y = oracle.mlp_fwd(x, wgu, wd, 37)
    ref = oracle.mlp_bwd(x, wgu, wd, dy, 37)
    for tile in (1, 3, 8, 36):
        np.testing.assert_allclose(oracle.mlp_fwd(x, wgu, wd, tile), ref_y, rtol=0, atol=1e-12)
        for a, b in zip(oracle.mlp_bwd(x, wgu, wd, dy, tile), ref):
            np.testing.assert_allclose(a, b, rtol=0, atol=1e-12)


def test_rows_are_independent():
    """Changing one input row changes that output row only (the property that
    makes sequence tiling exact)."""
    x, wgu, wd, _ = _problem(L=9)
    y0 = oracle.mlp_fwd(x, wgu, wd, 4)
    x2 = x.copy()
    x2[5] += 1.0
    y1 = oracle.mlp_fwd(x2, wgu, wd, 4)
    changed = np.abs(y1 - y0).max(axis=1) > 0
    assert changed.tolist() == [i == 5 for i in range(9)]
