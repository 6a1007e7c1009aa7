"""Pins of the sequence-tiled cross-entropy oracle (CPU only) against things
other than itself: torch's cross_entropy with autograd, central differences,
the closed form of a zero output weight, the zero vocabulary sum of the
weight gradient, the ignore-index and out-of-range readings, and invariance
under the tile size."""
import math

import numpy as np
import pytest
import torch

import oracle

RNG = np.random.default_rng(77)
IGN = -100


def _problem(L=11, D=6, V=9, n_ignored=3):
    h = RNG.standard_normal((L, D))
    w = RNG.standard_normal((V, D)) * 0.7
    t = RNG.integers(0, V, size=L)
    t[RNG.choice(L, size=n_ignored, replace=False)] = IGN
    return h, w, t


@pytest.mark.parametrize("tile", [1, 4, 11, 50])
@pytest.mark.parametrize("dloss", [1.0, 0.37])
def test_loss_matches_torch_cross_entropy(tile, dloss):
    """torch's cross_entropy (mean over non-ignored targets) and autograd in
    float64 on the CPU, one untiled pass."""
    h, w, t = _problem()
    th, tw = torch.tensor(h, requires_grad=True), torch.tensor(w, requires_grad=True)
    logits = th @ tw.T
    tl = torch.nn.functional.cross_entropy(logits, torch.tensor(t), ignore_index=IGN, reduction="mean")
    (tl * dloss).backward()
    loss, lse = oracle.loss_fwd(h, w, t, IGN, tile)
    dh, dw = oracle.loss_bwd(h, w, t, IGN, lse, dloss, tile)
    assert abs(loss - tl.item()) <= 1e-13
    np.testing.assert_allclose(lse, torch.logsumexp(logits, dim=1).detach().numpy(), rtol=0, atol=1e-13)
    np.testing.assert_allclose(dh, th.grad.numpy(), rtol=0, atol=1e-14)
    np.testing.assert_allclose(dw, tw.grad.numpy(), rtol=0, atol=1e-14)


def test_loss_backward_matches_central_differences():
    h, w, t = _problem(L=5, D=3, V=7, n_ignored=1)
    dloss = 1.3

    def f(h_, w_):
        return dloss * oracle.loss_fwd(h_, w_, t, IGN, 2)[0]

    _, lse = oracle.loss_fwd(h, w, t, IGN, 2)
    dh, dw = oracle.loss_bwd(h, w, t, IGN, lse, dloss, 2)
    eps = 1e-6
    for arr, grad in ((h, dh), (w, dw)):
        num = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            a0 = arr[idx]
            arr[idx] = a0 + eps
            fp = f(h, w)
            arr[idx] = a0 - eps
            fm = f(h, w)
            arr[idx] = a0
            num[idx] = (fp - fm) / (2 * eps)
        np.testing.assert_allclose(grad, num, rtol=0, atol=1e-8)


def test_zero_weight_closed_form():
    """W = 0: every logit is 0, the softmax is uniform 1/V, the loss and every
    row's log-sum-exp are log V, dh = 0 and dW[v] = dloss/count *
    sum_r (1/V - [v == t_r]) h_r over the valid rows."""
    h, _, t = _problem(L=8, D=5, V=6, n_ignored=2)
    V = 6
    w = np.zeros((V, 5))
    loss, lse = oracle.loss_fwd(h, w, t, IGN, 3)
    assert abs(loss - math.log(V)) <= 1e-15
    np.testing.assert_allclose(lse, np.full(8, math.log(V)), rtol=0, atol=1e-15)
    dh, dw = oracle.loss_bwd(h, w, t, IGN, lse, 2.0, 3)
    assert np.abs(dh).max() == 0.0
    valid = t != IGN
    expect = np.zeros((V, 5))
    for r in np.nonzero(valid)[0]:
        expect += (1.0 / V) * h[r]
        expect[t[r]] -= h[r]
    expect *= 2.0 / valid.sum()
    np.testing.assert_allclose(dw, expect, rtol=0, atol=1e-14)


def test_weight_gradient_sums_to_zero_over_the_vocabulary():
    """Each valid row's softmax minus its one-hot target sums to zero, so the
    weight gradient summed over the vocabulary rows vanishes (a dropped
    target term or a wrong normalisation breaks this)."""
    h, w, t = _problem(L=20, D=7, V=13, n_ignored=4)
    _, lse = oracle.loss_fwd(h, w, t, IGN, 6)
    dh, dw = oracle.loss_bwd(h, w, t, IGN, lse, 1.0, 6)
    assert np.abs(dw.sum(axis=0)).max() <= 1e-14
    # and every valid row of dh is that row's dlogits times W, with dlogits
    # summing to zero: projecting dh on a W shifted by a constant row changes
    # nothing
    assert np.abs(dh).max() > 1e-3


def test_ignored_rows_and_all_ignored():
    h, w, t = _problem(L=9, D=4, V=5, n_ignored=4)
    loss, lse = oracle.loss_fwd(h, w, t, IGN, 4)
    dh, _ = oracle.loss_bwd(h, w, t, IGN, lse, 1.0, 4)
    assert np.all(dh[t == IGN] == 0.0)
    # the mean runs over the valid rows only
    valid = t != IGN
    manual = np.mean([lse[r] - (h[r] @ w[t[r]]) for r in np.nonzero(valid)[0]])
    assert abs(loss - manual) <= 1e-14
    t_all = np.full(9, IGN)
    loss0, lse0 = oracle.loss_fwd(h, w, t_all, IGN, 4)
    dh0, dw0 = oracle.loss_bwd(h, w, t_all, IGN, lse0, 1.0, 4)
    assert loss0 == 0.0 and np.all(dh0 == 0.0) and np.all(dw0 == 0.0)


def test_out_of_range_target_is_nan():
    h, w, t = _problem(L=6, D=4, V=5, n_ignored=1)
    t = t.copy()
    bad = int(np.nonzero(t != IGN)[0][0])
    t[bad] = 5  # == V
    loss, lse = oracle.loss_fwd(h, w, t, IGN, 4)
    dh, dw = oracle.loss_bwd(h, w, t, IGN, lse, 1.0, 4)
    assert math.isnan(loss)
    assert np.isnan(dh[bad]).all()
    others = [r for r in range(6) if r != bad]
    assert np.isfinite(dh[others]).all()
    assert np.isnan(dw).all()


def test_tile_invariance():
    h, w, t = _problem(L=23, D=5, V=8, n_ignored=5)
    ref_loss, ref_lse = oracle.loss_fwd(h, w, t, IGN, 23)
    ref_dh, ref_dw = oracle.loss_bwd(h, w, t, IGN, ref_lse, 1.0, 23)
    for tile in (1, 2, 7, 100):
        loss, lse = oracle.loss_fwd(h, w, t, IGN, tile)
        dh, dw = oracle.loss_bwd(h, w, t, IGN, lse, 1.0, tile)
        assert abs(loss - ref_loss) <= 1e-14
        np.testing.assert_allclose(lse, ref_lse, rtol=0, atol=1e-14)
        np.testing.assert_allclose(dh, ref_dh, rtol=0, atol=1e-15)
        np.testing.assert_allclose(dw, ref_dw, rtol=0, atol=1e-14)


def test_large_logits_do_not_overflow():
    """Logits of 1000 would overflow a plain exp; the shifted log-sum-exp
    equals the exact value 1000 + log(1 + (V-1) e^-1000) = 1000."""
    z = np.array([[1000.0, 0.0, 0.0, 0.0], [-1000.0, -1000.0, -1000.0, -1000.0]])
    np.testing.assert_allclose(oracle.logsumexp_rows(z), [1000.0, -1000.0 + math.log(4)], rtol=0,
                               atol=1e-12)
