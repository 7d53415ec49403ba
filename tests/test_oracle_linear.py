"""Pins for the oracle's LoRA linear forward and backward (CPU only)."""
import numpy as np
import pytest

from oracle import qlora_nf4_oracle as O


def _case(t=3, n=5, k=64, r=2, seed=0):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((t, k))
    w = rng.standard_normal((n, k)) * 0.02
    a = rng.standard_normal((r, k)) / np.sqrt(r)
    b = rng.standard_normal((n, r)) * 0.1
    dy = rng.standard_normal((t, n))
    return x, w, a, b, dy


def test_forward_matches_scalar_loops():
    """ta-paperlens, gradient section: h = W x + B A x per token column;
    waylandz 26.2.4: the adapter term carries alpha / r."""
    x, w, a, b, _ = _case()
    alpha, r = 6.0, 2
    y, u = O.linear_forward(x, w, a, b, alpha, r)
    t, k = x.shape
    n = w.shape[0]
    for i in range(t):
        ax = [sum(a[j, kk] * x[i, kk] for kk in range(k)) for j in range(r)]
        assert np.allclose(u[i], ax, rtol=1e-13, atol=1e-13)
        for o in range(n):
            wx = sum(w[o, kk] * x[i, kk] for kk in range(k))
            bax = sum(b[o, j] * ax[j] for j in range(r))
            assert abs(y[i, o] - (wx + alpha / r * bax)) <= 1e-12 * (1 + abs(y[i, o]))


def test_forward_b_zero_is_base_output_exactly():
    """waylandz 26.2.3: with B = 0 the adapted layer is the original layer."""
    x, w, a, b, _ = _case(t=4, n=7, k=128, r=4)
    y, _ = O.linear_forward(x, w, a, np.zeros_like(b), 8.0, 4)
    assert np.array_equal(y, x @ w.T)
    y, _ = O.linear_forward(x, w, np.zeros_like(a), b, 8.0, 4)
    assert np.array_equal(y, x @ w.T)


def test_forward_merged_identity():
    """waylandz 26.2.2: merging gives W + (alpha/r) B A; same output."""
    x, w, a, b, _ = _case(t=4, n=7, k=128, r=4)
    y, _ = O.linear_forward(x, w, a, b, 8.0, 4)
    assert np.allclose(y, x @ (w + 2.0 * b @ a).T, rtol=1e-12, atol=1e-12)


def _loss(x, w, a, b, dy, alpha, r):
    y, _ = O.linear_forward(x, w, a, b, alpha, r)
    return float(np.sum(dy * y))


@pytest.mark.parametrize("which", ["x", "a", "b"])
def test_backward_matches_finite_differences(which):
    """L = <dY, Y> is linear in each of X, A, B, so central differences are
    exact up to rounding; every entry is checked."""
    x, w, a, b, dy = _case(t=3, n=5, k=64, r=2, seed=4)
    alpha, r = 5.0, 2
    dx, da, db = O.linear_backward(x, dy, w, a, b, alpha, r)
    target = {"x": (x, dx), "a": (a, da), "b": (b, db)}[which]
    param, grad = target
    h = 1e-3
    fd = np.zeros_like(param)
    for idx in np.ndindex(param.shape):
        orig = param[idx]
        param[idx] = orig + h
        lp = _loss(x, w, a, b, dy, alpha, r)
        param[idx] = orig - h
        lm = _loss(x, w, a, b, dy, alpha, r)
        param[idx] = orig
        fd[idx] = (lp - lm) / (2 * h)
    assert np.allclose(grad, fd, rtol=1e-8, atol=1e-9)


def test_backward_special_cases():
    """B = 0: dA = 0 and dX is the plain W^T path; no gradient for W exists
    (ta-paperlens, gradient section: only A and B are trained)."""
    x, w, a, b, dy = _case(t=4, n=6, k=64, r=2, seed=8)
    dx, da, db = O.linear_backward(x, dy, w, a, np.zeros_like(b), 4.0, 2)
    assert np.all(da == 0)
    assert np.array_equal(dx, dy @ w)
    assert np.allclose(db, 2.0 * dy.T @ (x @ a.T))
    out = O.linear_backward(x, dy, w, a, b, 4.0, 2)
    assert len(out) == 3


def test_rel_frobenius():
    ref = np.array([[3.0, 4.0]])
    assert O.rel_frobenius(ref, ref) == 0.0
    assert abs(O.rel_frobenius(ref + [[0.0, 0.05]], ref) - 0.01) < 1e-15
