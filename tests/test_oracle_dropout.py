"""Pins for the oracle's lora_dropout (CPU only): the Philox-4x32-10 stream
against its published known-answer vectors, the keep decision and its
packing, the keep rate, and the layer with dropout against the plain layer
and against finite differences.

The pages set lora_dropout in the adapter config (ta-paperlens コードで見る;
waylandz 26.4.2, 26.5.1, 26.6.4) and define no random stream; the stream is
Philox-4x32-10 (Salmon, Moraes, Dror, Shaw, SC11)."""
import json
import os

import numpy as np
import pytest

from oracle import qlora_nf4_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "philox4x32_10_kat.json")


def _kat():
    with open(GOLDEN) as f:
        vec = json.load(f)["vectors"]
    for v in vec:
        yield (tuple(int(x, 16) for x in v["counter"]), tuple(int(x, 16) for x in v["key"]),
               tuple(int(x, 16) for x in v["output"]))


def test_philox_known_answer_vectors():
    for ctr, key, out in _kat():
        assert O.philox4x32_10(ctr, key) == out


def test_philox_array_form_matches_the_scalar_form():
    """The vectorised form on the published vectors and on random counters
    and keys, including words with the top bit set."""
    for ctr, key, out in _kat():
        got = O.philox4x32_10_array(*(np.array([c]) for c in ctr), key)
        assert tuple(int(w[0]) for w in got) == out
    rng = np.random.default_rng(0)
    for _ in range(20):
        key = tuple(int(v) for v in rng.integers(0, 2 ** 32, 2))
        ctr = rng.integers(0, 2 ** 32, (4, 50))
        got = O.philox4x32_10_array(*ctr, key)
        for i in range(50):
            assert tuple(int(w[i]) for w in got) == O.philox4x32_10(tuple(ctr[:, i]), key)


def test_threshold_closed_form():
    assert O.dropout_threshold(0.0) == 0
    assert O.dropout_threshold(0.5) == 2 ** 31
    assert O.dropout_threshold(0.05) == 214748364          # 0.05 * 2^32 = 214748364.8
    assert O.dropout_threshold(np.nextafter(1.0, 0.0)) == 2 ** 32 - 1
    for bad in (-0.1, 1.0, float("nan")):
        with pytest.raises(ValueError):
            O.dropout_threshold(bad)


def test_keep_decision_of_single_elements():
    """Element (t, k): word t mod 4 of the call at counter (k, t // 4,
    offset low, offset high), key (seed low, seed high); seed and offset
    above 2^32 check the split into words."""
    seed, offset, p = 0x1234_5678_9ABC_DEF0, 0xFEDC_BA98_7654_3210, 0.3
    thr = O.dropout_threshold(p)
    keep = O.dropout_keep_mask(11, 6, p, seed, offset)
    for t, k in [(0, 0), (1, 0), (2, 5), (3, 3), (4, 0), (7, 2), (10, 5)]:
        words = O.philox4x32_10((k, t // 4, offset & 0xFFFFFFFF, offset >> 32),
                                (seed & 0xFFFFFFFF, seed >> 32))
        assert keep[t, k] == (words[t % 4] >= thr)
    sel = [10, 2, 7]
    assert np.array_equal(O.dropout_keep_mask(11, 6, p, seed, offset, tokens=sel), keep[sel])
    feats = [5, 0, 3]
    assert np.array_equal(O.dropout_keep_mask(11, 6, p, seed, offset, features=feats),
                          keep[:, feats])
    assert np.array_equal(O.dropout_keep_mask(11, 6, p, seed, offset, tokens=sel,
                                              features=feats), keep[sel][:, feats])


def test_p_zero_keeps_everything():
    assert O.dropout_keep_mask(37, 64, 0.0, 1, 2).all()


@pytest.mark.parametrize("p", [0.05, 0.5, 0.9])
def test_keep_rate_and_positions(p):
    """The kept fraction is within 5 standard deviations of 1 - p overall and
    for each of the four words of a call (a wrong word index or a wrong
    comparison shows here); two offsets give independent masks."""
    T, cols = 512, 1024
    keep = O.dropout_keep_mask(T, cols, p, 7, 0)
    q = 1.0 - O.dropout_threshold(p) / 2.0 ** 32
    sd = np.sqrt(q * (1 - q) / keep.size)
    assert abs(keep.mean() - q) < 5 * sd
    for j in range(4):
        part = keep[j::4]
        assert abs(part.mean() - q) < 5 * np.sqrt(q * (1 - q) / part.size)
    other = O.dropout_keep_mask(T, cols, p, 7, 1)
    agree = np.mean(keep == other)
    want = q * q + (1 - q) * (1 - q)
    assert abs(agree - want) < 5 * np.sqrt(want * (1 - want) / keep.size)


def test_mask_bytes_layout():
    """Hand-packed example: T = 6 (a partial last quad), 4 features."""
    keep = np.array([[1, 0, 1, 1],
                     [0, 0, 1, 0],
                     [1, 1, 1, 0],
                     [1, 0, 0, 0],
                     [0, 1, 1, 1],
                     [1, 1, 0, 1]], dtype=bool)
    # quad 0, feature 0: tokens 0..3 -> bits 1,0,1,1 = 0xD; feature 1: 0,0,1,0 = 0x4
    # feature 2: 1,1,1,0 = 0x7; feature 3: 1,0,0,0 = 0x1
    # quad 1 (tokens 4, 5; 6 and 7 absent): f0 0,1 = 0x2; f1 1,1 = 0x3; f2 1,0 = 0x1; f3 1,1 = 0x3
    want = np.array([[0x4D, 0x17], [0x32, 0x31]], dtype=np.uint8)
    assert np.array_equal(O.dropout_mask_bytes(keep), want)


def _case(t=6, n=5, k=64, r=2, seed=3):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((t, k))
    w = rng.standard_normal((n, k)) * 0.02
    a = rng.standard_normal((r, k)) / np.sqrt(r)
    b = rng.standard_normal((n, r)) * 0.1
    dy = rng.standard_normal((t, n))
    return x, w, a, b, dy


def test_keep_all_is_the_plain_layer_exactly():
    x, w, a, b, dy = _case()
    keep = np.ones(x.shape, dtype=bool)
    y0, u0 = O.linear_forward(x, w, a, b, 6.0, 2)
    y1, u1 = O.linear_forward_dropout(x, w, a, b, 6.0, 2, keep, 0.0)
    assert np.array_equal(y0, y1) and np.array_equal(u0, u1)
    g0 = O.linear_backward(x, dy, w, a, b, 6.0, 2)
    g1 = O.linear_backward_dropout(x, dy, w, a, b, 6.0, 2, keep, 0.0)
    for u, v in zip(g0, g1):
        assert np.array_equal(u, v)


def test_keep_none_leaves_only_the_frozen_path():
    x, w, a, b, dy = _case()
    keep = np.zeros(x.shape, dtype=bool)
    y, u = O.linear_forward_dropout(x, w, a, b, 6.0, 2, keep, 0.25)
    assert np.array_equal(y, x @ w.T) and not u.any()
    dx, da, db = O.linear_backward_dropout(x, dy, w, a, b, 6.0, 2, keep, 0.25)
    assert np.array_equal(dx, dy @ w) and not da.any() and not db.any()


def test_forward_is_the_plain_layer_on_the_scaled_input_for_the_adapter():
    """Y = X W^T + s ((keep X / (1 - p)) A^T) B^T, written with the plain
    layer: base output of X plus the adapter output of the dropped input."""
    x, w, a, b, _ = _case(t=8, n=7, k=128, r=4)
    p = 0.5
    keep = O.dropout_keep_mask(8, 128, p, 3, 4)
    y, u = O.linear_forward_dropout(x, w, a, b, 8.0, 4, keep, p)
    xd = np.where(keep, x, 0.0) * 2.0
    y_adapter, u_ref = O.linear_forward(xd, np.zeros_like(w), a, b, 8.0, 4)
    assert np.allclose(y, x @ w.T + y_adapter, rtol=1e-13, atol=1e-13)
    assert np.allclose(u, u_ref, rtol=1e-13, atol=1e-13)


def _loss(x, w, a, b, dy, keep, p):
    y, _ = O.linear_forward_dropout(x, w, a, b, 5.0, 2, keep, p)
    return float(np.sum(dy * y))


@pytest.mark.parametrize("which", ["x", "a", "b"])
def test_backward_matches_finite_differences(which):
    """With the mask fixed, L = <dY, Y> is linear in each of X, A, B, so
    central differences are exact up to rounding; every entry is checked
    (a mask missing from the adapter part of dX, or a missing 1 / (1 - p),
    fails here)."""
    x, w, a, b, dy = _case(t=6, n=5, k=64, r=2, seed=9)
    p = 0.4
    keep = O.dropout_keep_mask(6, 64, p, 11, 12)
    assert 0 < keep.mean() < 1
    dx, da, db = O.linear_backward_dropout(x, dy, w, a, b, 5.0, 2, keep, p)
    param, grad = {"x": (x, dx), "a": (a, da), "b": (b, db)}[which]
    h = 1e-3
    fd = np.zeros_like(param)
    for idx in np.ndindex(param.shape):
        orig = param[idx]
        param[idx] = orig + h
        lp = _loss(x, w, a, b, dy, keep, p)
        param[idx] = orig - h
        lm = _loss(x, w, a, b, dy, keep, p)
        param[idx] = orig
        fd[idx] = (lp - lm) / (2 * h)
    assert np.allclose(grad, fd, rtol=1e-8, atol=1e-9)


def test_expectation_over_masks_is_the_plain_layer():
    """Inverted dropout keeps the mean: the average of the adapter output
    over 400 offsets is within 5 standard errors of the undropped one."""
    x, w, a, b, _ = _case(t=4, n=3, k=64, r=2, seed=5)
    p = 0.5
    y0, _ = O.linear_forward(x, w, a, b, 4.0, 2)
    ys = np.stack([O.linear_forward_dropout(x, w, a, b, 4.0, 2,
                                            O.dropout_keep_mask(4, 64, p, 21, off), p)[0]
                   for off in range(400)])
    se = ys.std(axis=0) / np.sqrt(len(ys))
    assert np.all(np.abs(ys.mean(axis=0) - y0) < 5 * se + 1e-12)
