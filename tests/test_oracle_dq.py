"""Pins for the oracle's double quantisation, 8-bit float codec, mean tree,
bf16 rounding and dequantisation (CPU only)."""
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import qlora_nf4_oracle as O


# ---------------------------------------------------------------- E4M3 codec
def _torch_e4m3_bits(x):
    t = torch.from_numpy(np.asarray(x, np.float32)).to(torch.float8_e4m3fn)
    return t.view(torch.uint8).numpy()


def test_e4m3_decode_matches_torch_for_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = O.e4m3_decode(codes)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


def test_e4m3_encode_matches_torch_on_ties_and_neighbours():
    """All representable values, every midpoint between neighbours (exact
    ties), one float32 ulp around each, random values and the subnormal range;
    torch's float8_e4m3fn conversion rounds to nearest even."""
    pos = np.array([O.e4m3_value(k) for k in range(0x7F)])
    mids = (pos[:-1] + pos[1:]) / 2
    xs = [pos, mids]
    m32 = mids.astype(np.float32)
    xs += [np.nextafter(m32, np.float32(np.inf)), np.nextafter(m32, np.float32(-np.inf))]
    rng = np.random.default_rng(5)
    xs += [rng.uniform(0, 448, 20000), rng.uniform(0, 2 ** -6, 20000),
           np.exp2(rng.uniform(-12, 8.8, 20000))]
    x = np.concatenate([np.asarray(v, np.float64) for v in xs]).astype(np.float32)
    x = x[np.abs(x) <= 448]
    x = np.concatenate([x, -x, np.array([0.0, -0.0], np.float32)])
    assert np.array_equal(O.e4m3_encode_rne(x), _torch_e4m3_bits(x))


def test_e4m3_group_absmax_code():
    assert O.e4m3_encode_rne(np.float32([256.0]))[0] == 0x78
    assert O.e4m3_encode_rne(np.float32([-256.0]))[0] == 0xF8


# ---------------------------------------------------------------- mean tree
def test_pairwise_tree_order():
    """The tree adds neighbours first: with 1 and three 2^-53 a left-to-right
    float64 sum stays at 1 (each step is a tie to even), the tree gives
    (1 + 2^-53) + (2^-53 + 2^-53) = 1 + 2^-52."""
    t = 2.0 ** -53
    v = np.array([1.0, t, t, t], np.float32)
    assert O.pairwise_tree_sum(v) == 1.0 + 2.0 ** -52
    seq = 0.0
    for x in v.astype(np.float64):
        seq += x
    assert seq == 1.0
    # zero padding to a power of two: 5 leaves -> 8
    v = np.array([1.0, t, t, t, 3.0], np.float32)
    assert O.pairwise_tree_sum(v) == (1.0 + 2.0 ** -52) + 3.0


def test_mean_close_to_exact():
    rng = np.random.default_rng(11)
    for n in (1, 3, 255, 256, 257, 4096, 11008 * 4 + 17):
        c = np.abs(rng.standard_normal(n)).astype(np.float32) * np.float32(0.05)
        mu = O.dq_mean(c)
        exact = Fraction(math.fsum(float(x) for x in c)) / n
        err = abs(Fraction(float(mu)) - exact)
        ulp = Fraction(float(np.spacing(np.float32(mu))))
        assert err <= ulp, n
    assert O.dq_mean(np.float32([1, 2, 3, 4, 5])) == np.float32(3.0)


# ---------------------------------------------------------------- DQ
def _dq_case(n_b, seed=0, outliers=True):
    rng = np.random.default_rng(seed)
    w = (rng.standard_normal(n_b * 64) * 0.02).astype(np.float32)
    if outliers:
        idx = rng.choice(w.size, w.size // 1000, replace=False)
        w[idx] *= 20
    return O.block_absmax(w)


def test_double_quantize_structure():
    c = _dq_case(256 * 3 + 100)
    code8, s2, mu = O.double_quantize(c)
    assert code8.shape == c.shape and s2.shape == (4,)
    d = (c - mu).astype(np.float32)
    for g in range(4):
        dg = d[g * 256:(g + 1) * 256]
        assert s2[g] == np.abs(dg).max()
        k = int(np.argmax(np.abs(dg)))
        assert code8[g * 256 + k] in (0x78, 0xF8)     # the group absmax maps to +-256
        # sign of each code follows the sign of the centred constant
        nz = dg != 0
        assert np.array_equal(code8[g * 256:(g + 1) * 256][nz] >= 0x80, dg[nz] < 0)


def test_block_constant_error_bound():
    """E4M3 has 3 fraction bits: relative step 2^-3, so the rounding error of
    a normal code is at most 2^-4 of |d|; subnormal codes err by at most
    2^-10 in units of s2/256; plus a few float32 roundings."""
    c = _dq_case(256 * 8)
    code8, s2, mu = O.double_quantize(c)
    cp = O.block_constants_from_dq(code8, s2, mu)
    d = np.abs(c.astype(np.float64) - float(mu))
    g = np.arange(c.size) // 256
    bound = 2.0 ** -4 * d + 2.0 ** -10 * s2[g].astype(np.float64) / 256 \
        + 4 * np.spacing(np.abs(c)).astype(np.float64)
    assert np.all(np.abs(cp.astype(np.float64) - c) <= bound)


def test_constant_tensor_is_exact():
    c = np.full(512, 0.0375, np.float32)
    code8, s2, mu = O.double_quantize(c)
    assert mu == np.float32(0.0375) and np.all(s2 == 0) and np.all(code8 == 0)
    assert np.all(O.block_constants_from_dq(code8, s2, mu) == c)


def test_centering_lowers_error():
    """ta-paperlens, double-quantisation section: the constants are positive,
    so without subtracting the mean half of the symmetric 8-bit float range
    is unused.  Quantising the same constants with mu forced to 0 (done here,
    in the test) must give a larger error than the oracle's centred codes."""
    c = _dq_case(256 * 16, seed=3)
    code8, s2, mu = O.double_quantize(c)
    err_c = np.mean(np.abs(O.block_constants_from_dq(code8, s2, mu) - c) / c)
    n_g = s2.size
    s2_0 = np.array([np.abs(c[g * 256:(g + 1) * 256]).max() for g in range(n_g)], np.float32)
    code0 = np.concatenate([O.e4m3_encode_rne((c[g * 256:(g + 1) * 256] / s2_0[g]).astype(np.float32)
                                              * np.float32(256)) for g in range(n_g)])
    err_0 = np.mean(np.abs(O.block_constants_from_dq(code0, s2_0, np.float32(0)) - c) / c)
    assert err_c < err_0


# ---------------------------------------------------------------- bf16 and dequant
def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(9)
    x = rng.standard_normal(100000).astype(np.float32) * np.float32(0.1)
    u = x.view(np.uint32)
    ties = ((u & np.uint32(0xFFFF0000)) | np.uint32(0x8000)).view(np.float32)
    near = np.concatenate([ties, np.nextafter(ties, np.float32(np.inf)),
                           np.nextafter(ties, np.float32(-np.inf))])
    x = np.concatenate([x, near, np.float32([0.0, -0.0, 1e-40, -1e-40, 3.4e38])])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(O.bf16_bits_rne(x), ref)


def test_dequantize_zero_and_error():
    rng = np.random.default_rng(2)
    w = (rng.standard_normal((64, 256)) * 0.02).astype(np.float32)
    w[5, :64] = 0.0
    w[6, 7] = 0.0
    st = O.quantize(w)
    bits = O.dequantize_bits(st)
    assert np.all(O.bf16_bits_to_f32(bits[5, :64]) == 0.0)
    assert O.bf16_bits_to_f32(bits[6, 7:8])[0] == 0.0
    wh = O.dequantize(st)
    c = O.block_absmax(w)
    cp = O.block_constants_from_dq(st["absmax_code"], st["absmax_scale"], st["absmax_offset"][0])
    q = O.nf4_levels()
    half_gap = np.diff(q).max() / 2
    err = np.abs(wh - w).reshape(-1, 64)
    bound = half_gap * c[:, None] + np.abs(cp - c)[:, None] + 2.0 ** -8 * c[:, None]
    assert np.all(err <= bound + 1e-12)


def test_dequantize_signed_zero_with_negative_constant():
    """A zero code times a negative decoded constant gives -0.0 (float32
    product, then bf16): the sign of zero is part of the bit pattern."""
    st = {"rows": 1, "cols": 64, "codes": np.full(32, 0x77, np.uint8),
          "absmax_code": np.array([0xF8], np.uint8), "absmax_scale": np.float32([2.0]),
          "absmax_offset": np.float32([1.0])}
    bits = O.dequantize_bits(st)
    # c' = RN32(-1 * 2 + 1) = -1; q[7] * -1 = -0.0
    assert np.all(bits == 0x8000)
