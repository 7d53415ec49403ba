"""Pins for the oracle's storage and compute variants (CPU only): the evenly
spaced INT4 comparison codebook ([UL] code example), quantisation without
double quantisation (the [PL] 4.5-bit count), and fp16 as the compute type
([PL] 落とし穴: FP16 where BF16 is missing; [WZ] 26.6.4)."""
import json
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import qlora_nf4_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------- INT4 levels
def test_int4_levels_closed_form():
    q = O.int4_levels()
    assert q.dtype == np.float32 and q.shape == (16,)
    assert q[0] == -1.0 and q[15] == 1.0
    assert np.all(np.diff(q) > 0)
    assert np.array_equal(q[::-1], -q)                     # symmetric, so no exact 0
    assert not np.any(q == 0.0)
    for i, v in enumerate(q):                              # each the float32 nearest -1 + 2i/15
        exact = Fraction(2 * i - 15, 15)
        err = abs(Fraction(float(v)) - exact)
        ulp = Fraction(float(np.spacing(np.float32(abs(float(v)))))) if v != 0 else 0
        assert err <= ulp / 2
    assert np.array_equal(q, np.linspace(-1, 1, 16).astype(np.float32))
    # the page's own construction, torch.linspace in float32, accumulates its
    # step's rounding: up to 7 ulp (5.2e-8) near +-1/15
    t = torch.linspace(-1, 1, 16).numpy()
    assert np.max(np.abs(t.astype(np.float64) - q)) < 1e-7


def test_int4_encode_brute_force_and_zero_tie():
    """Nearest level with ties to the lower index: 0 lies exactly between
    levels 7 (-1/15) and 8 (+1/15), so a zero inside a non-zero block takes
    code 7; an all-zero block also gets code 7 and decodes to -0."""
    q = O.int4_levels()
    rng = np.random.default_rng(3)
    for _ in range(20):
        blk = (rng.standard_normal(64) * 0.02).astype(np.float32)
        blk[rng.integers(0, 64, 4)] = 0.0
        c = O.block_absmax(blk)
        got = O.nf4_encode(blk, c, levels=q)
        want = []
        for x in blk:
            r = Fraction(float(np.float32(np.float32(x) / np.float32(c[0]))))
            d = [abs(r - Fraction(float(v))) for v in q]
            want.append(min(range(16), key=lambda k: (d[k], k)))
        assert list(got) == want
        assert all(g == 7 for g, x in zip(got, blk) if x == 0.0)
    st = O.quantize(np.zeros((16, 64), np.float32), "int4", double_quant=False)
    assert np.all(O.unpack_nibbles(st["codes"]) == 7)
    assert np.all(O.dequantize_bits(st) == 0x8000)         # (-1/15) * 0 = -0


def test_printed_mse_through_quantize_without_double_quant():
    """[UL] printed output: NF4 3.395e-06, INT4 4.053e-06 on torch.manual_seed(0);
    randn(4096, 64) * 0.02, one float32 absmax per block -- the codes and
    constants that quantize() stores without double quantisation reproduce
    both to the printed digits."""
    with open(os.path.join(GOLDEN, "nf4_mse_example.json")) as f:
        gold = json.load(f)
    torch.manual_seed(0)
    w = (torch.randn(4096, 64) * 0.02).numpy()
    for qt, key in (("nf4", "nf4_mse"), ("int4", "int4_mse")):
        st = O.quantize(w, qt, double_quant=False)
        assert np.array_equal(st["absmax_scale"], O.block_absmax(w))
        codes = O.unpack_nibbles(st["codes"]).reshape(-1, 64)
        restored = (O.levels_for(qt)[codes] * st["absmax_scale"][:, None]).astype(np.float32)
        mse = float(np.mean((restored - w).astype(np.float64) ** 2))
        assert f"{mse:.3e}" == gold[key], (qt, mse)


# ---------------------------------------------------------------- DQ off
def test_storage_without_double_quant_is_the_printed_4_5_bits():
    with open(os.path.join(GOLDEN, "storage_and_counts.json")) as f:
        gold = json.load(f)
    for rows, cols in ((1024, 1024), (4096, 11008), (16, 64)):
        assert O.storage_bits_per_param(rows, cols, double_quant=False) == \
            gold["storage_bits_without_double_quant"]["value"]
    # and the saving over it is the printed 0.373 (to 3 digits) at large n
    d = O.storage_bits_per_param(8192, 22016, False) - O.storage_bits_per_param(8192, 22016)
    assert f"{d:.3f}" == f"{gold['saving_bits']['value']:.3f}"


def test_without_double_quant_the_block_absmax_survives():
    """Without double quantisation the stored constant is c itself, so the
    element of largest magnitude decodes to RN(+-c) of the compute type
    ([PL] NF4: the endpoints -1 and +1 keep the absmax exact), for both
    codebooks; with double quantisation only c' is kept."""
    rng = np.random.default_rng(5)
    w = (rng.standard_normal((32, 128)) * 0.02).astype(np.float32)
    c = O.block_absmax(w)
    idx = np.abs(w.reshape(-1, 64)).argmax(axis=1)
    for qt in ("nf4", "int4"):
        st = O.quantize(w, qt, double_quant=False)
        assert "absmax_code" not in st
        for dt in ("bf16", "fp16"):
            bits = O.dequantize_bits(st, dt).reshape(-1, 64)
            got = bits[np.arange(bits.shape[0]), idx]
            want = O.round16_bits(np.sign(w.reshape(-1, 64)[np.arange(bits.shape[0]), idx]) * c, dt)
            assert np.array_equal(got, want), (qt, dt)


def test_dequant_value_is_level_times_constant_rounded_once():
    """Each dequantised value is q[code] * c rounded once to float32 and once
    to the compute type: within half a 16-bit ulp (plus the float32 rounding)
    of the exact product."""
    rng = np.random.default_rng(6)
    w = (rng.standard_normal((16, 192)) * 0.05).astype(np.float32)
    for qt in ("nf4", "int4"):
        for dq in (False, True):
            st = O.quantize(w, qt, dq)
            cp = O.block_constants(st).astype(np.float64)
            codes = O.unpack_nibbles(st["codes"]).reshape(-1, 64)
            exact = O.levels_for(qt).astype(np.float64)[codes] * cp[:, None]
            for dt, frac_bits in (("bf16", 7), ("fp16", 10)):
                got = O.bits16_to_f32(O.dequantize_bits(st, dt), dt).astype(np.float64)
                got = got.reshape(-1, 64)
                ulp = 2.0 ** (np.floor(np.log2(np.maximum(np.abs(exact), 2.0 ** -14))) - frac_bits)
                assert np.all(np.abs(got - exact) <= ulp / 2 + np.abs(exact) * 2.0 ** -24), (qt, dq, dt)


# ---------------------------------------------------------------- fp16
def test_fp16_rounding_against_torch_and_hand_cases():
    rng = np.random.default_rng(7)
    x = np.concatenate([rng.standard_normal(10000).astype(np.float32) * 10.0 ** rng.integers(-8, 5, 10000),
                        np.float32([1 + 2 ** -11, 1 + 3 * 2 ** -11, 65504.0, 65520.0, 2 ** -24,
                                    2 ** -25, 3 * 2 ** -26, -0.0, 0.0, 2 ** -14, -(2 ** -15)])])
    x = x.astype(np.float32)
    got = O.f16_bits_rne(x)
    want = torch.from_numpy(x).to(torch.float16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, want)
    hand = dict(zip([1 + 2 ** -11, 1 + 3 * 2 ** -11, 65504.0, 65520.0, 2 ** -24, 2 ** -25,
                     3 * 2 ** -26, -0.0, 2 ** -14, -(2 ** -15)],
                    [0x3C00, 0x3C02, 0x7BFF, 0x7C00, 0x0001, 0x0000, 0x0001, 0x8000, 0x0400,
                     0x8200]))
    for v, bits in hand.items():
        assert int(O.f16_bits_rne(np.float32([v]))[0]) == bits, v
    assert np.array_equal(O.f16_bits_to_f32(O.f16_bits_rne(np.float32([0.1, -3.5]))),
                          np.float32([0.0999755859375, -3.5]))


def test_fp16_merge_hand_derived_bits():
    """Merge in fp16 (10 fraction bits: ulp 2^-10 above 1, 2^-11 below):
    base 1.0, s = 2, A has 2^-4 in row 0, B puts value_n in column 0 of
    row n, so the added term is value_n / 8."""
    rows, cols, r, alpha = 16, 64, 16, 32.0
    base = np.full((rows, cols), 0x3C00, np.uint16)           # fp16 1.0
    a = np.zeros((r, cols))
    a[0, :] = 2.0 ** -4
    vals = [(8 * 2.0 ** -10, 0x3C01),      # 1 + 2^-10: one ulp
            (8 * 2.0 ** -11, 0x3C00),      # 1 + 2^-11: half an ulp, tie to even 1.0
            (8 * 3 * 2.0 ** -11, 0x3C02),  # 1 + 1.5 ulp: tie -> even 0x3C02
            (-8 * 2.0 ** -11, 0x3BFF),     # 1 - 2^-11: exact below 1
            (-8 * 2.0 ** -4, 0x3B80)]      # 1 - 2^-4 = 0.9375
    b = np.zeros((rows, r))
    for n, (v, _) in enumerate(vals):
        b[n, 0] = v
    got = O.merge_bits(base, a, b, alpha, r, compute_dtype="fp16")
    for n, (_, want) in enumerate(vals):
        assert np.all(got[n] == want), (n, hex(int(got[n, 0])), hex(want))
    assert np.all(got[len(vals):] == 0x3C00)


def test_variant_states_validate():
    with pytest.raises(ValueError):
        O.levels_for("fp4")
    with pytest.raises(ValueError):
        O.round16_bits(np.float32([1.0]), "fp32")


def test_int4_zero_threshold_with_denormal_quotients():
    """The INT4 threshold at 0 sees the quotient's sign and zero-ness: with
    c = 1, w = +2^-149 gives r = 2^-149 > 0 (code 8) and -2^-149 gives code 7;
    with c = 4, w = 2^-149 gives r = RN32(2^-151) = 0 (code 7)."""
    q = O.int4_levels()
    tiny = np.float32(2.0 ** -149)
    blk = np.zeros(64, np.float32)
    blk[0] = 1.0
    blk[1], blk[2] = tiny, -tiny
    codes = O.nf4_encode(blk, O.block_absmax(blk), levels=q)
    assert (codes[1], codes[2]) == (8, 7)
    blk[0] = 4.0
    codes = O.nf4_encode(blk, O.block_absmax(blk), levels=q)
    assert (codes[1], codes[2]) == (7, 7)
