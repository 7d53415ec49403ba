"""Pins for the oracle's merge of the adapter into the dequantised base (CPU only).

waylandz LLM book 26.2 (inference: W_merged = W + (alpha/r) B A, merged once);
ta-paperlens, pitfalls section, and the Ultralytics QLoRA page, trade-offs
section: the merge is done on the base dequantised to 16 bit."""
import numpy as np

from oracle import qlora_nf4_oracle as O


def _ones_weight_state(rows=16, cols=64):
    """A weight of all ones dequantises to exactly 1.0: every block constant
    is 1, the mean is 1, the centred constants and the group scale are 0, so
    c' = 1, and the code is the top level, 1.0."""
    state = O.quantize(np.ones((rows, cols), np.float32))
    bits = O.dequantize_bits(state)
    assert np.all(bits == 0x3F80)
    return bits


def test_merge_hand_derived_bf16_bits():
    """r = 16, alpha = 32 (s = 2); A has 2^-4 in its first row, B puts
    value_n in column 0 of row n, so s B A = value_n / 8 on every column of
    row n, added to 1.0 and rounded to bf16 (7 fraction bits; ulp 2^-7
    above 1, 2^-8 below)."""
    rows, cols, r, alpha = 16, 64, 16, 32.0
    base = _ones_weight_state(rows, cols)
    a = np.zeros((r, cols))
    a[0, :] = 2.0 ** -4
    values_and_bits = [
        (2.0 ** -3, 0x3F82),          # 1 + 2^-6: exact, two units of the ulp
        (2.0 ** -5, 0x3F80),          # 1 + 2^-8: half an ulp, tie to the even 1.0
        (3 * 2.0 ** -5, 0x3F82),      # 1 + 1.5 ulp: tie between 0x3F81 and 0x3F82 -> even
        (-(2.0 ** -3), 0x3F7C),       # 1 - 2^-6 = 0.984375: exponent -1, fraction 124/128
        (0.0, 0x3F80),
        (2.0 ** -13, 0x3F80),         # 1 + 2^-16: far below half an ulp
        (-(2.0 ** -5), 0x3F7F),       # 1 - 2^-8: exact below 1
        (-3 * 2.0 ** -5, 0x3F7D),     # 1 - 3 * 2^-8: exact below 1
    ]
    b = np.zeros((rows, r))
    for n, (v, _) in enumerate(values_and_bits):
        b[n, 0] = v
    got = O.merge_bits(base, a, b, alpha, r)
    for n, (_, want) in enumerate(values_and_bits):
        assert np.all(got[n] == want), (n, hex(int(got[n, 0])), hex(want))
    assert np.all(got[len(values_and_bits):] == 0x3F80)


def test_merge_with_zero_b_is_the_dequantised_weight():
    """waylandz 26.2.3: with B = 0 the adapter adds nothing, bit for bit."""
    rng = np.random.default_rng(11)
    w = (rng.standard_normal((32, 192)) * 0.02).astype(np.float32)
    bits = O.dequantize_bits(O.quantize(w))
    a = rng.standard_normal((16, 192)) / 4
    got = O.merge_bits(bits, a, np.zeros((32, 16)), 32.0, 16)
    assert np.array_equal(got, bits)


def test_merge_within_half_an_ulp_of_the_exact_sum():
    """Each merged value is the bf16 nearest to w_hat + s B A up to the
    float32 roundings before it, which are relative to the two addends:
    |merged - exact| <= ulp/2 + 2^-20 (|w_hat| + |s B A|).  A dropped scale,
    a wrong sign or a transposed product misses this."""
    rng = np.random.default_rng(12)
    rows, cols, r, alpha = 48, 320, 32, 16.0
    w = (rng.standard_normal((rows, cols)) * 0.02).astype(np.float32)
    bits = O.dequantize_bits(O.quantize(w))
    a = O.bf16_bits_to_f32(O.bf16_bits_rne(
        (rng.standard_normal((r, cols)) / np.sqrt(r)).astype(np.float32))).astype(np.float64)
    b = O.bf16_bits_to_f32(O.bf16_bits_rne(
        (rng.standard_normal((rows, r)) * 0.05).astype(np.float32))).astype(np.float64)
    got = O.bf16_bits_to_f32(O.merge_bits(bits, a, b, alpha, r)).astype(np.float64)
    base = O.bf16_bits_to_f32(bits).astype(np.float64)
    delta = (alpha / r) * (b @ a)
    exact = base + delta
    ulp = np.abs(np.spacing(got.astype(np.float32))).astype(np.float64) * 2.0 ** 16   # bf16 ulp
    assert np.all(np.abs(got - exact) <= ulp / 2 + 2.0 ** -20 * (np.abs(base) + np.abs(delta)))
    # and the adapter really moved the weights
    assert np.mean(got != O.bf16_bits_to_f32(bits)) > 0.5
