"""Pins for the oracle's NF4 table, encoder and packing (CPU only).

Each test checks the oracle against something other than itself: values the
pages print, another library's routine, exact rational brute force, or an
invariant the pages state.
"""
import json
import os
import statistics
from fractions import Fraction

import numpy as np
import pytest
import torch

import workloads as WL
from oracle import qlora_nf4_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _ulp_diff(a, b):
    ia = np.asarray(a, np.float32).view(np.int32).astype(np.int64)
    ib = np.asarray(b, np.float32).view(np.int32).astype(np.int64)
    # map sign-magnitude to a monotone integer line
    ia = np.where(ia < 0, -(ia & 0x7FFFFFFF), ia)
    ib = np.where(ib < 0, -(ib & 0x7FFFFFFF), ib)
    return np.abs(ia - ib)


# ---------------------------------------------------------------- NF4 table
def test_table_invariants():
    """ta-paperlens, NF4 section: exact zero, endpoints exactly -1 and +1,
    dense near 0; Ultralytics code example: 7 negative, one 0, 8 positive."""
    q = O.nf4_levels()
    assert q.dtype == np.float32 and q.shape == (16,)
    assert np.all(np.diff(q) > 0)
    assert q[0] == -1.0 and q[15] == 1.0
    assert q[7] == 0.0 and not np.signbit(q[7])
    assert (q < 0).sum() == 7 and (q > 0).sum() == 8
    gaps = np.diff(q)
    assert gaps[6] < gaps[0] and gaps[7] < gaps[14]     # denser around 0


def test_table_matches_stdlib_quantiles():
    """Same construction with Python's statistics.NormalDist inverse CDF in
    float64: identical float32 table (independent quantile routine)."""
    nd = statistics.NormalDist()
    p_pos = [0.9677083 + i * (0.5 - 0.9677083) / 8 for i in range(8)]
    p_neg = [0.9677083 + j * (0.5 - 0.9677083) / 7 for j in range(7)]
    lv = sorted([nd.inv_cdf(p) for p in p_pos] + [-nd.inv_cdf(p) for p in p_neg] + [0.0])
    mx = max(lv)
    ref = np.array([v / mx for v in lv], dtype=np.float32)
    assert np.array_equal(ref.view(np.uint32), O.nf4_levels().view(np.uint32))


def test_table_close_to_printed_snippet_in_torch_fp32():
    """The Ultralytics example evaluated literally in torch float32 gives a
    table within a few float32 ulps of the float64-evaluated one."""
    normal = torch.distributions.Normal(0.0, 1.0)
    positive = normal.icdf(torch.linspace(0.9677083, 0.5, 9)[:-1])
    negative = -normal.icdf(torch.linspace(0.9677083, 0.5, 8)[:-1])
    nf4 = torch.cat([negative, torch.zeros(1), positive]).sort().values
    nf4 = (nf4 / nf4.max()).numpy()
    assert _ulp_diff(nf4, O.nf4_levels()).max() <= 8


def test_mse_worked_example_matches_printed_values():
    """Ultralytics glossary, code example output: NF4 3.395e-06, INT4 4.053e-06
    on torch.manual_seed(0); randn(4096, 64) * 0.02 (no double quantisation)."""
    with open(os.path.join(GOLDEN, "nf4_mse_example.json")) as f:
        gold = json.load(f)
    torch.manual_seed(0)
    w = (torch.randn(4096, 64) * 0.02).numpy()
    c = O.block_absmax(w)
    for name, levels in (("nf4_mse", O.nf4_levels()),
                         ("int4_mse", np.linspace(-1, 1, 16).astype(np.float32))):
        codes = O.nf4_encode(w, c, levels=levels).reshape(-1, 64)
        restored = (levels[codes] * c[:, None]).astype(np.float32)
        mse = float(np.mean((restored - w).astype(np.float64) ** 2))
        assert f"{mse:.3e}" == gold[name], (name, mse)


# ---------------------------------------------------------------- encoder
def _rn32_exact(fr: Fraction) -> np.float32:
    """Nearest float32 to an exact rational, ties to even (brute force)."""
    f = np.float32(float(fr))
    cands = {f, np.nextafter(f, np.float32(np.inf)), np.nextafter(f, np.float32(-np.inf))}
    best = None
    for cnd in cands:
        d = abs(Fraction(float(cnd)) - fr)
        even = (int(np.array(cnd, np.float32).view(np.uint32)) & 1) == 0
        key = (d, 0 if even else 1)
        if best is None or key < best[0]:
            best = (key, cnd)
    return np.float32(best[1])


def _brute_codes(w_block, levels):
    """First argmin over levels of |RN32(w / c) - q_k| in exact rationals."""
    c = max(abs(float(x)) for x in w_block)
    out = []
    for x in w_block:
        if c == 0:
            out.append(O.NF4_ZERO_CODE)
            continue
        r = Fraction(float(_rn32_exact(Fraction(float(x)) / Fraction(c))))
        dist = [abs(r - Fraction(float(q))) for q in levels]
        out.append(min(range(16), key=lambda k: (dist[k], k)))
    return out


def test_encode_brute_force_random_blocks():
    rng = np.random.default_rng(1234)
    q = O.nf4_levels()
    for trial in range(12):
        scale = 10.0 ** rng.uniform(-6, 2)
        w = (rng.standard_normal(64) * scale).astype(np.float32)
        if trial % 3 == 0:
            w[rng.integers(64)] *= 30      # an outlier sets the scale
        got = O.nf4_encode(w, O.block_absmax(w))
        assert list(got) == _brute_codes(w, q)


def test_encode_midpoints_ties_and_neighbours():
    """Exact ties go to the lower index; one ulp either side decides."""
    q = O.nf4_levels()
    mids = (q[:-1].astype(np.float64) + q[1:].astype(np.float64)) / 2
    vals = [np.float32(1.0), np.float32(-1.0), np.float32(0.0), np.float32(-0.0)]
    n_ties = 0
    for m in mids:
        f = np.float32(m)
        if float(f) == m:
            n_ties += 1
        for v in (f, np.nextafter(f, np.float32(2)), np.nextafter(f, np.float32(-2))):
            vals.append(np.float32(v))
    assert n_ties >= 1   # some midpoints are float32 numbers, so ties do occur
    vals = np.array(vals, dtype=np.float32)
    vals = np.concatenate([vals, np.zeros((-len(vals)) % 64, np.float32)])
    # c = 1 exactly (the block contains +1), so r = w exactly
    for blk in vals.reshape(-1, 64):
        blk = blk.copy()
        blk[0] = 1.0
        got = O.nf4_encode(blk, O.block_absmax(blk))
        assert list(got) == _brute_codes(blk, q)
        for x, k in zip(blk, got):
            if float(x) in set(mids.tolist()):
                j = int(np.where(mids == float(x))[0][0])
                assert k == j           # lower of the two neighbours


def test_encode_zero_block_and_signed_zero():
    w = np.zeros(64, np.float32)
    assert np.all(O.nf4_encode(w, O.block_absmax(w)) == 7)
    w = np.full(64, -0.0, np.float32)
    assert np.all(O.nf4_encode(w, O.block_absmax(w)) == 7)
    w = np.zeros(64, np.float32)
    w[3] = -0.5
    w[5] = -0.0
    codes = O.nf4_encode(w, O.block_absmax(w))
    assert codes[3] == 0 and codes[5] == 7 and codes[0] == 7


def test_encode_monotone_and_absmax_survives():
    """Codes never decrease as w grows; the block absmax maps to code 0 or 15
    and c * q[code] gives back +-c exactly (ta-paperlens NF4 section)."""
    rng = np.random.default_rng(7)
    q = O.nf4_levels()
    w = np.sort(rng.standard_normal(64 * 50).astype(np.float32)).reshape(50, 64)
    w[:, :] = np.sort(w, axis=1)
    c = O.block_absmax(w)
    codes = O.nf4_encode(w, c).reshape(50, 64)
    assert np.all(np.diff(codes.astype(int), axis=1) >= 0)
    for b in range(50):
        i = int(np.argmax(np.abs(w[b])))
        assert codes[b, i] in (0, 15)
        assert np.float32(q[codes[b, i]] * c[b]) == np.float32(abs(w[b, i])) * np.sign(w[b, i])


def test_pack_order_and_roundtrip():
    codes = np.array([1, 2, 3, 4, 15, 0, 7, 8], dtype=np.uint8)
    packed = O.pack_nibbles(codes)
    assert list(packed) == [0x21, 0x43, 0x0F, 0x87]
    rng = np.random.default_rng(3)
    c = rng.integers(0, 16, 4096).astype(np.uint8)
    assert np.array_equal(O.unpack_nibbles(O.pack_nibbles(c)), c)


def test_lora_param_counts_printed():
    with open(os.path.join(GOLDEN, "storage_and_counts.json")) as f:
        gold = json.load(f)
    for key in ("lora_params_4096_r16", "lora_params_1024x512_r32"):
        g = gold[key]
        assert O.lora_param_count(g["d"], g["k"], g["r"]) == g["value"]


@pytest.mark.parametrize("rows,cols", [(1024, 1024), (4096, 4096), (8192, 22016)])
def test_storage_bits_closed_form(rows, cols):
    """ta-paperlens, double-quantisation section: 4 + 8/64 + 32/(64*256) bits
    per parameter (printed 4.127); Ultralytics: constants 0.5 -> ~0.127 bit."""
    with open(os.path.join(GOLDEN, "storage_and_counts.json")) as f:
        gold = json.load(f)
    n = rows * cols
    bits = O.storage_bits_per_param(rows, cols)
    # every config has a whole number of 256-block groups, so the closed form is exact
    assert (n // 64) % 256 == 0
    closed = Fraction(4) + Fraction(8, 64) + Fraction(32, 64 * 256) + Fraction(32, n)
    assert abs(bits - float(closed)) <= 1e-12
    assert round(bits, 3) == gold["storage_bits_with_double_quant"]["value"]
    assert round(bits - 4, 3) == gold["constant_overhead_after_dq"]["value"]
    no_dq = 4 + 32 / 64
    assert no_dq == gold["storage_bits_without_double_quant"]["value"]
    assert round(no_dq - bits, 3) == gold["saving_bits"]["value"]


def test_sampled_rows_equal_full_quantize_rows():
    """The sampled-row helpers (used for checks at full size) agree with the
    full quantize / dequantize on every selected row, including the first and
    last row and rows whose blocks straddle DQ-group boundaries."""
    w = WL.weight(96, 704, seed=13, outliers=True)     # 1056 blocks, 5 DQ groups
    sel = np.array([0, 5, 23, 24, 71, 95])
    full = O.quantize(w)
    part = O.quantize_sampled_rows(w, sel)
    for k in ("absmax_code", "absmax_scale", "absmax_offset"):
        assert np.array_equal(np.asarray(part[k]).view(np.uint8), np.asarray(full[k]).view(np.uint8))
    assert np.array_equal(part["codes"], full["codes"].reshape(96, 352)[sel])
    assert np.array_equal(O.dequantize_sampled_bits(part), O.dequantize_bits(full)[sel])


def test_sampled_cols_equal_full_dequantize_cols():
    """The sampled-column helpers agree with the full dequantisation on every
    selected column (columns in shared and separate blocks, first and last)."""
    w = WL.weight(96, 704, seed=14, outliers=True)
    sel = np.array([0, 3, 63, 64, 130, 131, 500, 703])
    full = O.dequantize_bits(O.quantize(w))
    part = O.quantize_sampled_cols(w, sel)
    assert np.array_equal(O.dequantize_sampled_cols_bits(part), full[:, sel])
