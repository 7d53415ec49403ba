"""Host checks of the arithmetic shortcuts the HIP kernels take, run on the CPU
against IEEE float32 results and the oracle.

The kernels avoid a per-element division, a 15-way compare and a correctly
rounded square root instruction; each shortcut is claimed to give exactly the
IEEE / oracle result.  These tests re-run each shortcut's steps in NumPy with
exact float32 semantics (a fused multiply-add is emulated exactly, see fma32)
on large sets of adversarial inputs and compare bit for bit:

  * the quantiser's decision thresholds and NF4 / INT4 levels (literals in
    the kernel source) against the codebook construction;
  * the 32-bin code table (quantize.hip, code_of) against the count of exact
    midpoints below the quotient;
  * the scaled-significand Markstein quotient (quantize.hip) against IEEE
    float32 division;
  * the corrected square root of the AdamW kernel (adamw.hip, sqrt_rn)
    against the correctly rounded root, from every estimate within one ulp.
The GPU tests then compare the kernels' outputs with the oracle bit for bit;
these tests show the shortcuts are exact on far more inputs than a GPU test
can enumerate."""
import os
import re
from fractions import Fraction

import numpy as np
import pytest

from oracle import qlora_nf4_oracle as O

F32 = np.float32
CSRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                    "bit_nf4_quantized_06_amd", "csrc")


def _float_array(name):
    """The float32 array literal `name` of device_common.h (hex floats)."""
    src = open(os.path.join(CSRC, "device_common.h")).read()
    m = re.search(r"\b" + re.escape(name) + r"\[\d+\]\s*=\s*\{([^}]*)\}", src)
    assert m, name
    vals = []
    for tok in m.group(1).replace("\n", " ").split(","):
        tok = tok.strip().rstrip("f")
        if tok:
            vals.append(float.fromhex(tok) if "0x" in tok.lower() else float(tok))
    return np.array(vals, dtype=F32)


# --------------------------------------------------------------------------
# exact float32 fused multiply-add
# --------------------------------------------------------------------------
def fma32(a, b, c):
    """RN32(a * b + c) for float32 arrays, exactly: a * b is exact in
    float64; the float64 sum is made round-to-odd (its exact error from
    TwoSum decides) and then rounded to float32, which is correct because
    float64 carries more than 2 * 24 + 2 bits (Boldo and Melquiond's
    round-to-odd argument)."""
    a64 = np.asarray(a, dtype=F32).astype(np.float64)
    b64 = np.asarray(b, dtype=F32).astype(np.float64)
    c64 = np.asarray(c, dtype=F32).astype(np.float64)
    p = a64 * b64
    s = p + c64
    bp = s - c64
    err = (p - bp) + (c64 - (s - bp))            # TwoSum: p + c = s + err exactly
    bits = s.view(np.uint64)
    even = (bits & np.uint64(1)) == 0
    fix = (err != 0) & even & np.isfinite(s) & (s != 0)
    toward = np.where(err > 0, np.inf, -np.inf)
    s = np.where(fix, np.nextafter(s, toward), s)
    return s.astype(F32)


def test_fma32_emulation_against_exact_rationals():
    rng = np.random.default_rng(0)
    a = (rng.standard_normal(3000) * 2.0 ** rng.integers(-30, 30, 3000)).astype(F32)
    b = (rng.standard_normal(3000) * 2.0 ** rng.integers(-30, 30, 3000)).astype(F32)
    c = (-(a.astype(np.float64) * b) * (1 + rng.standard_normal(3000) * 2.0 ** -20)).astype(F32)
    got = fma32(a, b, c)
    for i in range(a.size):
        exact = Fraction(float(a[i])) * Fraction(float(b[i])) + Fraction(float(c[i]))
        ref = _rn32_fraction(exact)
        assert got[i] == ref, (a[i], b[i], c[i], got[i], ref)


def _rn32_fraction(x: Fraction) -> F32:
    """Round an exact rational to the nearest float32, ties to even."""
    if x == 0:
        return F32(0.0)
    lo = F32(float(x))             # float64 nearest, then float32: maybe off by one
    cands = [np.nextafter(lo, F32(-np.inf)), lo, np.nextafter(lo, F32(np.inf))]
    best = min(cands, key=lambda v: (abs(Fraction(float(v)) - x),
                                     int(np.asarray(v, F32).view(np.uint32)) & 1))
    return F32(best)


# --------------------------------------------------------------------------
# codebook literals of the kernels
# --------------------------------------------------------------------------
def _thresholds_from_levels(levels):
    """Largest float32 not above each exact midpoint of neighbouring levels."""
    out = []
    for k in range(15):
        mid = (Fraction(float(levels[k])) + Fraction(float(levels[k + 1]))) / 2
        t = F32(float(mid))
        while Fraction(float(t)) > mid:
            t = np.nextafter(t, F32(-np.inf))
        while Fraction(float(np.nextafter(t, F32(np.inf)))) <= mid:
            t = np.nextafter(t, F32(np.inf))
        out.append(t)
    return np.array(out, dtype=F32)


@pytest.mark.parametrize("qt", ["nf4", "int4"])
def test_kernel_levels_and_thresholds(qt):
    levels = _float_array("kNF4" if qt == "nf4" else "kINT4")
    thr = _float_array("kNF4Thr" if qt == "nf4" else "kINT4Thr")
    assert np.array_equal(levels.view(np.uint32), O.levels_for(qt).view(np.uint32))
    assert np.array_equal(thr.view(np.uint32), _thresholds_from_levels(O.levels_for(qt)).view(np.uint32))


# --------------------------------------------------------------------------
# the 32-bin code table (quantize.hip: CodeBins, code_of)
# --------------------------------------------------------------------------
def _bins(thr):
    """The kernel's table: bin i covers [i/16 - 1, (i+1)/16 - 1) and holds the
    count of thresholds below its lower edge and its one threshold (+inf if
    none)."""
    base = np.zeros(32, dtype=np.int64)
    t = np.full(32, np.inf, dtype=F32)
    for i in range(32):
        lo = F32(F32(i) / F32(16.0) - F32(1.0))
        hi = F32(F32(i + 1) / F32(16.0) - F32(1.0))
        for x in thr:
            if x < lo:
                base[i] += 1
            elif x < hi:
                assert t[i] == np.inf, "two thresholds in one bin"
                t[i] = x
    return base, t


def _code_of(r, base, t):
    bi = np.floor(fma32(r, np.full_like(r, 16.0), np.full_like(r, 16.0))).astype(np.int64)
    bi = np.minimum(bi, 31)
    assert bi.min() >= 0
    return base[bi] + (r > t[bi])


def _adversarial_quotients(thr, n_random=400_000, ulps=200):
    rng = np.random.default_rng(1)
    parts = [rng.uniform(-1, 1, n_random).astype(F32),
             np.array([-1.0, 1.0, 0.0, -0.0, 2.0 ** -149, -2.0 ** -149], dtype=F32)]
    edges = np.array([i / 16 - 1 for i in range(33)], dtype=F32)
    for x in np.concatenate([thr, edges]):
        u = np.int64(np.asarray(x, F32).view(np.int32))
        k = np.arange(-ulps, ulps + 1, dtype=np.int64)
        if x >= 0:
            bits = (u + k)
        else:
            bits = (u - k)
        v = bits[(bits > -(2 ** 31)) & (bits < 2 ** 31)].astype(np.int32).view(F32)
        parts.append(v[np.isfinite(v)])
    r = np.concatenate(parts)
    return r[(r >= -1) & (r <= 1)]


@pytest.mark.parametrize("qt", ["nf4", "int4"])
def test_code_bins_equal_threshold_count(qt):
    thr = _float_array("kNF4Thr" if qt == "nf4" else "kINT4Thr")
    base, t = _bins(thr)
    r = _adversarial_quotients(thr)
    mids = O.nf4_midpoints(O.levels_for(qt))
    ref = np.zeros(r.shape, dtype=np.int64)
    for m in mids:
        ref += r.astype(np.float64) > m
    got = _code_of(r, base, t)
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, f"{bad.size} codes differ, e.g. r={r[bad[:5]]}"


# --------------------------------------------------------------------------
# the scaled-significand Markstein quotient (quantize.hip)
# --------------------------------------------------------------------------
def _markstein_quotient(w, c):
    """r = RN32(w / c) as the kernel forms it: c = cm * 2^ex (cm in [0.5, 1)),
    y = RN32(1 / cm), wm = w * 2^-ex, q0 = RN32(wm * y), rem = fma(-q0, cm, wm),
    r = fma(rem, y, q0)."""
    cm, ex = np.frexp(c)
    cm = cm.astype(F32)
    y = (F32(1.0) / cm).astype(F32)
    wm = np.ldexp(w, -ex).astype(F32)
    q0 = (wm * y).astype(F32)
    rem = fma32(-q0, cm, wm)
    return fma32(rem, y, q0), wm


def _quotient_cases():
    rng = np.random.default_rng(2)
    n = 300_000
    c = np.abs(rng.standard_normal(n) * 2.0 ** rng.integers(-20, 20, n)).astype(F32)
    c = np.where(c == 0, F32(1.0), c)
    w = (rng.uniform(-1, 1, n) * c).astype(F32)
    parts_w, parts_c = [w, c, -c], [c, c, c]
    # quotients within 64 ulps of every NF4 / INT4 threshold, for varied c
    cs = np.abs(rng.standard_normal(600) * 2.0 ** rng.integers(-30, 30, 600)).astype(F32)
    for thr in (_float_array("kNF4Thr"), _float_array("kINT4Thr")):
        for x in thr:
            for cc in cs[:40]:
                w0 = F32(np.float64(x) * np.float64(cc))
                u = np.int64(np.asarray(w0, F32).view(np.int32))
                k = np.arange(-64, 65, dtype=np.int64)
                bits = (u + k) if w0 >= 0 else (u - k)
                wv = bits.astype(np.int32).view(F32)
                wv = wv[np.isfinite(wv) & (np.abs(wv) <= cc)]
                parts_w.append(wv)
                parts_c.append(np.full(wv.shape, cc, dtype=F32))
    # denormal constants and weights, and huge constants
    cd = np.array([2.0 ** -149, 3 * 2.0 ** -149, 2.0 ** -140, 2.0 ** -127, 1.5 * 2.0 ** -126,
                   2.0 ** 100, 3.0e38], dtype=F32)
    for cc in cd:
        wv = (rng.uniform(-1, 1, 2000) * np.float64(cc)).astype(F32)
        wv = np.concatenate([wv, [cc, -cc, F32(0.0)]]).astype(F32)
        parts_w.append(wv)
        parts_c.append(np.full(wv.shape, cc, dtype=F32))
    return np.concatenate(parts_w).astype(F32), np.concatenate(parts_c).astype(F32)


def test_markstein_quotient_equals_ieee_division():
    """r = RN32(w / c) bit for bit wherever the quotient is at least 2^-120.
    Below that the residual w - q0 c can itself fall under the normal range
    and round, so r may be one ulp off; the code is then still the IEEE
    quotient's (next test), since every decision threshold is either 0 or at
    least 0.04 in magnitude."""
    w, c = _quotient_cases()
    r, _ = _markstein_quotient(w, c)
    ref = (w / c).astype(F32)
    big = np.abs(ref) >= F32(2.0 ** -120)
    diff = (r.view(np.uint32) != ref.view(np.uint32)) & big
    assert not diff.any(), f"{int(diff.sum())} quotients differ, e.g. w={w[diff][:3]} c={c[diff][:3]}"
    assert big.sum() > 0.9 * big.size


def _kernel_code(w, c, qt):
    """The quantiser's code of w in a block with constant c (c > 0): the
    Markstein quotient, for the evenly spaced codebook the sign-and-size
    decision where the scaled w is below the normal range, then the bins."""
    thr = _float_array("kNF4Thr" if qt == "nf4" else "kINT4Thr")
    base, t = _bins(thr)
    r, wm = _markstein_quotient(w, c)
    if qt == "int4":
        tinyw = np.abs(wm) < F32(2.0 ** -126)
        with np.errstate(over="ignore"):
            nz = np.ldexp(np.abs(w), 150).astype(F32) > c
        sub = np.copysign(np.where(nz, F32(2.0 ** -149), F32(0.0)), w).astype(F32)
        r = np.where(tinyw, sub, r).astype(F32)
    return _code_of(r, base, t)


@pytest.mark.parametrize("qt", ["nf4", "int4"])
def test_quotient_codes_equal_ieee_codes_everywhere(qt):
    w, c = _quotient_cases()
    ref = (w / c).astype(F32)
    mids = O.nf4_midpoints(O.levels_for(qt))
    want = np.zeros(w.shape, dtype=np.int64)
    for m in mids:
        want += ref.astype(np.float64) > m
    got = _kernel_code(w, c, qt)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, f"{bad.size} codes differ, e.g. w={w[bad[:3]]} c={c[bad[:3]]}"


def test_quantizer_codes_equal_oracle_codes():
    """The whole per-element path (quotient + bins) against the oracle's
    nf4_encode on blocks built around the thresholds."""
    rng = np.random.default_rng(3)
    thr = _float_array("kNF4Thr")
    blocks = []
    for k in range(4000):
        c = F32(abs(rng.standard_normal()) * 2.0 ** rng.integers(-20, 10) + 1e-30)
        x = thr[rng.integers(0, 15, 63)].astype(np.float64) * np.float64(c)
        u = np.asarray(x.astype(F32), F32).view(np.int32).astype(np.int64)
        step = rng.integers(-3, 4, 63)
        wv = np.where(x >= 0, u + step, u - step).astype(np.int32).view(F32)
        wv = np.clip(wv, -c, c).astype(F32)
        blocks.append(np.concatenate([[c], wv]).astype(F32))
    w = np.stack(blocks)
    cabs = O.block_absmax(w)
    ref = O.nf4_encode(w, cabs).reshape(w.shape)
    got = _kernel_code(w.reshape(-1), np.repeat(cabs, 64), "nf4").reshape(w.shape)
    assert np.array_equal(got, ref)


# --------------------------------------------------------------------------
# the corrected square root (adamw.hip, sqrt_rn)
# --------------------------------------------------------------------------
def _sqrt_rn_model(x, s):
    """The kernel's correction from an estimate s of sqrt(x): sd, su = s's
    neighbours; r = sd if RN32(x - sd s) <= 0, then r = su if RN32(x - su s)
    > 0 (signs of the exact residuals); inputs below 2^-96 are scaled by 2^32
    before and the root by 2^-16 after."""
    tiny = x < F32(2.0 ** -96)
    with np.errstate(over="ignore"):
        xs = np.where(tiny, (x * F32(2.0 ** 32)).astype(F32), x)
    sd = (s.view(np.uint32) - np.uint32(1)).view(F32)
    su = (s.view(np.uint32) + np.uint32(1)).view(F32)
    r = np.where(fma32(-sd, s, xs) <= 0, sd, s)
    r = np.where(fma32(-su, s, xs) > 0, su, r)
    r = np.where(tiny, (r * F32(2.0 ** -16)).astype(F32), r)
    return np.where(xs == 0, xs, r).astype(F32)


def test_sqrt_correction_from_every_estimate_within_one_ulp():
    rng = np.random.default_rng(4)
    parts = [rng.uniform(0, 4, 200_000).astype(F32),
             (rng.uniform(1, 2, 200_000) * 2.0 ** rng.integers(-149, 127, 200_000)).astype(F32)]
    # every float32 in windows around powers of 4 and 2 (binade changes of
    # the root), the smallest denormals and the 2^-96 scaling switch
    for e in (-148, -140, -126, -100, -96, -95, -50, -2, 0, 1, 2, 3, 50, 126):
        u = np.asarray(F32(2.0 ** e), F32).view(np.int32)
        parts.append(np.arange(max(u - 4096, 1), u + 4096, dtype=np.int32).view(F32))
    parts.append(np.arange(1, 8192, dtype=np.int32).view(F32))
    x = np.concatenate(parts).astype(F32)
    x = x[np.isfinite(x) & (x >= 0)]
    exact = np.sqrt(x.astype(np.float64)).astype(F32)      # correctly rounded (53 >= 2*24+2)
    tiny = x < F32(2.0 ** -96)
    with np.errstate(over="ignore"):
        xs = np.where(tiny, (x * F32(2.0 ** 32)).astype(F32), x)
    root_s = np.sqrt(xs.astype(np.float64)).astype(F32)     # rounded root of the scaled input
    for k in (-1, 0, 1):                                    # every estimate within one ulp
        s = (root_s.view(np.int32) + np.int32(k)).view(F32)
        s = np.where(xs == 0, F32(0.0), s).astype(F32)
        got = _sqrt_rn_model(x, s)
        bad = got.view(np.uint32) != exact.view(np.uint32)
        assert not bad.any(), f"estimate offset {k}: {int(bad.sum())} roots differ, e.g. {x[bad][:3]}"


# --------------------------------------------------------------------------
# double quantisation: the rounding order of the oracle, pinned by hand
# --------------------------------------------------------------------------
def test_double_quant_rounding_order_hand_derived():
    """A group whose 8-bit code depends on the rounding order of t = d / s2.

    Constants +-s2, +-d and 252 zeros: the mean is exactly 0, so d_b = c_b and
    s2 = max |d_b|.  With s2 = 0x1.4e6a96p-1 and d = 0x1.b6ebe6p-15 the exact
    d / s2 * 256 lies 8.02e-10 above 0.0205078125, the midpoint of the E4M3
    values 0x0A (0.01953125) and 0x0B (0.021484375); float32 quotients there
    are 2^-37 apart and the offset / 256 = 3.1e-12 is below half of that, so
    RN32(d / s2) * 256 is exactly the midpoint and rounds to the even 0x0A.
    Kept in float64, t would round up to 0x0B; through the float32
    reciprocal, d * RN32(1 / s2) lands one float32 above the midpoint, 0x0B
    as well.  The bytes below are therefore only reached with the oracle's
    order (an IEEE float32 quotient, then the E4M3 rounding)."""
    s2 = F32(float.fromhex("0x1.4e6a96p-1"))
    d = F32(float.fromhex("0x1.b6ebe6p-15"))
    assert abs(float(s2) - 0.6531569361686707) < 1e-15
    c = np.zeros(256, dtype=F32)
    c[:4] = [s2, -s2, d, -d]
    code8, s2_out, mu = O.double_quantize(c)
    assert mu == F32(0.0)
    assert s2_out.view(np.uint32)[0] == np.asarray(s2, F32).view(np.uint32)
    assert code8[:4].tolist() == [0x78, 0xF8, 0x0A, 0x8A]
    assert np.all(code8[4:] == 0x00)
    # the two other orders give 0x0B here (the case separates them)
    via_recip = F32(d * F32(F32(1.0) / s2)) * F32(256.0)
    assert O.e4m3_encode_rne(np.array([via_recip], F32))[0] == 0x0B
    t64 = np.float64(d) / np.float64(s2) * 256.0
    assert t64 > 0.0205078125 and O.e4m3_value(0x0B) - t64 < t64 - O.e4m3_value(0x0A)
