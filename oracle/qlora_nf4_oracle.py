"""CPU oracle for the frozen-NF4 linear layer with a LoRA adapter.

TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only the test suite, the smoke check
in ``__graft_entry__`` and the ``cpu_baseline`` leg of ``bench.py`` may import
this module.  It shares no code, table or constant with the HIP library: the
NF4 levels, the decision thresholds, the 8-bit float codec and the bf16
rounding are all derived here from their definitions.

Everything is plain NumPy.  Floating-point steps whose rounding is part of the
method (the codes and the dequantised weights must match bit for bit) are done
in float32 exactly as the step states it; the matrix products of the forward
and backward pass are done in float64 on the exact values of the bf16 inputs.

Sources (titles of the pages this follows; sections named in each function):
  [PL]  "QLoRA — 650億パラメータのモデルをGPU 1枚で微調整する" (ta-paperlens)
  [WZ]  LLM book, chapter 26 "LoRA/QLoRA" (waylandz.com)
  [HF]  "Hugging Face 4ビット量子化とQLoRAリリース" (agentlenshq)
  [UL]  Ultralytics glossary "QLoRA" (German edition)

Readings where the pages are silent (each is listed in the design doc):
  * blocks are 64 consecutive elements of the row-major [rows, cols] weight;
  * the code is the nearest level to RN32(w / c) in exact arithmetic, ties to
    the lower index; an all-zero block gets code 7 (the level 0);
  * two codes per byte, element 2i in the low nibble;
  * double quantisation: one mean mu per tensor (fixed float64 pairwise tree),
    d = RN32(c - mu), s2 = max |d| per group of 256 blocks, code8 = OCP E4M3
    round-to-nearest-even of RN32(d / s2) * 256;
  * dequantisation: c' = RN32(RN32(e4m3(code8) * 2^-8 * s2) + mu),
    w_hat = bf16_RNE(RN32(q[code] * c'));
  * lora_dropout acts on the adapter's input only, with keep decisions from
    Philox-4x32-10 (Salmon, Moraes, Dror, Shaw, SC11) as dropout_keep_mask
    states, and inverted scaling 1 / (1 - p).
"""

from __future__ import annotations

import numpy as np
from scipy.special import ndtri

BLOCK = 64          # weights per absmax block   [PL] 量子化を1段落で
DQ_GROUP = 256      # block constants per second-level constant   [PL] 二重量子化
NF4_ZERO_CODE = 7   # index of the exact 0 level

F32 = np.float32
F64 = np.float64


# --------------------------------------------------------------------------
# NF4 codebook
# --------------------------------------------------------------------------
def nf4_levels() -> np.ndarray:
    """The 16 NF4 levels as float32, ascending.

    [UL] code example under "So funktioniert QLoRA": eight positive levels are
    the standard-normal quantiles at 8 evenly spaced probabilities from
    0.9677083 toward 0.5 (0.5 excluded), seven negative levels are the negated
    quantiles at 7 evenly spaced probabilities over the same range, an exact 0
    is added, and the sorted set is divided by its largest value.  [PL] NF4
    section: dense near zero, an exact zero, endpoints exactly -1 and +1.
    Evaluated in float64, rounded once to float32.
    """
    p_pos = np.linspace(0.9677083, 0.5, 9)[:-1]
    p_neg = np.linspace(0.9677083, 0.5, 8)[:-1]
    levels = np.concatenate([-ndtri(p_neg), [0.0], ndtri(p_pos)])
    levels = np.sort(levels)
    levels = levels / levels.max()
    return levels.astype(F32)


def int4_levels() -> np.ndarray:
    """The 16 evenly spaced 4-bit levels -1 + 2i/15 (i = 0 .. 15) as float32.

    [UL] code example under "So funktioniert QLoRA": the comparison codebook
    of 16 evenly spaced levels from -1 to 1 (no exact zero).  Each level is
    the exact rational rounded once to float32.
    """
    from fractions import Fraction
    return np.array([float(Fraction(2 * i - 15, 15)) for i in range(16)], dtype=F64).astype(F32)


def levels_for(quant_type: str) -> np.ndarray:
    """Codebook of a quantisation type: "nf4" or "int4" (evenly spaced)."""
    if quant_type == "nf4":
        return nf4_levels()
    if quant_type == "int4":
        return int4_levels()
    raise ValueError(f"unknown quantisation type {quant_type!r}")


def nf4_midpoints(levels: np.ndarray | None = None) -> np.ndarray:
    """Exact midpoints between neighbouring levels, float64 (15 values).

    The sum of two float32 numbers of similar magnitude and the halving are
    exact in float64, so these are the real-number decision boundaries of the
    nearest-level rule ([PL] 量子化を1段落で: store the index of the nearest level).
    """
    q = (nf4_levels() if levels is None else levels).astype(F64)
    return (q[:-1] + q[1:]) / 2.0


# --------------------------------------------------------------------------
# (a1) block absmax, (a2) nearest-level encode and packing
# --------------------------------------------------------------------------
def block_absmax(w: np.ndarray) -> np.ndarray:
    """c_b = max |w_i| over each block of 64 consecutive row-major elements.

    [PL] 量子化を1段落で (one high-precision constant per block of 64, the
    largest absolute value in the block); [UL] code example (one scale per row
    of 64).  Returns float32 [n / 64].
    """
    w = np.asarray(w, dtype=F32).reshape(-1, BLOCK)
    return np.abs(w).max(axis=1)


def nf4_encode(w: np.ndarray, c: np.ndarray, levels: np.ndarray | None = None,
               chunk_blocks: int = 1 << 16) -> np.ndarray:
    """NF4 code of every element, uint8 in [0, 15], one per element.

    [PL] 量子化を1段落で: each value is stored as the index of the level nearest
    to w / c.  The quotient is the float32 IEEE quotient RN32(w / c); the code
    is the number of exact midpoints strictly below it, i.e. the nearest level
    with ties going to the lower index.  A block whose constant is 0 holds
    only zeros and gets the zero level.  Rows are processed in chunks only to
    bound memory; every element is independent.
    """
    w = np.asarray(w, dtype=F32).reshape(-1, BLOCK)
    c = np.asarray(c, dtype=F32).reshape(-1)
    mids = nf4_midpoints(levels)
    codes = np.empty(w.shape, dtype=np.uint8)
    for s in range(0, w.shape[0], chunk_blocks):
        wb = w[s:s + chunk_blocks]
        cb = c[s:s + chunk_blocks]
        zero = cb == 0
        safe_c = np.where(zero, F32(1.0), cb).astype(F32)
        r = (wb / safe_c[:, None]).astype(F32)        # float32 IEEE division
        r64 = r.astype(F64)
        code = np.zeros(r.shape, dtype=np.uint8)
        for m in mids:
            code += (r64 > F64(m))
        code[zero] = NF4_ZERO_CODE
        codes[s:s + chunk_blocks] = code
    return codes.reshape(-1)


def pack_nibbles(codes: np.ndarray) -> np.ndarray:
    """Two 4-bit codes per byte, element 2i in the low nibble.

    [WZ] 26.6.3: NF4 is kept as 4-bit integers, half a byte per weight.  The
    order inside the byte is not given on the pages.
    """
    codes = np.asarray(codes, dtype=np.uint8).reshape(-1)
    assert codes.size % 2 == 0
    return (codes[0::2] | (codes[1::2] << 4)).astype(np.uint8)


def unpack_nibbles(packed: np.ndarray) -> np.ndarray:
    packed = np.asarray(packed, dtype=np.uint8).reshape(-1)
    out = np.empty(packed.size * 2, dtype=np.uint8)
    out[0::2] = packed & 0x0F
    out[1::2] = packed >> 4
    return out


# --------------------------------------------------------------------------
# (a3) mean of the block constants, (a4) 8-bit float codes per group of 256
# --------------------------------------------------------------------------
def pairwise_tree_sum(x: np.ndarray) -> float:
    """Perfect binary tree of float64 additions over x in index order.

    The input is zero-padded to the next power of two; level by level,
    element 2j and element 2j+1 are added.  Fixes the rounding order of the
    mean so that it is reproducible.
    """
    v = np.asarray(x, dtype=F64).reshape(-1)
    if v.size == 0:
        return 0.0
    size = 1
    while size < v.size:
        size *= 2
    v = np.concatenate([v, np.zeros(size - v.size, dtype=F64)])
    while v.size > 1:
        v = v[0::2] + v[1::2]
    return float(v[0])


def dq_mean(c: np.ndarray) -> np.float32:
    """mu = RN32(RN64(S / n_b)), S the pairwise tree sum of all constants.

    [PL] 二重量子化, last paragraph: the constants are all positive, so their
    mean is subtracted before they are quantised to a symmetric 8-bit float.
    One mean per tensor (the pages do not say per what).
    """
    c = np.asarray(c, dtype=F32).reshape(-1)
    s = pairwise_tree_sum(c)
    return F32(F64(s) / F64(c.size))


def e4m3_value(code: int) -> float:
    """Real value of an OCP FP8 E4M3 bit pattern (float64, exact); NaN for 0x7F/0xFF.

    Format: 1 sign bit, 4 exponent bits with bias 7, 3 fraction bits; exponent
    field 0 is subnormal (fraction * 2^-9); 0x7F and 0xFF are NaN; no infinity.
    """
    code = int(code) & 0xFF
    sign = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0x0F
    m = code & 0x07
    if e == 0x0F and m == 0x07:
        return float("nan")
    if e == 0:
        return sign * m * 2.0 ** -9
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


# the 127 finite non-negative E4M3 values, in code order (which is value order)
_E4M3_POS = np.array([e4m3_value(k) for k in range(0x7F)], dtype=F64)


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    """Vector decode of E4M3 bit patterns to float64 (exact)."""
    table = np.array([e4m3_value(k) for k in range(256)], dtype=F64)
    return table[np.asarray(codes, dtype=np.uint8)]


def e4m3_encode_rne(x: np.ndarray) -> np.ndarray:
    """E4M3 bit pattern nearest to each float32 x, ties to the even pattern.

    The nearest finite E4M3 magnitude is found among all 127 of them; on an
    exact tie the pattern with an even last bit wins (round to nearest even).
    The sign bit is copied, so -0 and tiny negatives give 0x80.  Inputs must
    satisfy |x| <= 448 (no saturation or NaN handling is needed here).
    """
    x = np.asarray(x, dtype=F32)
    a = np.abs(x).astype(F64)
    assert np.all(a <= 448.0), "E4M3 encode: |x| > 448 is out of range"
    hi = np.searchsorted(_E4M3_POS, a, side="left")      # first value >= a
    hi = np.minimum(hi, _E4M3_POS.size - 1)
    lo = np.maximum(hi - 1, 0)
    d_lo = a - _E4M3_POS[lo]
    d_hi = _E4M3_POS[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    mag = np.where(pick_hi, hi, lo)
    mag = np.where(_E4M3_POS[hi] == a, hi, mag)
    sign = np.signbit(x).astype(np.int64) << 7
    return (mag | sign).astype(np.uint8)


def double_quantize(c: np.ndarray):
    """Second-level quantisation of the float32 block constants.

    [PL] 二重量子化: the float32 constants are taken in groups of 256, stored as
    8-bit floats, with one float32 second-level constant per group, after the
    mean has been subtracted.  [UL] "Doppelte Quantisierung": 8 bits per block
    constant in blocks of 256.

    Returns (code8 uint8 [n_b], s2 float32 [n_g], mu float32).
    """
    c = np.asarray(c, dtype=F32).reshape(-1)
    n_b = c.size
    mu = dq_mean(c)
    d = (c - mu).astype(F32)                        # RN32(c - mu)
    n_g = (n_b + DQ_GROUP - 1) // DQ_GROUP
    s2 = np.zeros(n_g, dtype=F32)
    code8 = np.zeros(n_b, dtype=np.uint8)
    for g in range(n_g):
        dg = d[g * DQ_GROUP:(g + 1) * DQ_GROUP]
        s = np.abs(dg).max()
        s2[g] = s
        if s == 0:
            code8[g * DQ_GROUP:(g + 1) * DQ_GROUP] = 0x00
            continue
        t = (dg / s).astype(F32)                    # RN32(d / s2), in [-1, 1]
        code8[g * DQ_GROUP:(g + 1) * DQ_GROUP] = e4m3_encode_rne(t * F32(256.0))
    return code8, s2, mu


def block_constants_from_dq(code8: np.ndarray, s2: np.ndarray, mu) -> np.ndarray:
    """c'_b = RN32(RN32(e4m3(code8_b) * 2^-8 * s2_g) + mu), float32 [n_b].

    Inverse of double_quantize: e4m3 * 2^-8 is exact in float32; the product
    with s2 and the sum with mu are each rounded once (no fused multiply-add).
    """
    code8 = np.asarray(code8, dtype=np.uint8).reshape(-1)
    s2 = np.asarray(s2, dtype=F32).reshape(-1)
    g = np.arange(code8.size) // DQ_GROUP
    scaled = (e4m3_decode(code8) * 2.0 ** -8).astype(F32)
    prod = (scaled * s2[g]).astype(F32)
    return (prod + F32(mu)).astype(F32)


# --------------------------------------------------------------------------
# bf16 round to nearest even
# --------------------------------------------------------------------------
def bf16_bits_rne(x: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) nearest to each finite float32, ties to even.

    bf16 keeps the upper 16 bits of the float32 pattern; the discarded lower
    half decides: above half goes up, below goes down, exactly half goes to
    the pattern whose last kept bit is 0.
    """
    u = np.asarray(x, dtype=F32).view(np.uint32)
    keep = u >> np.uint32(16)
    rest = u & np.uint32(0xFFFF)
    up = (rest > 0x8000) | ((rest == 0x8000) & ((keep & 1) == 1))
    return (keep + up.astype(np.uint32)).astype(np.uint16)


def f16_bits_rne(x: np.ndarray) -> np.ndarray:
    """IEEE binary16 bit patterns of float32 values, round to nearest even
    (subnormals kept, overflow to infinity): NumPy's float16 conversion.
    The compute type of older GPUs ([PL] 落とし穴: compute_dtype FP16 where
    BF16 is missing; [WZ] 26.6.4 uses float16)."""
    with np.errstate(over="ignore"):
        return np.asarray(x, dtype=F32).astype(np.float16).view(np.uint16)


def f16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """float32 value of binary16 bit patterns (exact widening)."""
    return np.asarray(b, dtype=np.uint16).view(np.float16).astype(F32)


def round16_bits(x: np.ndarray, compute_dtype: str) -> np.ndarray:
    """Bit patterns of float32 values rounded to the 16-bit compute type."""
    if compute_dtype == "bf16":
        return bf16_bits_rne(x)
    if compute_dtype == "fp16":
        return f16_bits_rne(x)
    raise ValueError(f"unknown compute dtype {compute_dtype!r}")


def bits16_to_f32(b: np.ndarray, compute_dtype: str) -> np.ndarray:
    """float32 values of 16-bit patterns of the compute type."""
    return bf16_bits_to_f32(b) if compute_dtype == "bf16" else f16_bits_to_f32(b)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(F32)


# --------------------------------------------------------------------------
# (a1-a5) quantise and dequantise a weight
# --------------------------------------------------------------------------
def quantize(w: np.ndarray, quant_type: str = "nf4", double_quant: bool = True) -> dict:
    """Blockwise 4-bit quantisation of a float32 [rows, cols] weight.

    The codes are taken against the original float32 block constants; with
    double quantisation the 8-bit constant codes are what is stored ([PL]
    order of presentation: blockwise NF4 first, then the constants are
    quantised).  Without it ([PL] 二重量子化, the 4.5-bit count: one float32
    constant per 64 weights) absmax_scale holds the float32 constants.
    quant_type "nf4" or "int4" (the evenly spaced comparison codebook).
    """
    w = np.asarray(w, dtype=F32)
    rows, cols = w.shape
    assert cols % BLOCK == 0, "cols must be a multiple of 64"
    c = block_absmax(w)
    codes = nf4_encode(w, c, levels=levels_for(quant_type))
    st = {"rows": rows, "cols": cols, "quant_type": quant_type, "double_quant": double_quant,
          "codes": pack_nibbles(codes), "absmax_fp32": c}
    if double_quant:
        code8, s2, mu = double_quantize(c)
        st.update(absmax_code=code8, absmax_scale=s2, absmax_offset=np.array([mu], dtype=F32))
    else:
        st.update(absmax_scale=c.copy())
    return st


def block_constants(state: dict) -> np.ndarray:
    """The constants the dequantiser multiplies by: c' from the 8-bit codes
    (double quantisation) or the stored float32 c."""
    if state.get("double_quant", True):
        return block_constants_from_dq(state["absmax_code"], state["absmax_scale"],
                                       state["absmax_offset"][0])
    return np.asarray(state["absmax_scale"], dtype=F32)


def dequantize_bits(state: dict, compute_dtype: str = "bf16") -> np.ndarray:
    """16-bit patterns of the dequantised weight, uint16 [rows, cols].

    [PL] 量子化を1段落で: restore by table lookup and multiply, x_hat = c * q[index];
    [PL] 勾配は実際どこへ行くのか: the storage type is NF4, compute is bf16
    (fp16 where bf16 is missing, [PL] 落とし穴).
    """
    rows, cols = state["rows"], state["cols"]
    codes = unpack_nibbles(state["codes"]).reshape(-1, BLOCK)
    return _decode_bits(codes, block_constants(state), state.get("quant_type", "nf4"),
                        compute_dtype).reshape(rows, cols)


def _decode_bits(codes: np.ndarray, cprime: np.ndarray, quant_type: str = "nf4",
                 compute_dtype: str = "bf16") -> np.ndarray:
    """round16(RN32(q[code] * c')) for codes [n_blocks, 64] and c' [n_blocks]."""
    q = levels_for(quant_type)
    prod = (q[codes] * np.asarray(cprime, dtype=F32)[:, None]).astype(F32)
    return round16_bits(prod, compute_dtype)


def _constants_state(c: np.ndarray, quant_type: str, double_quant: bool) -> dict:
    """The stored constants of quantize() for block constants c."""
    st = {"quant_type": quant_type, "double_quant": double_quant}
    if double_quant:
        code8, s2, mu = double_quantize(c)
        st.update(absmax_code=code8, absmax_scale=s2, absmax_offset=np.array([mu], dtype=F32))
    else:
        st.update(absmax_scale=np.asarray(c, dtype=F32).copy())
    return st


def quantize_sampled_rows(w: np.ndarray, sel, quant_type: str = "nf4",
                          double_quant: bool = True) -> dict:
    """quantize() of the whole weight, keeping the NF4 codes of rows `sel` only.

    The block constants and their double quantisation cover every block (they
    are exactly quantize()'s); only the per-element encode is restricted.
    Meant for sampled checks of weights too large for a full CPU encode.
    The packed codes are [len(sel), cols // 2]; 'sel' is kept in the state.
    """
    w = np.asarray(w, dtype=F32)
    rows, cols = w.shape
    assert cols % BLOCK == 0, "cols must be a multiple of 64"
    sel = np.asarray(sel, dtype=np.int64).reshape(-1)
    kb = cols // BLOCK
    c = block_absmax(w)
    codes = nf4_encode(w[sel], c.reshape(rows, kb)[sel], levels=levels_for(quant_type))
    st = {"rows": rows, "cols": cols, "sel": sel,
          "codes": pack_nibbles(codes).reshape(sel.size, cols // 2)}
    st.update(_constants_state(c, quant_type, double_quant))
    return st


def dequantize_sampled_bits(state: dict, compute_dtype: str = "bf16") -> np.ndarray:
    """dequantize_bits() restricted to the rows of a quantize_sampled_rows()
    state: uint16 [len(sel), cols]."""
    rows, cols, sel = state["rows"], state["cols"], state["sel"]
    kb = cols // BLOCK
    cprime = block_constants(state).reshape(rows, kb)[sel]
    codes = unpack_nibbles(state["codes"]).reshape(-1, BLOCK)
    return _decode_bits(codes, cprime.reshape(-1), state.get("quant_type", "nf4"),
                        compute_dtype).reshape(sel.size, cols)


def quantize_sampled_cols(w: np.ndarray, sel, quant_type: str = "nf4",
                          double_quant: bool = True) -> dict:
    """quantize() of the whole weight, keeping the NF4 codes of the 64-wide
    blocks that contain columns `sel` (every row).  The constants and their
    double quantisation cover every block, exactly as quantize()'s.
    """
    w = np.asarray(w, dtype=F32)
    rows, cols = w.shape
    assert cols % BLOCK == 0, "cols must be a multiple of 64"
    sel = np.asarray(sel, dtype=np.int64).reshape(-1)
    kb = cols // BLOCK
    c = block_absmax(w)
    bsel = np.unique(sel // BLOCK)
    wb = w.reshape(rows, kb, BLOCK)[:, bsel, :]
    cb = c.reshape(rows, kb)[:, bsel]
    codes = nf4_encode(wb.reshape(-1, BLOCK), cb.reshape(-1), levels=levels_for(quant_type))
    st = {"rows": rows, "cols": cols, "sel": sel, "block_cols": bsel,
          "codes": pack_nibbles(codes)}
    st.update(_constants_state(c, quant_type, double_quant))
    return st


def dequantize_sampled_cols_bits(state: dict, compute_dtype: str = "bf16") -> np.ndarray:
    """dequantize_bits() restricted to the columns of a quantize_sampled_cols()
    state: uint16 [rows, len(sel)]."""
    rows, cols, sel, bsel = state["rows"], state["cols"], state["sel"], state["block_cols"]
    kb = cols // BLOCK
    cprime = block_constants(state).reshape(rows, kb)[:, bsel]
    codes = unpack_nibbles(state["codes"]).reshape(-1, BLOCK)
    bits = _decode_bits(codes, cprime.reshape(-1), state.get("quant_type", "nf4"),
                        compute_dtype).reshape(rows, bsel.size * BLOCK)
    pos = np.searchsorted(bsel, sel // BLOCK) * BLOCK + sel % BLOCK
    return bits[:, pos]


def dequantize(state: dict, compute_dtype: str = "bf16") -> np.ndarray:
    """Dequantised weight as float64 values of the 16-bit results."""
    return bits16_to_f32(dequantize_bits(state, compute_dtype), compute_dtype).astype(F64)


def storage_bits_per_param(rows: int, cols: int, double_quant: bool = True) -> float:
    """Bytes of the packed state * 8 / number of weights.

    [PL] 二重量子化: 4 bits per code, 8 bits per 64 weights, 32 bits per
    64*256 weights; plus one float32 mean per tensor (the reading taken
    here).  Without double quantisation: 4 bits per code and one float32
    per 64 weights, the page's 4.5 bits.
    """
    n = rows * cols
    n_b = n // BLOCK
    n_g = (n_b + DQ_GROUP - 1) // DQ_GROUP
    nbytes = n // 2 + (n_b + 4 * n_g + 4 if double_quant else 4 * n_b)
    return nbytes * 8.0 / n


# --------------------------------------------------------------------------
# Merge of the adapter into the dequantised base (deployment step)
# --------------------------------------------------------------------------
def merge_values_f32(w_hat_bits: np.ndarray, a: np.ndarray, b: np.ndarray, alpha: float,
                     r: int, compute_dtype: str = "bf16") -> np.ndarray:
    """float32 sum RN32(w_hat + RN32(s * RN32(B A))) before the final rounding.

    [WZ] 26.2 (inference: merge once, W_merged = W + (alpha/r) B A); [PL]
    落とし穴 and [UL] Kompromisse: the merge happens on the base dequantised
    to 16 bit.  Reading: the 16-bit base is the bf16 dequantised weight
    (w_hat_bits, uint16 [rows, cols]); B A is formed exactly (float64 of the
    bf16 values of B [rows, r] and A [r, cols]) and rounded once to float32;
    s = RN32(alpha / r) multiplies in float32; the sum with the base is one
    float32 addition.
    """
    base = bits16_to_f32(w_hat_bits, compute_dtype)
    s = np.float32(np.float32(alpha) / np.float32(r))
    ba = (np.asarray(b, dtype=F64) @ np.asarray(a, dtype=F64)).astype(np.float32)
    return (base + (s * ba).astype(np.float32)).astype(np.float32)


def merge_bits(w_hat_bits: np.ndarray, a: np.ndarray, b: np.ndarray, alpha: float,
               r: int, compute_dtype: str = "bf16") -> np.ndarray:
    """16-bit patterns of the merged weight: merge_values_f32 rounded to the
    compute type (bf16 or fp16, nearest even).

    [PL] 落とし穴: merge on the 16-bit base and, if wanted, quantise the
    result again (that is quantize() of these values as float32).
    """
    return round16_bits(merge_values_f32(w_hat_bits, a, b, alpha, r, compute_dtype),
                        compute_dtype)


# --------------------------------------------------------------------------
# Adapter optimizer step (AdamW, 32-bit states)
# --------------------------------------------------------------------------
def power_by_squaring(x: float, t: int) -> float:
    """x^t for an integer t >= 0 by binary exponentiation in float64, a fixed
    sequence of IEEE multiplications (the library computes the same)."""
    r, b = 1.0, float(x)
    while t:
        if t & 1:
            r *= b
        b *= b
        t >>= 1
    return r


def adamw_scalars(step: int, lr: float, beta1: float, beta2: float, eps: float,
                  weight_decay: float) -> dict:
    """float32 constants of step `step` (1-based), each one rounding of a
    float64 value computed from the float64 hyperparameters: the decay
    factor 1 - lr*wd, beta1, 1 - beta1, beta2, 1 - beta2, the step size
    lr / (1 - beta1^step), sqrt(1 - beta2^step) and eps."""
    f = np.float32
    lr, b1, b2, wd, e = F64(lr), F64(beta1), F64(beta2), F64(weight_decay), F64(eps)
    return {
        "decay": f(1.0 - lr * wd),
        "b1": f(b1), "omb1": f(1.0 - b1),
        "b2": f(b2), "omb2": f(1.0 - b2),
        "step_size": f(lr / (1.0 - power_by_squaring(b1, step))),
        "bc2_sqrt": f(np.sqrt(1.0 - power_by_squaring(b2, step))),
        "eps": f(e),
    }


def adamw_step(param, exp_avg, exp_avg_sq, grad, step: int, lr: float, beta1: float,
               beta2: float, eps: float, weight_decay: float, copy_dtype: str = "bf16"):
    """One AdamW step on float32 arrays; returns (param, exp_avg, exp_avg_sq,
    the 16-bit copy's bit patterns: bf16, or fp16 for fp16 compute).

    [PL] ページ化オプティマイザ and page 2 26.6.4 (paged_adamw_32bit: Adam's two
    moments per trainable parameter, kept in 32 bit; only the adapters A, B
    have them).  The update is Adam with decoupled weight decay (Loshchilov &
    Hutter) and bias-corrected moments, in the form PyTorch's AdamW documents.
    Reading: float32 master parameters and moments; with the constants of
    adamw_scalars, every operation one IEEE float32 rounding in this order,
    no fused multiply-add:
      p1 = p * decay;  m1 = b1 m + (1-b1) g;  v1 = b2 v + (1-b2) (g g);
      den = sqrt(v1) / sqrt(bc2) + eps;  p2 = p1 - step_size (m1 / den);
    the 16-bit copy for the next forward is p2 rounded to nearest even.
    """
    k = adamw_scalars(step, lr, beta1, beta2, eps, weight_decay)
    f32 = np.float32
    p = np.asarray(param, f32)
    m = np.asarray(exp_avg, f32)
    v = np.asarray(exp_avg_sq, f32)
    g = np.asarray(grad, f32)
    p1 = (p * k["decay"]).astype(f32)
    m1 = ((k["b1"] * m).astype(f32) + (k["omb1"] * g).astype(f32)).astype(f32)
    gg = (g * g).astype(f32)
    v1 = ((k["b2"] * v).astype(f32) + (k["omb2"] * gg).astype(f32)).astype(f32)
    den = ((np.sqrt(v1).astype(f32) / k["bc2_sqrt"]).astype(f32) + k["eps"]).astype(f32)
    upd = (k["step_size"] * (m1 / den).astype(f32)).astype(f32)
    p2 = (p1 - upd).astype(f32)
    return p2, m1, v1, round16_bits(p2, copy_dtype)


# --------------------------------------------------------------------------
# (a6-a11) LoRA linear layer, forward and backward, float64
# --------------------------------------------------------------------------
def linear_forward(x: np.ndarray, w_hat: np.ndarray, a: np.ndarray, b: np.ndarray,
                   alpha: float, r: int):
    """Y = X W^T + (alpha/r) (X A^T) B^T, float64.

    [PL] 勾配は実際どこへ行くのか: h = dequant(W_NF4) x + B A x in bf16;
    [WZ] 26.2.4: the adapter term is scaled by alpha / r.  Rows of X are
    tokens, W is [out, in] like nn.Linear, A is [r, in], B is [out, r]
    ([WZ] 26.2.1 shapes).  Returns (Y, U) with U = X A^T.
    """
    x = np.asarray(x, dtype=F64)
    s = F64(alpha) / F64(r)
    u = x @ np.asarray(a, dtype=F64).T
    y = x @ np.asarray(w_hat, dtype=F64).T + s * (u @ np.asarray(b, dtype=F64).T)
    return y, u


def linear_backward(x: np.ndarray, dy: np.ndarray, w_hat: np.ndarray, a: np.ndarray,
                    b: np.ndarray, alpha: float, r: int):
    """Gradients of L = <dY, Y> for the layer above: dX, dA, dB; no dW.

    [PL] 勾配は実際どこへ行くのか: the input gradient passes through the
    dequantised W^T; only A and B receive gradients; W is never written.
      G  = dY B
      dX = dY W_hat + s G A
      dA = s G^T X
      dB = s dY^T (X A^T)
    """
    dx = linear_input_grad(dy, w_hat, a, b, alpha, r)
    da, db = lora_grads(x, dy, a, b, alpha, r)
    return dx, da, db


def linear_input_grad(dy: np.ndarray, w_hat: np.ndarray, a: np.ndarray, b: np.ndarray,
                      alpha: float, r: int) -> np.ndarray:
    """dX = dY W_hat + s (dY B) A (the dX part of linear_backward).  Columns of
    W_hat and A may be any subset of the input features: dX is then the same
    subset of its columns."""
    dy = np.asarray(dy, dtype=F64)
    s = F64(alpha) / F64(r)
    g = dy @ np.asarray(b, dtype=F64)
    return dy @ np.asarray(w_hat, dtype=F64) + s * (g @ np.asarray(a, dtype=F64))


def lora_grads(x: np.ndarray, dy: np.ndarray, a: np.ndarray, b: np.ndarray, alpha: float,
               r: int):
    """dA = s (dY B)^T X and dB = s dY^T (X A^T) (the adapter part of
    linear_backward; W does not enter)."""
    x = np.asarray(x, dtype=F64)
    dy = np.asarray(dy, dtype=F64)
    a = np.asarray(a, dtype=F64)
    s = F64(alpha) / F64(r)
    g = dy @ np.asarray(b, dtype=F64)
    da = s * (g.T @ x)
    db = s * (dy.T @ (x @ a.T))
    return da, db


# --------------------------------------------------------------------------
# lora_dropout: counter-based keep mask, and the layer with dropout
# --------------------------------------------------------------------------
PHILOX_M = (0xD2511F53, 0xCD9E8D57)   # round multipliers of Philox-4x32
PHILOX_W = (0x9E3779B9, 0xBB67AE85)   # key increments between rounds
_U32 = 0xFFFFFFFF


def philox4x32_10(counter, key):
    """Philox-4x32 with 10 rounds on one counter, in Python integers.

    Salmon, Moraes, Dror and Shaw, "Parallel Random Numbers: As Easy as 1, 2,
    3" (SC11), the Philox-4x32 bijection: a round forms the 64-bit products of
    counter words 0 and 2 with the two round multipliers; the new counter is
    (hi(M1 x2) ^ x1 ^ k0, lo(M1 x2), hi(M0 x0) ^ x3 ^ k1, lo(M0 x0)); the first
    round uses the key as given and each later round the key advanced by the
    two increments once more (all words modulo 2^32).
    """
    x0, x1, x2, x3 = (int(v) & _U32 for v in counter)
    k0, k1 = (int(v) & _U32 for v in key)
    for rnd in range(10):
        if rnd:
            k0 = (k0 + PHILOX_W[0]) & _U32
            k1 = (k1 + PHILOX_W[1]) & _U32
        p0 = PHILOX_M[0] * x0
        p1 = PHILOX_M[1] * x2
        x0, x1, x2, x3 = (p1 >> 32) ^ x1 ^ k0, p1 & _U32, (p0 >> 32) ^ x3 ^ k1, p0 & _U32
    return x0, x1, x2, x3


def philox4x32_10_array(c0, c1, c2, c3, key):
    """philox4x32_10 on arrays of counters (any integer arrays of 32-bit
    words, broadcast together) with one key; returns four uint64 arrays.
    The products of two 32-bit words fit uint64 exactly."""
    m = np.uint64(_U32)
    x0, x1, x2, x3 = np.broadcast_arrays(*(np.asarray(v).astype(np.uint64) & m
                                           for v in (c0, c1, c2, c3)))
    k0, k1 = (int(v) & _U32 for v in key)
    for rnd in range(10):
        if rnd:
            k0 = (k0 + PHILOX_W[0]) & _U32
            k1 = (k1 + PHILOX_W[1]) & _U32
        p0 = x0 * np.uint64(PHILOX_M[0])
        p1 = x2 * np.uint64(PHILOX_M[1])
        x0, x1, x2, x3 = ((p1 >> np.uint64(32)) ^ x1 ^ np.uint64(k0), p1 & m,
                          (p0 >> np.uint64(32)) ^ x3 ^ np.uint64(k1), p0 & m)
    return x0, x1, x2, x3


def dropout_threshold(p: float) -> int:
    """floor(p 2^32) for 0 <= p < 1: a random word below it drops its
    element, so an element is kept with probability 1 - floor(p 2^32) / 2^32."""
    p = F64(p)
    if not (0.0 <= p < 1.0):
        raise ValueError("dropout probability must lie in [0, 1)")
    return int(np.floor(p * F64(2.0 ** 32)))


def dropout_keep_mask(T: int, cols: int, p: float, seed: int, offset: int,
                      tokens=None, features=None) -> np.ndarray:
    """Keep mask (bool [T, cols]; [len(tokens), len(features)] for selected
    token and feature indices) of the adapter's input dropout.

    [PL] コードで見る and 現場ではこう使う, [WZ] 26.4.2 / 26.5.1 / 26.6.4: the
    adapter config sets lora_dropout (0.05 in every example); the pages
    define no random stream.  Reading: element (t, k) of X [T, cols] is kept
    iff word (t mod 4) of Philox-4x32-10 at counter (k, floor(t / 4),
    offset mod 2^32, floor(offset / 2^32)) with key (seed mod 2^32,
    floor(seed / 2^32)) is at least dropout_threshold(p).  The generator runs
    once per needed (t // 4, k).
    """
    thr = dropout_threshold(p)
    t = np.arange(T, dtype=np.int64) if tokens is None else np.asarray(tokens, dtype=np.int64)
    k = np.arange(cols, dtype=np.int64) if features is None else np.asarray(features, np.int64)
    quads, inv = np.unique(t >> 2, return_inverse=True)
    words = philox4x32_10_array(k[None, :], quads[:, None], offset & _U32,
                                (offset >> 32) & _U32, (seed & _U32, (seed >> 32) & _U32))
    w = np.stack(words)                                  # [4, quads, features]
    return w[t & 3, inv.reshape(-1)] >= np.uint64(thr)


def dropout_mask_bytes(keep: np.ndarray) -> np.ndarray:
    """The packed form of a keep mask [T, cols] (cols even): uint8
    [ceil(T/4), cols/2], the bit of element (t, k) is bit (t mod 4) of the
    low nibble (k even) or high nibble (k odd) of byte [t // 4, k // 2];
    bits of tokens past T are 0.  Four consecutive tokens of one feature
    share a nibble."""
    keep = np.asarray(keep, dtype=bool)
    T, cols = keep.shape
    quads = (T + 3) // 4
    full = np.zeros((quads * 4, cols), dtype=np.uint8)
    full[:T] = keep
    nib = np.zeros((quads, cols), dtype=np.uint8)
    for j in range(4):
        nib |= full[j::4] << j
    return (nib[:, 0::2] | (nib[:, 1::2] << 4)).astype(np.uint8)


def dropout_input(x: np.ndarray, keep: np.ndarray) -> np.ndarray:
    """The dropped adapter input before scaling: x where kept, +0 elsewhere
    (float64 of the bf16 values)."""
    return np.where(keep, np.asarray(x, dtype=F64), 0.0)


def linear_forward_dropout(x: np.ndarray, w_hat: np.ndarray, a: np.ndarray, b: np.ndarray,
                           alpha: float, r: int, keep: np.ndarray, p: float):
    """Y = X W^T + s (D(X) A^T) B^T with D(X) = keep * X / (1 - p), float64.

    Reading of lora_dropout (see dropout_keep_mask): dropout acts on the
    adapter's input only, the frozen path sees X unchanged, and kept elements
    are scaled by 1 / (1 - p) so the expectation is the undropped layer.
    Returns (Y, U) with U = D(X) A^T, the tensor the backward needs for dB.
    """
    x = np.asarray(x, dtype=F64)
    xd = dropout_input(x, keep) / (1.0 - F64(p))
    s = F64(alpha) / F64(r)
    u = xd @ np.asarray(a, dtype=F64).T
    y = x @ np.asarray(w_hat, dtype=F64).T + s * (u @ np.asarray(b, dtype=F64).T)
    return y, u


def linear_backward_dropout(x: np.ndarray, dy: np.ndarray, w_hat: np.ndarray, a: np.ndarray,
                            b: np.ndarray, alpha: float, r: int, keep: np.ndarray, p: float):
    """Gradients of L = <dY, Y> for linear_forward_dropout; no dW.
      G  = dY B
      dX = dY W_hat + keep * (s G A) / (1 - p)
      dA = s G^T D(X)
      dB = s dY^T (D(X) A^T)
    """
    dy = np.asarray(dy, dtype=F64)
    a = np.asarray(a, dtype=F64)
    s = F64(alpha) / F64(r)
    inv = 1.0 / (1.0 - F64(p))
    xd = dropout_input(x, keep) * inv
    g = dy @ np.asarray(b, dtype=F64)
    dx = dy @ np.asarray(w_hat, dtype=F64) + np.where(keep, s * (g @ a), 0.0) * inv
    da = s * (g.T @ xd)
    db = s * (dy.T @ (xd @ a.T))
    return dx, da, db


def lora_param_count(d: int, k: int, r: int) -> int:
    """Trainable numbers of one adapter, r (d + k).  [PL] 前提: LoRAの低ランク更新."""
    return r * (d + k)


def rel_frobenius(got: np.ndarray, ref: np.ndarray) -> float:
    """||got - ref||_F / ||ref||_F in float64."""
    got = np.asarray(got, dtype=F64)
    ref = np.asarray(ref, dtype=F64)
    den = np.linalg.norm(ref)
    num = np.linalg.norm(got - ref)
    return float(num / den) if den > 0 else float(num)
