"""GPU parity of the storage and compute variants against the oracle.

Quantise / dequantise / merge for both codebooks (NF4 and the evenly spaced
INT4 of the Ultralytics code example), with and without double
quantisation (ta-paperlens 二重量子化: 4.5 bits with float32 constants), in
bf16 and fp16 (ta-paperlens 落とし穴; waylandz 26.6.4): codes, constants and
dequantised weights bit for bit, merged weights within one 16-bit ulp and
>= 99% bit-identical.  The linear layer (NF4) with fp16 compute and / or
float32 constants, forward and backward, the skinny path and lora_dropout:
within the 5e-3 relative Frobenius bound of the float64 oracle."""
import dataclasses

import numpy as np
import pytest
import torch

import workloads as WL
from gpu_util import GEMM_TOL, bits_host, dev, f32_dev
from oracle import qlora_nf4_oracle as O

pytestmark = pytest.mark.gpu

FORMATS = [("nf4", True), ("nf4", False), ("int4", True), ("int4", False)]
DTYPES = ("bf16", "fp16")


def _q():
    import bit_nf4_quantized_06_amd as q
    return q


def _adversarial(rows=48, cols=320, seed=4):
    """Zero / -0 / denormal / huge blocks, zeros inside non-zero blocks (the
    INT4 zero tie), exact midpoints of both codebooks and their float32
    neighbours; n_b is not a multiple of 256."""
    rng = np.random.default_rng(seed)
    w = (rng.standard_normal((rows, cols)) * 0.02).astype(np.float32)
    blk = w.reshape(-1, 64)
    blk[0] = 0.0
    blk[1] = -0.0
    blk[2] = (rng.standard_normal(64) * 1e-41).astype(np.float32)
    blk[3] = (rng.standard_normal(64) * 1e37).astype(np.float32)
    for bi, levels in ((4, O.nf4_levels()), (5, O.int4_levels())):
        q = levels.astype(np.float64)
        vals = []
        for m in (q[:-1] + q[1:]) / 2:
            f = np.float32(m)
            vals += [f, np.nextafter(f, np.float32(2)), np.nextafter(f, np.float32(-2))]
        blk[bi, :] = 0.0
        blk[bi, 0] = 1.0
        blk[bi, 1:1 + min(63, len(vals))] = np.array(vals[:63], np.float32)
    blk[6, ::5] = 0.0                         # zeros in a non-zero block
    blk[7, :] = 0.125
    blk[8, :] = -0.0
    blk[8, 9] = np.float32(1e-45)
    blk[9] = np.linspace(-1, 1, 64).astype(np.float32) * np.float32(3.0)
    # a float32 product q[10] * c that is an exact binary16 tie (without
    # double quantisation c is stored as it is): rounding to float32 first
    # and then to fp16 must give the even neighbour
    c = np.float32(float.fromhex("0x1.72a384p-5"))
    blk[10, :] = np.float32(O.nf4_levels()[10]) * c
    blk[10, 0] = c
    return w


def _state_equal(wq, ref, what):
    gc = wq.codes.cpu().numpy()
    bad = np.nonzero(gc != ref["codes"])[0]
    assert bad.size == 0, f"{what}: codes differ at bytes {bad[:8]}: {gc[bad[:8]]} vs {ref['codes'][bad[:8]]}"
    got_s = wq.absmax_scale.cpu().numpy().view(np.uint32)
    assert np.array_equal(got_s, np.asarray(ref["absmax_scale"], np.float32).view(np.uint32)), \
        f"{what}: constants"
    if ref["double_quant"]:
        assert np.array_equal(wq.absmax_code.cpu().numpy(), ref["absmax_code"]), f"{what}: code8"
        assert np.array_equal(wq.absmax_offset.cpu().numpy().view(np.uint32),
                              np.asarray(ref["absmax_offset"], np.float32).view(np.uint32))
    else:
        assert wq.absmax_code.numel() == 0 and wq.absmax_offset.numel() == 0


CASES = {
    "adversarial": _adversarial,
    "ragged_272x1088": lambda: WL.weight(272, 1088, seed=5, outliers=True),
    "groups_1040x4160": lambda: WL.weight(1040, 4160, seed=6),
    # the merge test's weight: with double quantisation several blocks share
    # a constant whose NF4 product is a binary16 tie
    "fp16_ties_272x1088": lambda: WL.linear_inputs(
        WL.Workload(index=101, name="m", tokens=0, linears=(WL.Linear("l", 272, 1088),),
                    rank=32, alpha=16.0, outliers=True), 0, seed=9)["w"],
}


@pytest.mark.parametrize("fmt", FORMATS, ids=[f"{a}-{'dq' if b else 'nodq'}" for a, b in FORMATS])
@pytest.mark.parametrize("case", list(CASES))
def test_quantize_dequantize_variant_bit_exact(case, fmt):
    q = _q()
    qt, dq = fmt
    print(f"[variant] quantise case={case} {qt} dq={dq}", flush=True)
    w = CASES[case]()
    wq = q.qlora_nf4_quantize(f32_dev(w), quant_type=qt, double_quant=dq)
    ref = O.quantize(w, qt, dq)
    torch.cuda.synchronize()
    _state_equal(wq, ref, f"{case} {qt} dq={dq}")
    for dt in DTYPES:
        got = q.qlora_nf4_dequantize(dataclasses.replace(wq, compute_dtype=dt))
        torch.cuda.synchronize()
        bad = np.argwhere(bits_host(got) != O.dequantize_bits(ref, dt))
        assert bad.size == 0, f"{case} {qt} dq={dq} {dt}: dequant differs at {bad[:5].tolist()}"


@pytest.mark.parametrize("fmt", [("nf4", False), ("int4", True)], ids=["nf4-nodq", "int4-dq"])
def test_variant_full_size_bulk_sampled_rows(fmt):
    """The 8192 x 22016 weight: every constant, 50 sampled rows of codes and
    of the bf16 and fp16 dequantised weight."""
    q = _q()
    qt, dq = fmt
    w = WL.linear_inputs(WL.WORKLOADS["bulk_8192x22016"], 0)["w"]
    rows, cols = w.shape
    print(f"[variant] bulk 8192x22016 {qt} dq={dq}", flush=True)
    wq = q.qlora_nf4_quantize(f32_dev(w), quant_type=qt, double_quant=dq)
    deq = {dt: q.qlora_nf4_dequantize(dataclasses.replace(wq, compute_dtype=dt)) for dt in DTYPES}
    torch.cuda.synchronize()
    sel = np.unique(np.concatenate([np.random.default_rng(8).choice(rows, 48, replace=False),
                                    [0, rows - 1]]))
    st = O.quantize_sampled_rows(w, sel, qt, dq)
    got_codes = wq.codes.view(rows, cols // 2)[torch.from_numpy(sel).to(dev())].cpu().numpy()
    assert np.array_equal(got_codes, st["codes"])
    assert np.array_equal(wq.absmax_scale.cpu().numpy().view(np.uint32),
                          np.asarray(st["absmax_scale"], np.float32).view(np.uint32))
    if dq:
        assert np.array_equal(wq.absmax_code.cpu().numpy(), st["absmax_code"])
    for dt in DTYPES:
        got = bits_host(deq[dt][torch.from_numpy(sel).to(dev())])
        assert np.array_equal(got, O.dequantize_sampled_bits(st, dt)), dt


def _check_merge(got_bits, ref_bits, dt, what):
    got, ref = O.bits16_to_f32(got_bits, dt), O.bits16_to_f32(ref_bits, dt)
    frac = 7 if dt == "bf16" else 10
    ulp = 2.0 ** (np.floor(np.log2(np.maximum(np.abs(ref.astype(np.float64)),
                                              2.0 ** -14))) - frac)
    bad = np.argwhere(np.abs(got.astype(np.float64) - ref) > ulp)
    assert bad.size == 0, f"{what}: more than 1 ulp at {bad[:5].tolist()}"
    exact = np.mean(got_bits == ref_bits)
    print(f"[variant] {what} bit-identical fraction {exact:.5f}", flush=True)
    assert exact >= 0.99, (what, exact)


MERGE = [(qt, dq, dt) for qt, dq in FORMATS for dt in DTYPES]


@pytest.mark.parametrize("fmt", MERGE, ids=[f"{a}-{'dq' if b else 'nodq'}-{c}" for a, b, c in MERGE])
def test_merge_variant(fmt):
    q = _q()
    qt, dq, dt = fmt
    rows, cols, r, alpha = 272, 1088, 32, 16.0
    print(f"[variant] merge {qt} dq={dq} {dt}", flush=True)
    wl = WL.Workload(index=101, name="m", tokens=0, linears=(WL.Linear("l", rows, cols),),
                     rank=r, alpha=alpha, outliers=True)
    inp = WL.linear_inputs(wl, 0, seed=9, dtype=dt)
    wq = q.qlora_nf4_quantize(f32_dev(inp["w"]), quant_type=qt, double_quant=dq,
                              compute_dtype=dt)
    dt_t = torch.float16 if dt == "fp16" else torch.bfloat16
    A = torch.from_numpy(inp["a"].view(np.int16)).to(dev()).view(dt_t)
    B = torch.from_numpy(inp["b"].view(np.int16)).to(dev()).view(dt_t)
    got = q.qlora_nf4_merge(wq, A, B, alpha)
    zero = q.qlora_nf4_merge(wq, A, torch.zeros_like(B), alpha)
    deq = q.qlora_nf4_dequantize(wq)
    torch.cuda.synchronize()
    st = O.quantize(inp["w"], qt, dq)
    base = O.dequantize_bits(st, dt)
    ref = O.merge_bits(base, WL.bits16_value(inp["a"], dt).astype(np.float64),
                       WL.bits16_value(inp["b"], dt).astype(np.float64), alpha, r, dt)
    _check_merge(bits_host(got), ref, dt, f"merge {qt} dq={dq} {dt}")
    assert np.array_equal(bits_host(zero), base)
    assert np.array_equal(bits_host(deq), base)


def _dev16(bits, dt):
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev())
    return t.view(torch.float16 if dt == "fp16" else torch.bfloat16)


def _val16(t, dt):
    return WL.bits16_value(bits_host(t), dt).astype(np.float64)


# (name, T, N, K, r, alpha, double_quant, dtype, dropout p)
LINEAR = [
    ("fp16_dq_T300_N1040_K1088_r32", 300, 1040, 1088, 32, 32.0, True, "fp16", None),
    ("fp16_nodq_T520_N528_K576_r64", 520, 528, 576, 64, 16.0, False, "fp16", None),
    ("bf16_nodq_T300_N1040_K1088_r16", 300, 1040, 1088, 16, 32.0, False, "bf16", None),
    ("fp16_dq_skinny_T16_N272_K320_r128", 16, 272, 320, 128, 16.0, True, "fp16", None),
    ("bf16_nodq_skinny_T40_N528_K1024_r64", 40, 528, 1024, 64, 16.0, False, "bf16", None),
    # the skinny finish's 16-row form without double quantisation, and fp16
    # with two token groups
    ("bf16_nodq_skinny_T8_N144_K576_r32", 8, 144, 576, 32, 32.0, False, "bf16", None),
    ("fp16_dq_skinny_T48_N160_K640_r16", 48, 160, 640, 16, 16.0, True, "fp16", None),
    ("fp16_nodq_dropout_T260_N272_K1024_r16", 260, 272, 1024, 16, 32.0, False, "fp16", 0.1),
    # K-split of the last round in both fused GEMMs (270 and 261 tiles), fp16
    # and float32 constants
    ("fp16_nodq_ksplit_T2300_N7440_K7424_r16", 2300, 7440, 7424, 16, 16.0, False, "fp16", None),
]


@pytest.mark.parametrize("case", LINEAR, ids=[c[0] for c in LINEAR])
def test_linear_variant_parity(case):
    q = _q()
    name, T, N, K, r, alpha, dq, dt, p = case
    print(f"[variant] linear case={name}", flush=True)
    wl = WL.Workload(index=102, name="v", tokens=T, linears=(WL.Linear("l", N, K),), rank=r,
                     alpha=alpha, outliers=True)
    inp = WL.linear_inputs(wl, 0, seed=10, dtype=dt)
    wq = q.qlora_nf4_quantize(f32_dev(inp["w"]), double_quant=dq, compute_dtype=dt)
    X, A, B, dY = (_dev16(inp[k], dt) for k in ("x", "a", "b", "dy"))
    x, a, b, dy = (WL.bits16_value(inp[k], dt).astype(np.float64) for k in ("x", "a", "b", "dy"))
    w_hat = O.dequantize(O.quantize(inp["w"], "nf4", dq), dt)
    if p is None:
        Y, U = q.qlora_linear_fwd(wq, X, A, B, alpha)
        dX, dA, dB = q.qlora_linear_bwd(wq, X, dY, A, B, alpha, U_saved=U)
        y, u = O.linear_forward(x, w_hat, a, b, alpha, r)
        dx, da, db = O.linear_backward(x, dy, w_hat, a, b, alpha, r)
    else:
        Y, U, keep = q.qlora_linear_fwd_dropout(wq, X, A, B, alpha, p, 5, 6)
        dX, dA, dB = q.qlora_linear_bwd_dropout(wq, X, dY, A, B, alpha, p, 5, 6,
                                                keep_saved=keep, U_saved=U)
        km = O.dropout_keep_mask(T, K, p, 5, 6)
        y, u = O.linear_forward_dropout(x, w_hat, a, b, alpha, r, km, p)
        dx, da, db = O.linear_backward_dropout(x, dy, w_hat, a, b, alpha, r, km, p)
    torch.cuda.synchronize()
    got = {"y": _val16(Y, dt), "u": _val16(U, dt), "dx": _val16(dX, dt),
           "da": dA.cpu().numpy().astype(np.float64), "db": dB.cpu().numpy().astype(np.float64)}
    ref = {"y": y, "u": u, "dx": dx, "da": da, "db": db}
    errs = {k: O.rel_frobenius(got[k], ref[k]) for k in ref}
    print(f"[variant] {name} rel_frobenius " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()),
          flush=True)
    for k, v in errs.items():
        assert v <= GEMM_TOL, (name, k, v)


def test_attn_4096_fp16_full_size():
    """The attention workload in fp16 at full size (4096 tokens, 4096 x 4096,
    r = 16), in the benchmark's launch configuration: Y and dX on 50 sampled
    features, U, dA, dB in full."""
    q = _q()
    wl = WL.WORKLOADS["attn_4096"]
    dt = "fp16"
    inp = WL.linear_inputs(wl, 0, dtype=dt)
    N, K = inp["w"].shape
    T, r, alpha = wl.tokens, wl.rank, wl.alpha
    print("[variant] attn_4096 fp16 full size", flush=True)
    wq = q.qlora_nf4_quantize(f32_dev(inp["w"]), compute_dtype=dt)
    X, A, B, dY = (_dev16(inp[k], dt) for k in ("x", "a", "b", "dy"))
    Y, U = q.qlora_linear_fwd(wq, X, A, B, alpha)
    dX, dA, dB = q.qlora_linear_bwd(wq, X, dY, A, B, alpha, U_saved=U)
    torch.cuda.synchronize()
    del wq, X, A, B, dY
    rng = np.random.default_rng(102)
    sel_n = np.unique(np.concatenate([rng.choice(N, 48, replace=False), [0, N - 1]]))
    sel_k = np.unique(np.concatenate([rng.choice(K, 48, replace=False), [0, K - 1]]))
    w_rows = O.bits16_to_f32(O.dequantize_sampled_bits(
        O.quantize_sampled_rows(inp["w"], sel_n), dt), dt).astype(np.float64)
    w_cols = O.bits16_to_f32(O.dequantize_sampled_cols_bits(
        O.quantize_sampled_cols(inp["w"], sel_k), dt), dt).astype(np.float64)
    x, a, b, dy = (WL.bits16_value(inp[k], dt).astype(np.float64) for k in ("x", "a", "b", "dy"))
    y_ref, u_ref = O.linear_forward(x, w_rows, a, b[sel_n], alpha, r)
    dx_ref = O.linear_input_grad(dy, w_cols, a[:, sel_k], b, alpha, r)
    da_ref, db_ref = O.lora_grads(x, dy, a, b, alpha, r)
    got = {"y": _val16(Y, dt)[:, sel_n], "u": _val16(U, dt), "dx": _val16(dX, dt)[:, sel_k],
           "da": dA.cpu().numpy().astype(np.float64), "db": dB.cpu().numpy().astype(np.float64)}
    ref = {"y": y_ref, "u": u_ref, "dx": dx_ref, "da": da_ref, "db": db_ref}
    errs = {k: O.rel_frobenius(got[k], ref[k]) for k in ref}
    print("[variant] attn_4096 fp16 rel_frobenius "
          + " ".join(f"{k}={v:.2e}" for k, v in errs.items()), flush=True)
    for k, v in errs.items():
        assert v <= GEMM_TOL, (k, v)
