"""GPU parity of the fused forward and backward: Y, U, dX, dA and dB against
the float64 oracle (every element within its accumulation bound, relative
Frobenius error <= 5e-3 over the whole tensor and every 256 x 256 tile), plus
the special cases and invariants of the layer."""
import numpy as np
import pytest
import torch

import workloads as WL
from gpu_util import (GEMM_TOL, assert_state_equal, bf16_dev, bits_host, check_linear_outputs,
                      f32_dev, linear_case, oracle_linear, state_host)
from oracle import qlora_nf4_oracle as O

pytestmark = pytest.mark.gpu

# (name, T, N=rows=out, K=cols=in, r, alpha)
CASES = [
    ("tiny_T1", 1, 16, 64, 16, 16.0),
    ("ragged_T300_N1040_K1088_r32", 300, 1040, 1088, 32, 32.0),
    ("r128_T17_N272_K320", 17, 272, 320, 128, 16.0),
    ("r64_T520_N528_K576", 520, 528, 576, 64, 16.0),
    ("r48_T256_N256_K256", 256, 256, 256, 48, 96.0),
    # ranks past one 64-column seed tile: a second, partial (80) or whole
    # (128) tile of the adapter columns
    ("r80_T300_N528_K320", 300, 528, 320, 80, 16.0),
    ("r128_T300_N272_K576", 300, 272, 576, 128, 16.0),
    # more than 256 tiles with a last round at most half full: the forward
    # (270 tiles, 17 reduction steps) and the dX GEMM (261 tiles, 17 steps)
    # split their last 14 and 5 tiles into two reduction halves; ragged token
    # and row tiles
    ("ksplit_fwd_T2300_N7440_K1088", 2300, 7440, 1088, 16, 16.0),
    ("ksplit_dx_T2300_N1040_K7424", 2300, 1040, 7424, 16, 16.0),
]


def _api():
    import bit_nf4_quantized_06_amd as q
    return q


def _run(inp, r, alpha, save_u=True):
    q = _api()
    wq = q.qlora_nf4_quantize(f32_dev(inp["w"]))
    X, A, B = bf16_dev(inp["x"]), bf16_dev(inp["a"]), bf16_dev(inp["b"])
    Y, U = q.qlora_linear_fwd(wq, X, A, B, alpha)
    res = {"wq": wq, "Y": Y, "U": U}
    if "dy" in inp:
        dY = bf16_dev(inp["dy"])
        dX, dA, dB = q.qlora_linear_bwd(wq, X, dY, A, B, alpha, U_saved=U if save_u else None)
        res.update(dX=dX, dA=dA, dB=dB)
    torch.cuda.synchronize()
    return res


def _host(res):
    out = {"y": WL.bf16_bits_value(bits_host(res["Y"])).astype(np.float64),
           "u": WL.bf16_bits_value(bits_host(res["U"])).astype(np.float64)}
    if "dX" in res:
        out["dx"] = WL.bf16_bits_value(bits_host(res["dX"])).astype(np.float64)
        out["da"] = res["dA"].cpu().numpy().astype(np.float64)
        out["db"] = res["dB"].cpu().numpy().astype(np.float64)
    return out


def _check(name, got, ref):
    errs = {k: O.rel_frobenius(got[k], ref[k]) for k in ref if k in got}
    print(f"[linear] {name} rel_frobenius " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()),
          flush=True)
    for k, v in errs.items():
        assert v <= GEMM_TOL, (name, k, v)
    return errs


def test_single_1024_workload():
    wl = WL.WORKLOADS["single_1024"]
    inp = WL.linear_inputs(wl, 0)
    print("[linear] single_1024", flush=True)
    st = O.quantize(inp["w"])
    res = _run(inp, wl.rank, wl.alpha)
    assert_state_equal(state_host(res["wq"]), st, "single_1024")
    deq = _api().qlora_nf4_dequantize(res["wq"])
    torch.cuda.synchronize()
    assert np.array_equal(bits_host(deq), O.dequantize_bits(st)), "dequantised weight differs"
    check_linear_outputs("single_1024", _host(res), inp, O.dequantize(st), wl.rank, wl.alpha)


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_linear_parity(case):
    name, T, N, K, r, alpha = case
    print(f"[linear] case={name}", flush=True)
    inp = linear_case(T, N, K, r, alpha, seed=11, outliers=True)
    st = O.quantize(inp["w"])
    res = _run(inp, r, alpha)
    assert_state_equal(state_host(res["wq"]), st, name)
    check_linear_outputs(name, _host(res), inp, O.dequantize(st), r, alpha)


def test_b_zero_gives_base_output_and_zero_da():
    """B = 0 (the adapter's initial state) and A = 0 both reduce the layer to
    the frozen base: identical bits; with B = 0, dA is exactly 0."""
    T, N, K, r, alpha = 260, 528, 576, 16, 32.0
    print("[linear] b_zero", flush=True)
    inp_b0 = linear_case(T, N, K, r, alpha, seed=5, b_zero=True)
    inp_a0 = linear_case(T, N, K, r, alpha, seed=5, a_zero=True)
    rb = _run(inp_b0, r, alpha)
    ra = _run(inp_a0, r, alpha)
    assert torch.equal(rb["Y"].view(torch.int16), ra["Y"].view(torch.int16))
    assert torch.count_nonzero(rb["dA"]).item() == 0
    st = O.quantize(inp_b0["w"])
    ref = oracle_linear(inp_b0, O.dequantize(st), r, alpha)
    _check("b_zero", _host(rb), ref)


def test_deterministic_frozen_weight_and_recompute_path():
    T, N, K, r, alpha = 384, 512, 640, 64, 16.0
    print("[linear] determinism", flush=True)
    inp = linear_case(T, N, K, r, alpha, seed=7, outliers=True)
    q = _api()
    wq = q.qlora_nf4_quantize(f32_dev(inp["w"]))
    before = [t.clone() for t in (wq.codes, wq.absmax_code, wq.absmax_scale, wq.absmax_offset)]
    X, A, B, dY = (bf16_dev(inp[k]) for k in ("x", "a", "b", "dy"))
    outs = []
    for _ in range(2):
        Y, U = q.qlora_linear_fwd(wq, X, A, B, alpha)
        dX, dA, dB = q.qlora_linear_bwd(wq, X, dY, A, B, alpha, U_saved=U)
        outs.append((Y.clone(), U.clone(), dX.clone(), dA.clone(), dB.clone()))
    dX2, dA2, dB2 = q.qlora_linear_bwd(wq, X, dY, A, B, alpha, U_saved=None)
    torch.cuda.synchronize()
    for a, b in zip(outs[0], outs[1]):
        assert torch.equal(a, b)
    assert torch.equal(dX2, outs[0][2]) and torch.equal(dA2, outs[0][3])
    assert torch.equal(dB2, outs[0][4])
    after = (wq.codes, wq.absmax_code, wq.absmax_scale, wq.absmax_offset)
    for a, b in zip(before, after):
        assert torch.equal(a, b)


def test_empty_batch():
    """T = 0: Y, U and dX are empty and dA, dB are exactly the oracle's sums
    over no tokens (all +0.0), overwriting whatever the buffers held; the
    same through the lora_dropout entry points."""
    import bit_nf4_quantized_06_amd as q
    N, K, r, alpha = 272, 320, 16, 32.0
    print("[linear] empty batch T=0", flush=True)
    inp = linear_case(4, N, K, r, alpha, seed=21)
    wq = q.qlora_nf4_quantize(f32_dev(inp["w"]))
    A, B = bf16_dev(inp["a"]), bf16_dev(inp["b"])
    X = torch.empty(0, K, dtype=torch.bfloat16, device=A.device)
    dY = torch.empty(0, N, dtype=torch.bfloat16, device=A.device)
    x0 = np.zeros((0, K))
    dy0 = np.zeros((0, N))
    da_ref, db_ref = O.lora_grads(x0, dy0, WL.bf16_bits_value(inp["a"]),
                                  WL.bf16_bits_value(inp["b"]), alpha, r)
    for drop in (None, 0.1):
        dA = torch.full((r, K), float("nan"), device=A.device)
        dB = torch.full((N, r), float("nan"), device=A.device)
        if drop is None:
            Y, U = q.qlora_linear_fwd(wq, X, A, B, alpha)
            dX, dA, dB = q.qlora_linear_bwd(wq, X, dY, A, B, alpha, U_saved=U, dA=dA, dB=dB)
        else:
            Y, U, keep = q.qlora_linear_fwd_dropout(wq, X, A, B, alpha, drop, 3, 4)
            assert keep.numel() == 0
            dX, dA, dB = q.qlora_linear_bwd_dropout(wq, X, dY, A, B, alpha, drop, 3, 4,
                                                    keep_saved=keep, U_saved=U, dA=dA, dB=dB)
        torch.cuda.synchronize()
        assert tuple(Y.shape) == (0, N) and tuple(U.shape) == (0, r)
        assert tuple(dX.shape) == (0, K)
        got_a, got_b = dA.cpu().numpy(), dB.cpu().numpy()
        assert np.array_equal(got_a.view(np.uint32), da_ref.astype(np.float32).view(np.uint32))
        assert np.array_equal(got_b.view(np.uint32), db_ref.astype(np.float32).view(np.uint32))
    keep_only, none = q.qlora_dropout_mask(0, K, 0.1, 1, 2, device=A.device)
    torch.cuda.synchronize()
    assert keep_only.numel() == 0 and none is None


def test_side_stream_allocations_follow_the_call_stream():
    """Calls on a side stream while the current stream keeps allocating: the
    binding takes the workspaces it creates from the side stream's pool, so
    the current stream's allocations cannot reuse them while the side
    stream's kernels still run.  Results equal the current-stream call bit
    for bit (a torch.cuda.Stream and a raw stream handle)."""
    T, N, K, r, alpha = 1024, 1024, 2048, 16, 32.0
    print("[linear] side stream", flush=True)
    q = _api()
    inp = linear_case(T, N, K, r, alpha, seed=17, outliers=True)
    wq = q.qlora_nf4_quantize(f32_dev(inp["w"]))
    X, A, B, dY = (bf16_dev(inp[k]) for k in ("x", "a", "b", "dy"))
    Y0, U0 = q.qlora_linear_fwd(wq, X, A, B, alpha)
    dX0, dA0, dB0 = q.qlora_linear_bwd(wq, X, dY, A, B, alpha, U_saved=U0)
    torch.cuda.synchronize()
    ws_f = q.qlora_linear_workspace(T, N, K, r, False)
    ws_b = q.qlora_linear_workspace(T, N, K, r, True)
    side = torch.cuda.Stream()
    for handle in (side, side.cuda_stream):
        side.wait_stream(torch.cuda.current_stream())
        Y1, U1 = q.qlora_linear_fwd(wq, X, A, B, alpha, stream=handle)
        dX1, dA1, dB1 = q.qlora_linear_bwd(wq, X, dY, A, B, alpha, U_saved=U1, stream=handle)
        # the current stream allocates blocks of the workspaces' sizes and
        # overwrites them while the side stream may still be running
        junk = [torch.full((max(ws_f, ws_b),), 0x7F, dtype=torch.uint8, device=X.device)
                for _ in range(4)]
        side.synchronize()
        torch.cuda.synchronize()
        del junk
        for a, b in ((Y0, Y1), (U0, U1), (dX0, dX1)):
            assert torch.equal(a.view(torch.int16), b.view(torch.int16))
        assert torch.equal(dA0, dA1) and torch.equal(dB0, dB1)
