"""GPU parity of the skinny forward (T <= 64 tokens, the generation case):
Y and U against the float64 oracle (relative Frobenius error <= 5e-3) at
small ragged shapes, and at the 65B-style decode shapes (16 tokens) in
full, in the launch configuration the benchmark times.  Each comparison also
bounds every element (gpu_util.assert_gemm_close)."""
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
    ("T1_N16_K64_r16", 1, 16, 64, 16, 16.0),
    ("T16_N1040_K4096_r64", 16, 1040, 4096, 64, 16.0),     # ragged row tile, 4 splits
    ("T17_N144_K1024_r16", 17, 144, 1024, 16, 16.0),       # first T past the finish's 16-row form
    ("T31_N272_K1088_r32", 31, 272, 1088, 32, 32.0),       # 17 blocks per row
    ("T33_N528_K576_r16", 33, 528, 576, 16, 32.0),         # two token groups
    ("T64_N256_K2048_r128", 64, 256, 2048, 128, 16.0),     # largest skinny T, largest r
]


def _fwd(inp, alpha):
    import bit_nf4_quantized_06_amd as q
    wq = q.qlora_nf4_quantize(f32_dev(inp["w"]))
    X, A, B = bf16_dev(inp["x"]), bf16_dev(inp["a"]), bf16_dev(inp["b"])
    Y, U = q.qlora_linear_fwd(wq, X, A, B, alpha)
    torch.cuda.synchronize()
    return wq, X, A, B, Y, U


def _val(t):
    return WL.bf16_bits_value(bits_host(t)).astype(np.float64)


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_skinny_forward_parity(case):
    name, T, N, K, r, alpha = case
    print(f"[gemv] case={name}", flush=True)
    inp = linear_case(T, N, K, r, alpha, seed=21, outliers=True)
    inp.pop("dy")
    _, _, _, _, Y, U = _fwd(inp, alpha)
    check_linear_outputs(name, {"y": _val(Y), "u": _val(U)}, inp,
                         O.dequantize(O.quantize(inp["w"])), r, alpha)


def test_skinny_forward_deterministic_and_b_zero():
    """Repeated calls give identical bits; with B = 0 the output equals the
    A = 0 output (the frozen base alone), bit for bit."""
    T, N, K, r, alpha = 16, 528, 1024, 32, 32.0
    print("[gemv] determinism / b_zero", flush=True)
    import bit_nf4_quantized_06_amd as q
    inp_b0 = linear_case(T, N, K, r, alpha, seed=8, b_zero=True)
    inp_a0 = linear_case(T, N, K, r, alpha, seed=8, a_zero=True)
    wq, X, A, B, Y1, _ = _fwd(inp_b0, alpha)
    Y2, _ = q.qlora_linear_fwd(wq, X, A, B, alpha)
    _, _, _, _, Ya, _ = _fwd(inp_a0, alpha)
    torch.cuda.synchronize()
    assert torch.equal(Y1.view(torch.int16), Y2.view(torch.int16))
    assert torch.equal(Y1.view(torch.int16), Ya.view(torch.int16))


def _decode_cases():
    wl = WL.WORKLOADS["block_65b_decode"]
    seen, out = set(), []
    for li, lin in enumerate(wl.linears):
        shape = (lin.out_features, lin.in_features)
        if shape not in seen:
            seen.add(shape)
            out.append((lin.name, li))
    return out


@pytest.mark.parametrize("lin", _decode_cases(), ids=[c[0] for c in _decode_cases()])
def test_decode_65b_full_size(lin):
    """The 65B decode block at 16 tokens, one linear of each shape at full
    size through the same entry point the benchmark times: the packed state
    and the bf16 dequantised weight bit for bit, Y and U in full (every
    element within its accumulation bound, relative Frobenius error <= 5e-3
    over the whole tensor and every 256 x 256 tile)."""
    import bit_nf4_quantized_06_amd as q
    name, li = lin
    wl = WL.WORKLOADS["block_65b_decode"]
    inp = WL.linear_inputs(wl, li)
    inp.pop("dy", None)
    N, K = inp["w"].shape
    print(f"[gemv] decode {name} W={N}x{K} T={wl.tokens}", flush=True)
    wq, _, _, _, Y, U = _fwd(inp, wl.alpha)
    w_bf16 = q.qlora_nf4_dequantize(wq)
    torch.cuda.synchronize()
    got_state = state_host(wq)
    got_bits = bits_host(w_bf16)
    got = {"y": _val(Y), "u": _val(U)}
    del wq, w_bf16, Y, U
    st = O.quantize(inp["w"])
    assert_state_equal(got_state, st, f"decode {name}")
    ref_bits = O.dequantize_bits(st)
    assert np.array_equal(got_bits, ref_bits), "dequantised bf16 weight differs"
    w_hat = O.bf16_bits_to_f32(ref_bits).astype(np.float64)
    del ref_bits, got_bits
    check_linear_outputs(f"decode {name}", got, inp, w_hat, wl.rank, wl.alpha)
