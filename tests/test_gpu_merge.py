"""GPU parity of the adapter merge, bf16(w_hat + (alpha/r) B A), against the
oracle: every merged weight within one bf16 ulp of the oracle's and at least
99% of them bit-identical (the product B A is accumulated in float32 in a
different order, which moves a result only when it sits within a few float32
ulps of a bf16 rounding boundary); with B = 0, bit-identical to the
dequantised weight.  Small ragged shapes for every rank class, and the
8192 x 22016 weight with a rank-64 adapter on sampled rows in the launch
configuration the benchmark times."""
import numpy as np
import pytest
import torch

import workloads as WL
from gpu_util import bf16_dev, bits_host, f32_dev, linear_case
from oracle import qlora_nf4_oracle as O

pytestmark = pytest.mark.gpu

# (name, rows, cols, r, alpha)
CASES = [
    ("N16_K64_r16", 16, 64, 16, 32.0),            # one partial tile
    ("N272_K1088_r32", 272, 1088, 32, 16.0),      # ragged column tile, second row group of 16
    ("N1040_K4096_r64", 1040, 4096, 64, 16.0),    # several row groups and column tiles
    ("N48_K320_r128", 48, 320, 128, 8.0),         # largest rank
    ("N32_K256_r48", 32, 256, 48, 96.0),          # a rank that is not a power of two
]


def _value(bits):
    return WL.bf16_bits_value(bits).astype(np.float64)


def _check(got_bits, ref_bits, what):
    got, ref = _value(got_bits), _value(ref_bits)
    ulp = np.abs(np.spacing(ref.astype(np.float32))).astype(np.float64) * 2.0 ** 16
    bad = np.argwhere(np.abs(got - ref) > ulp)
    assert bad.size == 0, f"{what}: more than 1 ulp at {bad[:5].tolist()}"
    exact = np.mean(got_bits == ref_bits)
    print(f"[merge] {what} bit-identical fraction {exact:.5f}", flush=True)
    assert exact >= 0.99, (what, exact)


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_merge_parity(case):
    import bit_nf4_quantized_06_amd as q
    name, rows, cols, r, alpha = case
    print(f"[merge] case={name}", flush=True)
    inp = linear_case(16, rows, cols, r, alpha, seed=31, outliers=True)
    wq = q.qlora_nf4_quantize(f32_dev(inp["w"]))
    got = q.qlora_nf4_merge(wq, bf16_dev(inp["a"]), bf16_dev(inp["b"]), alpha)
    torch.cuda.synchronize()
    ref = O.merge_bits(O.dequantize_bits(O.quantize(inp["w"])), _value(inp["a"]),
                       _value(inp["b"]), alpha, r)
    _check(bits_host(got), ref, name)


def test_merge_with_zero_b_is_the_dequantised_weight():
    import bit_nf4_quantized_06_amd as q
    print("[merge] B = 0", flush=True)
    inp = linear_case(16, 528, 1024, 64, 16.0, seed=32, b_zero=True)
    wq = q.qlora_nf4_quantize(f32_dev(inp["w"]))
    got = q.qlora_nf4_merge(wq, bf16_dev(inp["a"]), bf16_dev(inp["b"]), 16.0)
    deq = q.qlora_nf4_dequantize(wq)
    torch.cuda.synchronize()
    assert torch.equal(got.view(torch.int16), deq.view(torch.int16))
    assert np.array_equal(bits_host(got), O.dequantize_bits(O.quantize(inp["w"])))


def test_merge_leaves_the_packed_weight_unchanged_and_requantises():
    """The packed weight is read only; quantising the merged weight again
    (ta-paperlens 落とし穴: merge in 16 bit, quantise the result if needed)
    gives the oracle's state of the same float32 values."""
    import bit_nf4_quantized_06_amd as q
    print("[merge] re-quantise", flush=True)
    inp = linear_case(16, 256, 2048, 16, 32.0, seed=33)
    wq = q.qlora_nf4_quantize(f32_dev(inp["w"]))
    before = [t.clone() for t in (wq.codes, wq.absmax_code, wq.absmax_scale, wq.absmax_offset)]
    merged = q.qlora_nf4_merge(wq, bf16_dev(inp["a"]), bf16_dev(inp["b"]), 32.0)
    wq2 = q.qlora_nf4_quantize(merged.float().contiguous())
    torch.cuda.synchronize()
    after = (wq.codes, wq.absmax_code, wq.absmax_scale, wq.absmax_offset)
    assert all(torch.equal(x, y) for x, y in zip(before, after))
    from gpu_util import assert_state_equal, state_host
    ref = O.quantize(merged.float().cpu().numpy())
    assert_state_equal(state_host(wq2), ref, "re-quantised merge")


def test_merge_8192x22016_r64_sampled_rows():
    """The benchmark's merge workload at full size: 48 sampled rows plus the
    first and last, every column."""
    import bit_nf4_quantized_06_amd as q
    wl = WL.WORKLOADS["merge_8192x22016"]
    inp = WL.linear_inputs(wl, 0)
    rows, cols = inp["w"].shape
    print(f"[merge] full size {rows}x{cols} r={wl.rank}", flush=True)
    wq = q.qlora_nf4_quantize(f32_dev(inp["w"]))
    got = q.qlora_nf4_merge(wq, bf16_dev(inp["a"]), bf16_dev(inp["b"]), wl.alpha)
    torch.cuda.synchronize()
    del wq
    sel = np.sort(np.random.default_rng(5).choice(rows, 48, replace=False))
    sel = np.unique(np.concatenate([sel, [0, rows - 1]]))
    got_rows = bits_host(got[torch.from_numpy(sel).to(got.device)])
    del got
    st = O.quantize_sampled_rows(inp["w"], sel)
    ref = O.merge_bits(O.dequantize_sampled_bits(st), _value(inp["a"]),
                       _value(inp["b"])[sel], wl.alpha, wl.rank)
    _check(got_rows, ref, "8192x22016 r64 sampled rows")
