"""The two weight paths of the linear layer give the same bits.  From
qlora_pre_dequant_min_tokens() tokens on, qlora_linear_* dequantise the
weight once per call into the workspace and the GEMM fetches that 16-bit
copy by DMA; below it the GEMM decodes each weight tile into LDS.  Both
round q[code] * c' once to 16 bit and run the same MFMA sequence in the same
order, so Y, U, dX, dA and dB must agree bit for bit: checked on ragged
shapes, with the K-split of the last GEMM tiles in either direction, in fp16
with float32 constants, and under lora_dropout.  (Parity of either path with
the oracle is in test_gpu_linear.py, test_gpu_variants.py and
test_gpu_dropout.py.)"""
import numpy as np
import pytest
import torch

import workloads as WL
from gpu_util import dev, f32_dev

pytestmark = pytest.mark.gpu

NEVER = 2 ** 63 - 1

# (name, T, N=rows, K=cols, r, alpha, double_quant, compute dtype, dropout p)
CASES = [
    ("ragged_T2300_N1040_K1088_r16", 2300, 1040, 1088, 16, 16.0, True, "bf16", None),
    ("ksplit_fwd_T2300_N7440_K1088_r32", 2300, 7440, 1088, 32, 32.0, True, "bf16", None),
    ("ksplit_dx_T2300_N1040_K7424_r16", 2300, 1040, 7424, 16, 16.0, True, "bf16", None),
    ("fp16_nodq_T2100_N784_K1024_r64", 2100, 784, 1024, 64, 16.0, False, "fp16", None),
    ("dropout_T2300_N1040_K1088_r16_p01", 2300, 1040, 1088, 16, 16.0, True, "bf16", 0.1),
    # a weight smaller than one tile both ways (16 rows: one partial reduction
    # step in the backward, 64 columns), and a ragged one just past a tile
    ("tiny_weight_T2048_N16_K64_r16", 2048, 16, 64, 16, 32.0, True, "bf16", None),
    ("ragged_T2049_N272_K320_r128", 2049, 272, 320, 128, 16.0, True, "bf16", None),
]


def _step(q, wq, X, A, B, dY, alpha, p):
    if p is None:
        Y, U = q.qlora_linear_fwd(wq, X, A, B, alpha)
        dX, dA, dB = q.qlora_linear_bwd(wq, X, dY, A, B, alpha, U_saved=U)
    else:
        Y, U, keep = q.qlora_linear_fwd_dropout(wq, X, A, B, alpha, p, 1234, 0)[:3]
        dX, dA, dB = q.qlora_linear_bwd_dropout(wq, X, dY, A, B, alpha, p, 1234, 0,
                                                keep_saved=keep, U_saved=U)
    torch.cuda.synchronize()
    return [t.clone() for t in (Y, U, dX, dA, dB)]


def _dev16(bits, dt):
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev())
    return t.view(torch.float16 if dt == "fp16" else torch.bfloat16)


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_pre_dequantised_equals_in_lds_decode(case):
    import bit_nf4_quantized_06_amd as q
    name, T, N, K, r, alpha, dq, dt, p = case
    print(f"[predq] case={name}", flush=True)
    wl = WL.Workload(index=103, name="p", tokens=T, linears=(WL.Linear("l", N, K),), rank=r,
                     alpha=alpha, outliers=True)
    inp = WL.linear_inputs(wl, 0, seed=23, dtype=dt)
    wq = q.qlora_nf4_quantize(f32_dev(inp["w"]), double_quant=dq, compute_dtype=dt)
    X, A, B, dY = (_dev16(inp[k], dt) for k in ("x", "a", "b", "dy"))
    assert q.qlora_pre_dequant_min_tokens() <= T
    pre = _step(q, wq, X, A, B, dY, alpha, p)
    prev = q.qlora_set_pre_dequant_min_tokens(NEVER)
    try:
        lds = _step(q, wq, X, A, B, dY, alpha, p)
    finally:
        q.qlora_set_pre_dequant_min_tokens(prev)
    for what, a, b in zip(("Y", "U", "dX", "dA", "dB"), pre, lds):
        assert a.dtype == b.dtype and a.shape == b.shape, what
        ia = a.view(torch.int16) if a.element_size() == 2 else a.view(torch.int32)
        ib = b.view(torch.int16) if b.element_size() == 2 else b.view(torch.int32)
        assert torch.equal(ia, ib), f"{name}: {what} differs between the two weight paths"
