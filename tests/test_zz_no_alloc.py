"""The allocation-free forward (qlora_linear_fwd_noalloc) through the C ABI:
its outputs equal qlora_linear_fwd's (given its own workspace) bit for bit,
on two calls in a row on one device, the second with a smaller input (the
shared device array keeps the first call's contents).  The allocation-free
forward always decodes the weight inside the GEMM; from 2048 tokens on
qlora_linear_fwd fetches a once-per-call 16-bit copy instead, so the
2300-token case also checks that both weight paths give the same bits."""
import ctypes

import numpy as np
import pytest
import torch

from gpu_util import bf16_dev, f32_dev, linear_case

pytestmark = pytest.mark.gpu


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


@pytest.mark.parametrize("cases", [[(1024, 1024, 2048, 32, 32.0), (16, 528, 1024, 16, 16.0)],
                                   [(64, 512, 1024, 64, 16.0), (33, 256, 512, 16, 32.0)],
                                   [(2300, 1040, 1088, 16, 16.0), (300, 528, 1024, 32, 32.0)]],
                         ids=["general_then_skinny", "skinny_then_smaller",
                              "predq_then_general"])
def test_noalloc_forward_equals_forward(cases):
    import bit_nf4_quantized_06_amd as q
    from bit_nf4_quantized_06_amd import _lib
    lib = _lib.load()
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    for i, (T, N, K, r, alpha) in enumerate(cases):
        print(f"[noalloc] call {i}: T={T} N={N} K={K} r={r}", flush=True)
        inp = linear_case(T, N, K, r, alpha, seed=31 + i, outliers=True)
        wq = q.qlora_nf4_quantize(f32_dev(inp["w"]))
        X, A, B = bf16_dev(inp["x"]), bf16_dev(inp["a"]), bf16_dev(inp["b"])
        Y0, U0 = q.qlora_linear_fwd(wq, X, A, B, alpha)
        Y1 = torch.full_like(Y0, float("nan"))
        U1 = torch.full_like(U0, float("nan"))
        torch.cuda.synchronize()
        desc = wq.descriptor()
        st = lib.qlora_linear_fwd_noalloc(ctypes.byref(desc), _ptr(X), T, _ptr(A), _ptr(B), r,
                                          ctypes.c_float(alpha), _ptr(Y1), _ptr(U1), stream)
        assert st == 0, lib.qlora_status_string(st)
        torch.cuda.synchronize()
        assert torch.equal(Y0.view(torch.int16), Y1.view(torch.int16)), f"Y differs (call {i})"
        assert torch.equal(U0.view(torch.int16), U1.view(torch.int16)), f"U differs (call {i})"
