"""The entry points under HIP graph capture: every kernel the library
launches goes on the caller's stream and none of them records a memset, so
a captured call replays.  Each case captures the calls once, then replays
the graph several times with eager work and synchronisations in between,
clearing the outputs before each replay, and checks every replay bit for
bit against the same calls made eagerly."""
import pytest
import torch

import workloads as WL
from gpu_util import bf16_dev, f32_dev, linear_case

pytestmark = pytest.mark.gpu

REPLAYS = 3


def _api():
    import bit_nf4_quantized_06_amd as q
    return q


def _bits(t):
    """bit patterns: 16-bit floats as int16, float32 as int32, bytes as they are"""
    if t.dtype in (torch.bfloat16, torch.float16):
        return t.view(torch.int16)
    if t.dtype == torch.float32:
        return t.view(torch.int32)
    return t


def _check_replays(name, run, outputs, eager_work):
    """run(): the calls, writing into `outputs` (a dict of tensors).  Eager
    reference first, then capture, then REPLAYS replays each against it."""
    run()
    torch.cuda.synchronize()
    ref = {k: _bits(v).clone() for k, v in outputs.items()}
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run()                        # warm-up on a side stream, as capture wants
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    torch.cuda.synchronize()
    for rep in range(REPLAYS):
        for v in outputs.values():
            v.zero_()
        g.replay()
        torch.cuda.synchronize()
        for k, v in outputs.items():
            assert torch.equal(_bits(v), ref[k]), (name, rep, k)
        print(f"[graph] {name} replay {rep} ok", flush=True)
        eager_work()                 # the program's own work between replays
        torch.cuda.synchronize()


# (name, T, N, K): the GEMM decoding in LDS; from 2048 tokens on, the
# once-per-call dequantisation inside the reduce launch and (7440 rows: 270
# tiles) the forward GEMM's K-split, whose arrival counters that launch
# zeroes on every replay
GENERAL = [("in_lds_T520", 520, 528, 576), ("predq_ksplit_T2300", 2300, 7440, 1088)]


@pytest.mark.parametrize("case", GENERAL, ids=[c[0] for c in GENERAL])
def test_general_fwd_bwd_graph(case):
    q = _api()
    name, T, N, K = case
    r, alpha = 64, 16.0
    print(f"[graph] general fwd+bwd {name}", flush=True)
    inp = linear_case(T, N, K, r, alpha, seed=31)
    wq = q.qlora_nf4_quantize(f32_dev(inp["w"]))
    X, A, B, dY = (bf16_dev(inp[k]) for k in ("x", "a", "b", "dy"))
    dev = X.device
    out = {"Y": torch.empty(T, N, dtype=torch.bfloat16, device=dev),
           "U": torch.empty(T, r, dtype=torch.bfloat16, device=dev),
           "dX": torch.empty(T, K, dtype=torch.bfloat16, device=dev),
           "dA": torch.empty(r, K, device=dev), "dB": torch.empty(N, r, device=dev)}
    wsf = torch.zeros(q.qlora_linear_workspace(T, N, K, r, False), dtype=torch.uint8, device=dev)
    wsb = torch.zeros(q.qlora_linear_workspace(T, N, K, r, True), dtype=torch.uint8, device=dev)

    def run():
        q.qlora_linear_fwd(wq, X, A, B, alpha, Y=out["Y"], U_save=out["U"], workspace=wsf)
        q.qlora_linear_bwd(wq, X, dY, A, B, alpha, U_saved=out["U"], dX=out["dX"], dA=out["dA"],
                           dB=out["dB"], workspace=wsb)

    other = torch.randn(1024, 1024, device=dev)
    _check_replays(f"general {name}", run, out, lambda: other.mul_(1.0001))


def test_skinny_forward_graph():
    q = _api()
    T, N, K, r, alpha = 16, 1040, 1024, 32, 32.0
    print("[graph] skinny fwd", flush=True)
    inp = linear_case(T, N, K, r, alpha, seed=32)
    wq = q.qlora_nf4_quantize(f32_dev(inp["w"]))
    X, A, B = (bf16_dev(inp[k]) for k in ("x", "a", "b"))
    dev = X.device
    out = {"Y": torch.empty(T, N, dtype=torch.bfloat16, device=dev),
           "U": torch.empty(T, r, dtype=torch.bfloat16, device=dev)}
    ws = torch.zeros(q.qlora_linear_workspace(T, N, K, r, False), dtype=torch.uint8, device=dev)

    def run():
        q.qlora_linear_fwd(wq, X, A, B, alpha, Y=out["Y"], U_save=out["U"], workspace=ws)

    # the eager work between replays: another skinny call on other inputs
    X2 = bf16_dev(linear_case(T, N, K, r, alpha, seed=33)["x"])
    _check_replays("skinny", run, out, lambda: q.qlora_linear_fwd(wq, X2, A, B, alpha))


def test_dropout_fwd_bwd_graph():
    q = _api()
    T, N, K, r, alpha, p = 300, 272, 1088, 16, 32.0, 0.1
    print("[graph] dropout fwd+bwd", flush=True)
    inp = linear_case(T, N, K, r, alpha, seed=34)
    wq = q.qlora_nf4_quantize(f32_dev(inp["w"]))
    X, A, B, dY = (bf16_dev(inp[k]) for k in ("x", "a", "b", "dy"))
    dev = X.device
    out = {"Y": torch.empty(T, N, dtype=torch.bfloat16, device=dev),
           "U": torch.empty(T, r, dtype=torch.bfloat16, device=dev),
           "keep": torch.empty((T + 3) // 4, K // 2, dtype=torch.uint8, device=dev),
           "dX": torch.empty(T, K, dtype=torch.bfloat16, device=dev),
           "dA": torch.empty(r, K, device=dev), "dB": torch.empty(N, r, device=dev)}
    wsf = torch.zeros(q.qlora_linear_workspace_dropout(T, N, K, r, False), dtype=torch.uint8,
                      device=dev)
    wsb = torch.zeros(q.qlora_linear_workspace_dropout(T, N, K, r, True), dtype=torch.uint8,
                      device=dev)

    def run():
        q.qlora_linear_fwd_dropout(wq, X, A, B, alpha, p, 7, 8, Y=out["Y"], U_save=out["U"],
                                   keep_save=out["keep"], workspace=wsf)
        q.qlora_linear_bwd_dropout(wq, X, dY, A, B, alpha, p, 7, 8, keep_saved=out["keep"],
                                   U_saved=out["U"], dX=out["dX"], dA=out["dA"], dB=out["dB"],
                                   workspace=wsb)

    _check_replays("dropout", run, out, lambda: q.qlora_dropout_mask(T, K, p, 1, 2, X=X))


def test_quantize_dequantize_graph():
    q = _api()
    rows, cols = 272, 1088
    print("[graph] quantize + dequantize", flush=True)
    w = f32_dev(WL.weight(rows, cols, seed=35, outliers=True))
    dev = w.device
    wq = q.NF4Weight.empty(rows, cols, dev)
    from bit_nf4_quantized_06_amd import _lib
    ws = torch.zeros(_lib.load().qlora_nf4_quantize_workspace(rows, cols), dtype=torch.uint8,
                     device=dev)
    deq = torch.empty(rows, cols, dtype=torch.bfloat16, device=dev)
    out = {"codes": wq.codes, "code8": wq.absmax_code, "s2": wq.absmax_scale,
           "mu": wq.absmax_offset, "deq": deq}

    def run():
        q.qlora_nf4_quantize(w, out=wq, workspace=ws)
        q.qlora_nf4_dequantize(wq, out=deq)

    w2 = f32_dev(WL.weight(rows, cols, seed=36))
    _check_replays("quantize", run, out, lambda: q.qlora_nf4_quantize(w2))
