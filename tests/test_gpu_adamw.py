"""GPU parity of the adapter AdamW step: parameters, both moments and the
bf16 copy equal the oracle's bit for bit over several steps, for a ragged
length (n % 4 != 0), with and without weight decay and without the bf16
copy, and for the adapters of a whole 7B block (r = 64, seven linears)."""
import numpy as np
import pytest
import torch

import workloads as WL
from gpu_util import bits_host, dev
from oracle import qlora_nf4_oracle as O

pytestmark = pytest.mark.gpu

HP = dict(lr=2e-4, beta1=0.9, beta2=0.999, eps=1e-8)


def _run(n, steps, wd, with_bf16, seed):
    import bit_nf4_quantized_06_amd as q
    rng = np.random.default_rng(seed)
    p = (rng.standard_normal(n) * 0.05).astype(np.float32)
    m = np.zeros(n, np.float32)
    v = np.zeros(n, np.float32)
    tp, tm, tv = (torch.from_numpy(x.copy()).to(dev()) for x in (p, m, v))
    tb = torch.empty(n, dtype=torch.bfloat16, device=dev()) if with_bf16 else None
    for step in range(1, steps + 1):
        g = (rng.standard_normal(n) * 10.0 ** rng.uniform(-5, -1)).astype(np.float32)
        g[:: 97] = 0.0                                   # some zero gradients
        tg = torch.from_numpy(g).to(dev())
        q.qlora_adamw_step(tp, tm, tv, tg, step, weight_decay=wd, param_bf16=tb, **HP)
        p, m, v, bits = O.adamw_step(p, m, v, g, step, HP["lr"], HP["beta1"], HP["beta2"],
                                     HP["eps"], wd)
        torch.cuda.synchronize()
        for name, got, ref in (("param", tp, p), ("exp_avg", tm, m), ("exp_avg_sq", tv, v)):
            gb = got.cpu().numpy().view(np.uint32)
            bad = np.nonzero(gb != ref.view(np.uint32))[0]
            assert bad.size == 0, (step, name, bad[:5], got.cpu().numpy()[bad[:5]], ref[bad[:5]])
        if with_bf16:
            assert np.array_equal(bits_host(tb), bits), step


@pytest.mark.parametrize("n,wd,with_bf16", [(4099, 0.0, True), (4099, 0.01, True),
                                            (1, 0.1, True), (1000, 0.0, False)])
def test_adamw_bit_exact(n, wd, with_bf16):
    print(f"[adamw] n={n} wd={wd} bf16={with_bf16}", flush=True)
    _run(n, steps=4, wd=wd, with_bf16=with_bf16, seed=n)


def test_adamw_7b_block_adapters():
    wl = WL.WORKLOADS["block_7b"]
    n = sum(wl.rank * (lin.in_features + lin.out_features) for lin in wl.linears)
    print(f"[adamw] 7B block adapters n={n}", flush=True)
    _run(n, steps=2, wd=0.01, with_bf16=True, seed=7)


@pytest.mark.parametrize("n", [4099, 257])
def test_adamw_fp16_copy_bit_exact(n):
    """qlora_adamw_step16 with an fp16 copy (fp16 compute): parameters,
    moments and the binary16 copy equal the oracle's bit for bit."""
    import bit_nf4_quantized_06_amd as q
    print(f"[adamw] fp16 copy n={n}", flush=True)
    rng = np.random.default_rng(n + 1)
    p = (rng.standard_normal(n) * 0.05).astype(np.float32)
    m = np.zeros(n, np.float32)
    v = np.zeros(n, np.float32)
    tp, tm, tv = (torch.from_numpy(x.copy()).to(dev()) for x in (p, m, v))
    t16 = torch.empty(n, dtype=torch.float16, device=dev())
    for step in range(1, 4):
        g = (rng.standard_normal(n) * 1e-3).astype(np.float32)
        q.qlora_adamw_step16(tp, tm, tv, torch.from_numpy(g).to(dev()), step, HP["lr"], t16,
                             beta1=HP["beta1"], beta2=HP["beta2"], eps=HP["eps"],
                             weight_decay=0.01)
        p, m, v, bits = O.adamw_step(p, m, v, g, step, HP["lr"], HP["beta1"], HP["beta2"],
                                     HP["eps"], 0.01, copy_dtype="fp16")
        torch.cuda.synchronize()
        assert np.array_equal(tp.cpu().numpy().view(np.uint32), p.view(np.uint32)), step
        assert np.array_equal(bits_host(t16), bits), step
