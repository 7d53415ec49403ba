"""GPU parity of the bulk path: packed codes, 8-bit constant codes, second-level
scales, the mean and the dequantised bf16 weights must equal the oracle's bit
for bit."""
import numpy as np
import pytest
import torch

import workloads as WL
from gpu_util import assert_state_equal, bits_host, f32_dev, state_dev, state_host
from oracle import qlora_nf4_oracle as O

pytestmark = pytest.mark.gpu


def _lib():
    from bit_nf4_quantized_06_amd import qlora_nf4_dequantize, qlora_nf4_quantize
    return qlora_nf4_quantize, qlora_nf4_dequantize


def _adversarial(rows=48, cols=320, seed=3):
    """Zero and -0 blocks, denormal blocks, huge blocks, exact midpoint ties
    and their float32 neighbours, single-element and constant blocks; n_b is
    not a multiple of 256."""
    rng = np.random.default_rng(seed)
    w = (rng.standard_normal((rows, cols)) * 0.02).astype(np.float32)
    blk = w.reshape(-1, 64)
    blk[0] = 0.0
    blk[1] = -0.0
    blk[2] = (rng.standard_normal(64) * 1e-41).astype(np.float32)      # denormals
    blk[3] = (rng.standard_normal(64) * 1e37).astype(np.float32)
    q = O.nf4_levels().astype(np.float64)
    mids = (q[:-1] + q[1:]) / 2
    vals = []
    for m in mids:
        f = np.float32(m)
        vals += [f, np.nextafter(f, np.float32(2)), np.nextafter(f, np.float32(-2))]
    vals = np.array(vals, np.float32)
    blk[4, :] = 0.0
    blk[4, 0] = 1.0
    blk[4, 1:1 + min(63, vals.size)] = vals[:63]
    blk[5, :] = 0.0
    blk[5, 0] = 2.0
    blk[5, 1:1 + min(63, vals.size - 20)] = vals[20:83] * np.float32(2.0)   # scaled ties
    blk[6, :] = 0.0
    blk[6, 17] = -3.5e-3
    blk[7, :] = 0.125
    blk[8] = (rng.standard_normal(64) * 1e-39).astype(np.float32)
    blk[8, ::3] *= np.float32(1e5)
    blk[9, :] = -0.0
    blk[9, 5] = np.float32(1e-45)                                        # smallest denormal
    blk[10] = np.linspace(-1, 1, 64).astype(np.float32)
    blk[11] = -np.linspace(-1, 1, 64).astype(np.float32) * np.float32(7.0)
    return w


CASES = {
    "single_1024": lambda: WL.linear_inputs(WL.WORKLOADS["single_1024"], 0)["w"],
    "adversarial_ragged": _adversarial,
    "ragged_groups_272x1088": lambda: WL.weight(272, 1088, seed=1, outliers=True),
    "one_block_16x64": lambda: WL.weight(16, 64, seed=2),
    "constant_absmax": lambda: np.where(np.arange(64 * 512) % 64 == 5, np.float32(0.5),
                                        (np.random.default_rng(4).uniform(-0.49, 0.49, 64 * 512))
                                        ).astype(np.float32).reshape(64, 512),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_quantize_and_dequantize_bit_exact(name):
    quantize, dequantize = _lib()
    w = CASES[name]()
    print(f"[quant] case={name} shape={w.shape}", flush=True)
    ref = O.quantize(w)
    wq = quantize(f32_dev(w))
    out = dequantize(wq)
    torch.cuda.synchronize()
    assert_state_equal(state_host(wq), ref, name)
    ref_bits = O.dequantize_bits(ref)
    got_bits = bits_host(out)
    bad = np.argwhere(got_bits != ref_bits)
    assert bad.size == 0, f"dequant differs at {bad[:8].tolist()}: " \
        f"{got_bits[tuple(bad[0])]:#06x} vs {ref_bits[tuple(bad[0])]:#06x}"


def test_dequantize_of_oracle_state():
    """Dequantisation checked on its own: the oracle's packed state goes in."""
    _, dequantize = _lib()
    w = _adversarial(rows=96, cols=704, seed=9)
    ref = O.quantize(w)
    out = dequantize(state_dev(ref))
    torch.cuda.synchronize()
    assert np.array_equal(bits_host(out), O.dequantize_bits(ref))


def test_quantize_is_deterministic_and_reuses_buffers():
    quantize, _ = _lib()
    w = WL.weight(512, 1024, seed=5, outliers=True)
    a = quantize(f32_dev(w))
    b = quantize(f32_dev(w), out=a.__class__.empty(512, 1024))
    torch.cuda.synchronize()
    for f in ("codes", "absmax_code", "absmax_scale", "absmax_offset"):
        assert torch.equal(getattr(a, f), getattr(b, f)), f


def test_bulk_8192x22016_full():
    """The bulk workload at full size, every value compared: the mean, every
    group scale, every 8-bit constant code, every packed code byte and every
    bf16 weight of the dequantised 8192 x 22016 tensor."""
    quantize, dequantize = _lib()
    wl = WL.WORKLOADS["bulk_8192x22016"]
    w = WL.linear_inputs(wl, 0)["w"]
    print(f"[quant] bulk shape={w.shape}", flush=True)
    wq = quantize(f32_dev(w))
    out = dequantize(wq)
    torch.cuda.synchronize()
    got = state_host(wq)
    got_bits = bits_host(out)
    del wq, out
    ref = O.quantize(w)
    del w
    assert_state_equal(got, ref, "bulk_8192x22016")
    ref_bits = O.dequantize_bits(ref)
    bad = np.argwhere(got_bits != ref_bits)
    assert bad.size == 0, f"dequant differs at {bad[:8].tolist()}"


def test_double_quant_constants_past_16384_groups():
    """A weight with more than 16384 groups of block constants (16448 x 16384:
    16448 groups), so the mean's tree folds runs of 32 group sums per thread:
    the mean, every second-level scale and every 8-bit constant code must
    equal the oracle's."""
    quantize, _ = _lib()
    rows, cols = 16448, 16384
    w = WL.weight(rows, cols, seed=6)
    print(f"[quant] long mean tree shape={w.shape}", flush=True)
    wq = quantize(f32_dev(w))
    torch.cuda.synchronize()
    got = state_host(wq)
    del wq
    c = O.block_absmax(w)
    del w
    code8, s2, mu = O.double_quantize(c)
    assert np.float32(got["absmax_offset"][0]) == mu
    assert np.array_equal(got["absmax_scale"].view(np.uint32), s2.view(np.uint32))
    assert np.array_equal(got["absmax_code"], code8)
