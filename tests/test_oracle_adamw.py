"""Pins for the oracle's adapter optimizer step (AdamW with 32-bit states;
ta-paperlens, paged optimizer section; waylandz 26.6.4), CPU only."""
import numpy as np
import pytest
import torch

from oracle import qlora_nf4_oracle as O


def _state(n, seed):
    rng = np.random.default_rng(seed)
    p = (rng.standard_normal(n) * 0.05).astype(np.float32)
    g = (rng.standard_normal(n) * 1e-3).astype(np.float32)
    return p, g


def test_power_by_squaring_is_exact_on_dyadic_values():
    assert O.power_by_squaring(0.5, 10) == 2.0 ** -10
    assert O.power_by_squaring(0.75, 3) == 27.0 / 64.0
    assert O.power_by_squaring(0.9, 0) == 1.0


@pytest.mark.parametrize("wd", [0.0, 0.01])
def test_matches_torch_adamw_over_several_steps(wd):
    """torch.optim.AdamW (CPU, float32, single-tensor path) is an independent
    implementation of the same update; it orders some float32 operations
    differently (the first moment as m + (1-b1)(g - m), products fused or
    not), so the two agree to a few float32 ulps of the operands."""
    n = 1000
    p, _ = _state(n, 1)
    lr, b1, b2, eps = 2e-4, 0.9, 0.999, 1e-8
    tp = torch.nn.Parameter(torch.from_numpy(p.copy()))
    opt = torch.optim.AdamW([tp], lr=lr, betas=(b1, b2), eps=eps, weight_decay=wd,
                            foreach=False)
    m = np.zeros(n, np.float32)
    v = np.zeros(n, np.float32)
    rng = np.random.default_rng(2)
    for step in range(1, 6):
        g = (rng.standard_normal(n) * 1e-3).astype(np.float32)
        tp.grad = torch.from_numpy(g.copy())
        opt.step()
        p, m, v, _ = O.adamw_step(p, m, v, g, step, lr, b1, b2, eps, wd)
        st = opt.state[tp]
        gmax = float(np.max(np.abs(g)))
        assert np.allclose(p, tp.detach().numpy(), rtol=1e-6, atol=1e-6 * lr)
        assert np.allclose(m, st["exp_avg"].numpy(), rtol=1e-5, atol=1e-6 * gmax)
        assert np.allclose(v, st["exp_avg_sq"].numpy(), rtol=1e-5, atol=1e-6 * gmax ** 2)


def test_first_step_moves_by_lr_against_the_gradient_sign():
    """From zero moments the bias-corrected ratio m/sqrt(v) is g/|g|, so with
    no weight decay and |g| >> eps every parameter moves by lr against the
    sign of its gradient."""
    n = 256
    p, g = _state(n, 3)
    lr = 1e-3
    p2, m, v, _ = O.adamw_step(p, np.zeros(n), np.zeros(n), g, 1, lr, 0.9, 0.999, 1e-12, 0.0)
    assert np.allclose(p - p2, lr * np.sign(g), rtol=1e-5)
    assert np.allclose(m, 0.1 * g, rtol=1e-6)


def test_zero_gradient_only_decays_exactly():
    """g = 0 and zero moments: the Adam term is 0 / eps = 0 and the parameter
    is scaled by 1 - lr*wd; lr = wd = 1/2 gives exactly 3/4 of it."""
    p = np.array([1.0, -2.0, 0.5, 3.0], np.float32)
    p2, m, v, bits = O.adamw_step(p, np.zeros(4), np.zeros(4), np.zeros(4), 7, 0.5, 0.9, 0.99,
                                  1e-8, 0.5)
    assert np.array_equal(p2, np.array([0.75, -1.5, 0.375, 2.25], np.float32))
    assert not m.any() and not v.any()
    assert np.array_equal(bits, np.array([0x3F40, 0xBFC0, 0x3EC0, 0x4010], np.uint16))
    # the fp16 copy of the same parameters: 0.75, -1.5, 0.375, 2.25 in binary16
    _, _, _, bits16 = O.adamw_step(p, np.zeros(4), np.zeros(4), np.zeros(4), 7, 0.5, 0.9, 0.99,
                                   1e-8, 0.5, copy_dtype="fp16")
    assert np.array_equal(bits16, np.array([0x3A00, 0xBE00, 0x3600, 0x4080], np.uint16))
