"""Helpers for the GPU parity tests: move seeded inputs to the device, run the
library, and bring results back as NumPy for comparison with the oracle."""
import numpy as np
import torch

import workloads as WL
from oracle import qlora_nf4_oracle as O

GEMM_TOL = 5e-3     # relative Frobenius error bound for GEMM outputs and gradients


def dev():
    return torch.device("cuda", 0)


def f32_dev(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(dev())


def bf16_dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev()).view(torch.bfloat16)


def bits_host(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def state_host(wq):
    """GPU packed weight -> dict in the oracle's layout."""
    return {
        "rows": wq.rows, "cols": wq.cols,
        "codes": wq.codes.cpu().numpy(),
        "absmax_code": wq.absmax_code.cpu().numpy(),
        "absmax_scale": wq.absmax_scale.cpu().numpy(),
        "absmax_offset": wq.absmax_offset.cpu().numpy(),
    }


def state_dev(st):
    """Oracle packed state -> NF4Weight on the device."""
    from bit_nf4_quantized_06_amd import NF4Weight
    return NF4Weight(st["rows"], st["cols"],
                     torch.from_numpy(st["codes"]).to(dev()),
                     torch.from_numpy(st["absmax_code"]).to(dev()),
                     torch.from_numpy(np.asarray(st["absmax_scale"], np.float32)).to(dev()),
                     torch.from_numpy(np.asarray(st["absmax_offset"], np.float32)).to(dev()))


def assert_state_equal(got, ref, what=""):
    assert np.array_equal(got["absmax_offset"].view(np.uint32),
                          np.asarray(ref["absmax_offset"], np.float32).view(np.uint32)), \
        f"{what}: mu {got['absmax_offset']} vs {ref['absmax_offset']}"
    s2g = got["absmax_scale"].view(np.uint32)
    s2r = np.asarray(ref["absmax_scale"], np.float32).view(np.uint32)
    bad = np.nonzero(s2g != s2r)[0]
    assert bad.size == 0, f"{what}: s2 differs at {bad[:10]}"
    bad = np.nonzero(got["absmax_code"] != ref["absmax_code"])[0]
    assert bad.size == 0, f"{what}: code8 differs at {bad[:10]} " \
        f"{got['absmax_code'][bad[:10]]} vs {ref['absmax_code'][bad[:10]]}"
    bad = np.nonzero(got["codes"] != ref["codes"])[0]
    assert bad.size == 0, f"{what}: packed codes differ at bytes {bad[:10]} " \
        f"{got['codes'][bad[:10]]} vs {ref['codes'][bad[:10]]}"


def linear_case(T, N, K, r, alpha, seed=0, outliers=False, b_zero=False, a_zero=False):
    """Seeded inputs of one linear, drawn like the workloads (bf16 bit patterns)."""
    wl = WL.Workload(index=100, name="case", tokens=T, linears=(WL.Linear("l", N, K),),
                     rank=r, alpha=alpha, outliers=outliers)
    inp = WL.linear_inputs(wl, 0, seed=seed)
    if b_zero:
        inp["b"] = np.zeros_like(inp["b"])
    if a_zero:
        inp["a"] = np.zeros_like(inp["a"])
    return inp


def oracle_linear(inp, w_hat, r, alpha):
    x = WL.bf16_bits_value(inp["x"]).astype(np.float64)
    a = WL.bf16_bits_value(inp["a"]).astype(np.float64)
    b = WL.bf16_bits_value(inp["b"]).astype(np.float64)
    y, u = O.linear_forward(x, w_hat, a, b, alpha, r)
    out = {"y": y, "u": u}
    if "dy" in inp:
        dy = WL.bf16_bits_value(inp["dy"]).astype(np.float64)
        dx, da, db = O.linear_backward(x, dy, w_hat, a, b, alpha, r)
        out.update(dx=dx, da=da, db=db)
    return out


# --------------------------------------------------------------------------
# Per-element and per-tile checks of GEMM outputs
# --------------------------------------------------------------------------
# A float32 accumulation of n exactly representable products (bf16 x bf16 is
# exact in float32) in any order is off by at most about n * u * sum |a_k b_k|
# with u = 2^-24; the factor 2u below also covers a matrix core that
# truncates instead of rounding.  sum |a_k b_k| <= |a| |b| (Cauchy-Schwarz),
# so each bound is an outer product of row norms and costs no extra matrix
# product.  A 16-bit output adds one rounding of at most 2^-8 of its value
# (bf16 keeps 8 significant bits).
U_ACC = 2.0 ** -23
TILE = 256


def _norms(m, axis):
    return np.sqrt(np.einsum("ij,ij->i" if axis == 1 else "ij,ij->j", m, m))


def linear_bounds(x, a, b, w_hat, alpha, r, dy=None):
    """Absolute per-element error bounds of the GPU's Y, U (and dX, dA, dB when
    dy is given) against the float64 oracle, from the float32 accumulations and
    the 16-bit roundings of the path: U and G = dY B are rounded to 16 bits
    (and s U, s G once more) before they feed the LoRA products, and dB uses
    the forward's 16-bit U.  All inputs are the float64 values of the 16-bit
    operands ([T, K] x, [r, K] a, [N, r] b, [N, K] w_hat, [T, N] dy)."""
    s = alpha / r
    T, K = x.shape
    N = w_hat.shape[0]
    nx, nw_r = _norms(x, 1), _norms(w_hat, 1)          # [T], [N]
    na_r, nb_r = _norms(a, 1), _norms(b, 1)            # [r], [N]
    u_ref = x @ a.T                                    # [T, r]
    nu = _norms(u_ref, 1)
    fro_a = float(np.sqrt((a * a).sum()))
    # |U16 - U| per element, and its row-norm bound
    eu = 2.0 ** -8 * np.abs(u_ref) + 1.01 * K * U_ACC * np.outer(nx, na_r)
    nu_err = 2.0 ** -8 * nu + 1.01 * K * U_ACC * nx * fro_a
    out = {"u": eu}
    # Y: accumulation over K + r terms, the rounded seed (two 16-bit roundings
    # of s U), then the output rounding (added by the checker)
    out["y"] = (1.01 * (K + r) * U_ACC * (np.outer(nx, nw_r) + s * np.outer(nu + nu_err, nb_r))
                + s * 1.01 * np.outer(2.0 ** -7 * nu + 1.01 * nu_err, nb_r))
    if dy is None:
        return out
    ndy = _norms(dy, 1)                                # [T]
    nw_c = _norms(w_hat, 0)                            # [K]
    na_c = _norms(a, 0)                                # [K]
    nb_c = _norms(b, 0)                                # [r]
    fro_b = float(np.sqrt((b * b).sum()))
    g_ref = dy @ b                                     # [T, r]
    ng = _norms(g_ref, 1)
    ng_err = 2.0 ** -8 * ng + 1.01 * N * U_ACC * ndy * fro_b
    out["dx"] = (1.01 * (N + r) * U_ACC * (np.outer(ndy, nw_c) + s * np.outer(ng + ng_err, na_c))
                 + s * 1.01 * np.outer(2.0 ** -7 * ng + 1.01 * ng_err, na_c))
    # dA = s G16^T X: per column p of G, |G16 - G| <= 2^-8 |G| + N u' |dy_t| |b_p|
    ng_c = _norms(g_ref, 0)                            # [r]
    nx_c = _norms(x, 0)                                # [K]
    n_ndy = float(np.sqrt((ndy * ndy).sum()))
    out["da"] = s * 1.01 * (
        (2.0 ** -8 + (T + 16) * U_ACC) * np.outer(ng_c, nx_c)
        + 1.01 * N * U_ACC * np.outer(nb_c * n_ndy, nx_c))
    # dB = s dY^T U16: |U16 - U| <= 2^-8 |U| + K u' |x_t| |a_p|
    nu_c = _norms(u_ref, 0)                            # [r]
    ndy_c = _norms(dy, 0)                              # [N]
    n_nx = float(np.sqrt((nx * nx).sum()))
    out["db"] = s * 1.01 * (
        (2.0 ** -8 + (T + 16) * U_ACC) * np.outer(ndy_c, nu_c)
        + 1.01 * K * U_ACC * np.outer(ndy_c, na_r * n_nx))
    return out


def _tile_sums(m, tile=TILE):
    rows = np.arange(0, m.shape[0], tile)
    cols = np.arange(0, m.shape[1], tile)
    return np.add.reduceat(np.add.reduceat(m, rows, axis=0), cols, axis=1)


def assert_gemm_close(what, got, ref, bound, out16=True, tol=GEMM_TOL):
    """got vs the float64 oracle ref, both [M, N]:
      * every element within `bound` (the accumulation bound of
        linear_bounds) plus the output's own rounding (2^-8 |ref| for a 16-bit
        output, 2^-23 |ref| for float32);
      * relative Frobenius error <= tol over the whole tensor and over every
        256 x 256 tile on its own, so one wrong tile or K-step cannot hide in
        the global norm."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    diff = got - ref
    lim = bound + (2.0 ** -8 if out16 else 2.0 ** -23) * np.abs(ref)
    bad = np.abs(diff) > lim
    if bad.any():
        idx = np.argwhere(bad)[:5]
        detail = ", ".join(f"{tuple(i)}: got {got[tuple(i)]:.6g} ref {ref[tuple(i)]:.6g} "
                           f"bound {lim[tuple(i)]:.3g}" for i in idx)
        raise AssertionError(f"{what}: {int(bad.sum())} elements beyond the per-element bound; "
                             f"{detail}")
    e = O.rel_frobenius(got, ref)
    assert e <= tol, f"{what}: relative Frobenius error {e:.3e} > {tol}"
    dsq = _tile_sums(diff * diff)
    rsq = _tile_sums(ref * ref)
    ok = rsq > 0
    tile_err = np.sqrt(dsq[ok] / rsq[ok])
    worst = float(tile_err.max()) if tile_err.size else 0.0
    assert worst <= tol, f"{what}: worst 256x256 tile relative Frobenius error {worst:.3e} > {tol}"
    return e, worst


def host_values(t):
    """float64 values of a 16-bit (bf16) or float32 device tensor."""
    if t.dtype == torch.float32:
        return t.cpu().numpy().astype(np.float64)
    return WL.bf16_bits_value(bits_host(t)).astype(np.float64)


def check_linear_outputs(name, got, inp, w_hat, r, alpha):
    """Compare the GPU outputs `got` (dict of float64 arrays, keys among y, u,
    dx, da, db) with the float64 oracle on the inputs `inp` and the oracle's
    dequantised weight `w_hat`, each with assert_gemm_close."""
    x = WL.bf16_bits_value(inp["x"]).astype(np.float64)
    a = WL.bf16_bits_value(inp["a"]).astype(np.float64)
    b = WL.bf16_bits_value(inp["b"]).astype(np.float64)
    dy = WL.bf16_bits_value(inp["dy"]).astype(np.float64) if "dx" in got else None
    ref = oracle_linear(inp if dy is not None else {k: v for k, v in inp.items() if k != "dy"},
                        w_hat, r, alpha)
    bounds = linear_bounds(x, a, b, w_hat, alpha, r, dy)
    res = {}
    for k in ("y", "u", "dx", "da", "db"):
        if k in got:
            res[k] = assert_gemm_close(f"{name} {k}", got[k], ref[k], bounds[k],
                                       out16=k not in ("da", "db"))
    print(f"[check] {name} rel_frobenius (whole, worst tile) "
          + " ".join(f"{k}={v[0]:.2e},{v[1]:.2e}" for k, v in res.items()), flush=True)
    return res
