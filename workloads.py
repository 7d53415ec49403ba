"""Seeded synthetic workloads for the NF4 + LoRA linear layer.

This module only draws random inputs and names the shapes; it holds none of
the method's arithmetic.  Both the oracle-based tests and the HIP path take
their inputs from here.

Recipe (every tensor is drawn from NumPy's PCG64 seeded with
[seed, workload index, linear index, tensor kind]):
  * W  float32 [out, in] ~ N(0, 0.02^2); where outliers are asked for,
    floor(0.001 * n) distinct positions (choice without replacement) are
    multiplied by 20;
  * X  [T, in] ~ N(0, 1), rounded to bf16 (round to nearest even);
  * A  [r, in] ~ N(0, 1/r), B [out, r] ~ N(0, 0.01^2), both rounded to bf16;
  * dY [T, out] ~ N(0, 1), rounded to bf16.
Weights ~N(0, 0.02^2) with rare large entries follow the pages' premise that
pretrained weights are roughly normal with outliers; token counts and linear
shapes are those of LLaMA-style 7B and 65B decoder blocks.
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np

KIND_W, KIND_X, KIND_A, KIND_B, KIND_DY = 0, 1, 2, 3, 4


@dataclass(frozen=True)
class Linear:
    name: str
    out_features: int   # N (rows of W)
    in_features: int    # K (cols of W)


@dataclass(frozen=True)
class Workload:
    index: int
    name: str
    tokens: int                      # T (0: quantize/dequantize only)
    linears: tuple
    rank: int = 0
    alpha: float = 0.0
    outliers: bool = False
    backward: bool = True


def _block(hidden: int, inter: int):
    return (Linear("q_proj", hidden, hidden), Linear("k_proj", hidden, hidden),
            Linear("v_proj", hidden, hidden), Linear("o_proj", hidden, hidden),
            Linear("gate_proj", inter, hidden), Linear("up_proj", inter, hidden),
            Linear("down_proj", hidden, inter))


WORKLOADS = {
    "single_1024": Workload(0, "single_1024", 512, (Linear("linear", 1024, 1024),),
                            rank=16, alpha=32.0),
    "attn_4096": Workload(1, "attn_4096", 4096, (Linear("attn_proj", 4096, 4096),),
                          rank=16, alpha=32.0, outliers=True),
    "block_7b": Workload(2, "block_7b", 8192, _block(4096, 11008), rank=64, alpha=16.0),
    "bulk_8192x22016": Workload(3, "bulk_8192x22016", 0,
                                (Linear("mlp", 8192, 22016),), outliers=True,
                                backward=False),
    # the bulk weight (same draws) with a rank-64 adapter, for the merge
    "merge_8192x22016": Workload(3, "merge_8192x22016", 0,
                                 (Linear("mlp", 8192, 22016),), rank=64, alpha=16.0,
                                 outliers=True, backward=False),
    "block_65b_decode": Workload(4, "block_65b_decode", 16, _block(8192, 22016),
                                 rank=64, alpha=16.0, backward=False),
    "block_65b_train": Workload(4, "block_65b_train", 2048, _block(8192, 22016),
                                rank=64, alpha=16.0),
}


def rng_for(seed: int, workload: int, linear: int, kind: int) -> np.random.Generator:
    return np.random.default_rng([seed, workload, linear, kind])


def weight(out_features: int, in_features: int, *, seed: int = 0, workload: int = 0,
           linear: int = 0, outliers: bool = False, std: float = 0.02) -> np.ndarray:
    """float32 [out, in] ~ N(0, std^2), optionally 0.1% of entries times 20."""
    rng = rng_for(seed, workload, linear, KIND_W)
    n = out_features * in_features
    w = rng.standard_normal(n, dtype=np.float32)
    w *= np.float32(std)
    if outliers:
        k = int(0.001 * n)
        idx = rng.choice(n, size=k, replace=False)
        w[idx] *= np.float32(20.0)
    return w.reshape(out_features, in_features)


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 (torch's CPU conversion, nearest even); uint16 bits."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def to_f16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to IEEE binary16 (torch's CPU conversion, nearest even); uint16 bits."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.float16)
    return t.view(torch.int16).numpy().view(np.uint16)


def to_16_bits(x: np.ndarray, dtype: str = "bf16") -> np.ndarray:
    """Round float32 to the 16-bit type "bf16" or "fp16"; uint16 bits."""
    return to_f16_bits(x) if dtype == "fp16" else to_bf16_bits(x)


def bf16_bits_value(bits: np.ndarray) -> np.ndarray:
    """float32 value of bf16 bit patterns (exact widening)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def bits16_value(bits: np.ndarray, dtype: str = "bf16") -> np.ndarray:
    """float32 value of 16-bit patterns of type "bf16" or "fp16" (exact widening)."""
    if dtype == "fp16":
        return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float32)
    return bf16_bits_value(bits)


def bf16_normal(shape, std: float, *, seed: int, workload: int, linear: int,
                kind: int, dtype: str = "bf16") -> np.ndarray:
    """16-bit patterns (bf16 unless dtype is "fp16") of N(0, std^2) draws."""
    rng = rng_for(seed, workload, linear, kind)
    x = rng.standard_normal(int(np.prod(shape)), dtype=np.float32).reshape(shape)
    if std != 1.0:
        x *= np.float32(std)
    return to_16_bits(x, dtype)


def linear_inputs(wl: Workload, li: int, *, seed: int = 0, tokens: int | None = None,
                  dtype: str = "bf16", with_weight: bool = True):
    """All inputs of linear `li` of workload `wl` (numpy; the 16-bit tensors as
    uint16 bit patterns of `dtype`, "bf16" or "fp16").  with_weight=False
    skips the float32 weight (every other draw is unchanged)."""
    lin = wl.linears[li]
    t = wl.tokens if tokens is None else tokens
    n, k, r = lin.out_features, lin.in_features, wl.rank
    out = {}
    if with_weight:
        out["w"] = weight(n, k, seed=seed, workload=wl.index, linear=li, outliers=wl.outliers)
    if r > 0:
        out["a"] = bf16_normal((r, k), float(np.sqrt(1.0 / r)), seed=seed, workload=wl.index,
                               linear=li, kind=KIND_A, dtype=dtype)
        out["b"] = bf16_normal((n, r), 0.01, seed=seed, workload=wl.index, linear=li, kind=KIND_B,
                               dtype=dtype)
    if t > 0:
        out["x"] = bf16_normal((t, k), 1.0, seed=seed, workload=wl.index, linear=li, kind=KIND_X,
                               dtype=dtype)
        if wl.backward:
            out["dy"] = bf16_normal((t, n), 1.0, seed=seed, workload=wl.index, linear=li,
                                    kind=KIND_DY, dtype=dtype)
    return out
