"""Seeded synthetic inputs for the N:M sparse GEMM workloads.

This module only draws random numbers and rounds them to the storage type.
It holds none of the method's arithmetic (no pruning, packing or products),
so both the CPU oracle's tests and the GPU path's tests, bench and smoke run
draw their inputs from here.

Recipe (the same everywhere):
  * generator: numpy PCG64 seeded with the sequence [workload_id, tensor_id,
    variant]; tensor_id 0 = weight W, 1 = activations, 2 = permutation,
    3 = hybrid tile flags, 4 = output gradient G (training products),
    5 = kept-block mask, 6 = diagonal offsets;
  * W, activations and G: float32 standard normal times sigma, then rounded to
    the storage type with round-to-nearest-even (fp16 through numpy's cast,
    bf16 through the bit routine below);
  * permutation: a uniform random permutation of 0..K-1 (int32);
  * tile flags: each tile dense (1) when a uniform draw is below the given
    fraction, else 2:4 (0);
  * block mask: each 32 x 32 block kept (1) when a uniform draw is below the
    kept fraction;
  * diagonal offsets: D distinct offsets drawn uniformly from 0..K-1 without
    replacement (int32, in the order drawn).

Half-precision arrays are returned as their raw uint16 bit patterns, the form
every consumer (oracle, C ABI) takes.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

F16 = "f16"
BF16 = "bf16"
I8 = "i8"
F8 = "f8e4m3"


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns, round to nearest, ties to even.

    Standard bias-and-truncate method: add 0x7FFF plus the lowest kept bit,
    then drop the low 16 bits.  Inputs here are finite normals (no NaN).
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    return ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)


def f32_to_f16_bits(x: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(x, dtype=np.float32).astype(np.float16).view(np.uint16)


def to_half_bits(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == F16:
        return f32_to_f16_bits(x)
    if dtype == BF16:
        return f32_to_bf16_bits(x)
    raise ValueError(f"unknown half dtype {dtype!r}")


def rng_for(workload_id: int, tensor_id: int, variant: int = 0) -> np.random.Generator:
    return np.random.default_rng([int(workload_id), int(tensor_id), int(variant)])


def normal_half(shape, sigma: float, dtype: str, workload_id: int, tensor_id: int,
                variant: int = 0) -> np.ndarray:
    """uint16 bits of N(0, sigma^2) samples rounded to `dtype`."""
    rng = rng_for(workload_id, tensor_id, variant)
    x = rng.standard_normal(size=shape, dtype=np.float32) * np.float32(sigma)
    return to_half_bits(x, dtype)


def integer_half(shape, lo: int, hi: int, dtype: str, workload_id: int, tensor_id: int,
                 variant: int = 0) -> np.ndarray:
    """uint16 bits of uniform integers in [lo, hi] (exact in fp16 and bf16)."""
    rng = rng_for(workload_id, tensor_id, variant)
    x = rng.integers(lo, hi + 1, size=shape).astype(np.float32)
    return to_half_bits(x, dtype)


def normal_i8(shape, scale: float, workload_id: int, tensor_id: int, variant: int = 0) -> np.ndarray:
    """int8 samples of N(0, 1) * scale, rounded to nearest and clipped to [-128, 127]
    (a symmetric per-tensor quantisation of normal data; many small magnitudes,
    so many ties)."""
    rng = rng_for(workload_id, tensor_id, variant)
    x = rng.standard_normal(size=shape, dtype=np.float32) * np.float32(scale)
    return np.clip(np.rint(x), -128, 127).astype(np.int8)


def normal_fp8(shape, scale: float, workload_id: int, tensor_id: int, variant: int = 0) -> np.ndarray:
    """uint8 OCP E4M3 bit patterns of N(0, 1) * scale, saturated to +-448 and
    rounded to nearest even by torch's float8_e4m3fn conversion."""
    import torch
    rng = rng_for(workload_id, tensor_id, variant)
    x = np.clip(rng.standard_normal(size=shape, dtype=np.float32) * np.float32(scale), -448.0, 448.0)
    return torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def block_mask(grid_shape, keep_fraction: float, workload_id: int, variant: int = 0) -> np.ndarray:
    """uint8 mask over a grid of 32 x 32 weight blocks: 1 (kept) with probability keep_fraction."""
    rng = rng_for(workload_id, 5, variant)
    return (rng.random(grid_shape) < keep_fraction).astype(np.uint8)


def diag_offsets(K: int, D: int, workload_id: int, variant: int = 0) -> np.ndarray:
    """D distinct diagonal offsets in [0, K), int32, in the order drawn."""
    rng = rng_for(workload_id, 6, variant)
    return rng.choice(int(K), size=int(D), replace=False).astype(np.int32)


def tile_flags(tile_grid_shape, dense_fraction: float, workload_id: int, variant: int = 0) -> np.ndarray:
    """uint8 flags over a grid of weight tiles: 1 (dense) with probability dense_fraction."""
    rng = rng_for(workload_id, 3, variant)
    return (rng.random(tile_grid_shape) < dense_fraction).astype(np.uint8)


def random_permutation(k: int, workload_id: int, variant: int = 0) -> np.ndarray:
    return rng_for(workload_id, 2, variant).permutation(int(k)).astype(np.int32)


@dataclass(frozen=True)
class Workload:
    """One synthetic workload: W is R x K, activations are T x K (K-contiguous)."""
    wid: int
    name: str
    R: int
    K: int
    Ts: tuple
    patterns: tuple  # (n, m) pairs
    dtype: str
    sigma_w: float
    sigma_x: float = 1.0
    permuted: bool = False
    note: str = ""
    hybrid: tuple = ()  # (tile_rows, tile_cols, dense fraction) for hybrid dense / 2:4 tiles
    train: bool = False  # the training-side products (dX, dW) of the layer
    host: tuple = ()  # ("block", kept fraction) or ("diag", D): the permutation on another structure

    def weights(self) -> np.ndarray:
        if self.dtype == I8:
            return normal_i8((self.R, self.K), self.sigma_w, self.wid, 0)
        if self.dtype == F8:
            return normal_fp8((self.R, self.K), self.sigma_w, self.wid, 0)
        return normal_half((self.R, self.K), self.sigma_w, self.dtype, self.wid, 0)

    def activations(self, T: int | None = None) -> np.ndarray:
        T = self.Ts[0] if T is None else T
        if self.dtype == I8:
            return normal_i8((T, self.K), self.sigma_x, self.wid, 1, T)
        if self.dtype == F8:
            return normal_fp8((T, self.K), self.sigma_x, self.wid, 1, T)
        return normal_half((T, self.K), self.sigma_x, self.dtype, self.wid, 1, T)

    def gradient(self, T: int | None = None) -> np.ndarray:
        """G = dL/dY in the forward output's [T, R] layout, N(0, 1) in the weight type."""
        T = self.Ts[0] if T is None else T
        return normal_half((T, self.R), 1.0, self.dtype, self.wid, 4, T)

    def permutation(self) -> np.ndarray | None:
        return random_permutation(self.K, self.wid) if self.permuted else None

    def block_mask(self) -> np.ndarray:
        return block_mask((self.R // 32, self.K // 32), self.host[1], self.wid)

    def diag_offsets(self) -> np.ndarray:
        return diag_offsets(self.K, self.host[1], self.wid)

    def tile_flags(self) -> np.ndarray:
        tr, tc, frac = self.hybrid
        return tile_flags((-(-self.R // tr), self.K // tc), frac, self.wid)


# The workloads (sizes R x K x T).  Shapes follow the layers the pages
# measure: a small 2:4 example, a LLaMA-2-7B projection at prefill and at
# decode, the general 1:4 / 1:8 forms, a ViT-B/16 MLP fc1 over 64 images of
# 197 tokens with a learned column permutation, the prefill shape in INT8 and
# in FP8 E4M3, the prefill shape with hybrid dense / 2:4 tiles, the prefill
# shape's training-side products, and the permuted ViT layer on a block-sparse
# and a diagonal-sparse weight at 90% sparsity.
WORKLOADS = {
    1: Workload(1, "small-2of4-fp16", 256, 256, (64,), ((2, 4),), F16, 1.0,
                note="2:4 fp16 small case"),
    2: Workload(2, "llama2-7b-proj-prefill-2of4-bf16", 4096, 4096, (2048,), ((2, 4),), BF16, 0.02,
                note="2:4 bf16 prefill, MFMA-bound"),
    3: Workload(3, "llama2-7b-mlp-decode-2of4-bf16", 11008, 4096, (1, 8, 16), ((2, 4),), BF16, 0.02,
                note="2:4 bf16 decode, HBM-bound"),
    4: Workload(4, "general-1of4-1of8-fp16", 4096, 4096, (512,), ((1, 4), (1, 8)), F16, 1.0,
                note="1:4 and 1:8 fp16"),
    5: Workload(5, "vit-b16-fc1-perm-2of4-fp16", 3072, 768, (12608,), ((2, 4),), F16, 0.02,
                permuted=True, note="2:4 fp16 with column permutation, 197 tokens x 64 images"),
    # INT8 2:4 (the pages chart INT8 sparse GEMMs against dense ones) at the
    # prefill projection's shape; weights and activations quantised normal data
    6: Workload(6, "int8-2of4-prefill", 4096, 4096, (2048,), ((2, 4),), I8, 32.0, 32.0,
                note="INT8 2:4, int32 output"),
    # the same shape in OCP FP8 E4M3 (an 8-bit float in the one-byte layout)
    7: Workload(7, "fp8-e4m3-2of4-prefill", 4096, 4096, (2048,), ((2, 4),), F8, 1.0, 1.0,
                note="FP8 E4M3 2:4, fp32 output"),
    # hybrid dense / 2:4 tiles (PATCH) at the prefill projection's shape: 128 x
    # 128 tiles, half of them (seeded at random) dense, so 25% of W is zero
    8: Workload(8, "llama2-7b-proj-prefill-hybrid-tiles-bf16", 4096, 4096, (2048,), ((2, 4),), BF16, 0.02,
                note="hybrid dense / 2:4 128x128 tiles, half dense", hybrid=(128, 128, 0.5)),
    # the training-side products of the prefill projection (retraining with the
    # 2:4 pattern held): dX = G W_nm and the packed dW, G [2048, 4096] N(0, 1)
    9: Workload(9, "llama2-7b-proj-backward-2of4-bf16", 4096, 4096, (2048,), ((2, 4),), BF16, 0.02,
                note="2:4 bf16 dX and packed dW", train=True),
    # the permutation on two other host structures (SHUFFLESPARSE's ViT-B/16
    # setting at 90% sparsity): 10% of the 32 x 32 blocks kept, or 77 of 768
    # diagonals (10% of each row), activations read through a permutation
    10: Workload(10, "vit-b16-fc1-perm-block-fp16", 3072, 768, (12608,), ((2, 4),), F16, 0.02,
                 permuted=True, note="block-sparse 32x32, 10% kept, with column permutation",
                 host=("block", 0.1)),
    11: Workload(11, "vit-b16-fc1-perm-diag-fp16", 3072, 768, (12608,), ((2, 4),), F16, 0.02,
                 permuted=True, note="diagonal-sparse, 77 of 768 diagonals, with column permutation",
                 host=("diag", 77)),
}
