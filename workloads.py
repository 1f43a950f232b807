"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module holds no arithmetic of the method: it draws random numbers
(numpy PCG64) and rounds them to the storage dtype (round-to-nearest-even
fp32 -> bf16, done by torch's CPU cast).  Both the HIP path and the CPU oracle
receive the same arrays from here.

Arrays are numpy: float32, or uint16 holding bf16 bit patterns.

Workloads follow the shapes and distributions of the activations in the
pages' training and inference benchmarks: rows of hidden size 256 .. 7168,
T up to 65536, x and dY standard normal, weight 1 + 0.1 * N(0, 1).
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np
import torch

SEED_BASE = 20261202


def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 array -> uint16 bf16 bit patterns (round to nearest even)."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _cast(a: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return np.ascontiguousarray(a, dtype=np.float32)
    if dtype == "bf16":
        return to_bf16_bits(a)
    raise ValueError(dtype)


@dataclass
class Workload:
    name: str
    T: int
    H: int
    x_dtype: str          # "f32" | "bf16"
    w_dtype: str          # "f32" | "bf16"
    eps: float = 1e-6
    x_std: float = 1.0
    outlier_frac: float = 0.0
    outlier_scale: float = 50.0
    residual: bool = False
    g_residual: bool = False
    seed: int = SEED_BASE


def generate(wl: Workload):
    """Draw x, w, dy (and residual, g_residual) for a workload.

    Draw order is x, w, dy, residual, g_residual from one PCG64 stream seeded with
    ``wl.seed``.  Outlier rows (a fraction ``outlier_frac`` of T, chosen by a
    seeded permutation) are multiplied by ``outlier_scale`` in fp32 before the
    cast to the storage dtype."""
    rng = np.random.Generator(np.random.PCG64(wl.seed))
    T, H = wl.T, wl.H
    x = rng.standard_normal((T, H), dtype=np.float32)
    if wl.x_std != 1.0:
        x *= np.float32(wl.x_std)
    w = (1.0 + 0.1 * rng.standard_normal((H,), dtype=np.float32)).astype(np.float32)
    dy = rng.standard_normal((T, H), dtype=np.float32)
    res = rng.standard_normal((T, H), dtype=np.float32) if wl.residual else None
    gres = rng.standard_normal((T, H), dtype=np.float32) if wl.g_residual else None
    if wl.outlier_frac > 0.0 and T > 0:
        n_out = int(round(wl.outlier_frac * T))
        perm = np.random.Generator(np.random.PCG64(wl.seed + 1)).permutation(T)[:n_out]
        x[np.sort(perm)] *= np.float32(wl.outlier_scale)
    out = dict(x=_cast(x, wl.x_dtype), w=_cast(w, wl.w_dtype), dy=_cast(dy, wl.x_dtype))
    if res is not None:
        out["residual"] = _cast(res, wl.x_dtype)
    if gres is not None:
        out["g_residual"] = _cast(gres, wl.x_dtype)
    return out


# The parity workloads at full size (the benchmark shape of the fused producer last).
CONFIGS = {
    "f32_T64_H256": Workload("f32_T64_H256", 64, 256, "f32", "f32", seed=SEED_BASE + 100),
    "bf16_T8192_H4096": Workload("bf16_T8192_H4096", 8192, 4096, "bf16", "bf16", seed=SEED_BASE + 200),
    "bf16_T58497_H2048_outliers_f32w": Workload("bf16_T58497_H2048_outliers_f32w", 58497, 2048, "bf16", "f32",
                                              x_std=2.0, outlier_frac=0.01, outlier_scale=50.0,
                                              seed=SEED_BASE + 300),
    "fp8_T4096_H7168": Workload("fp8_T4096_H7168", 4096, 7168, "bf16", "bf16", residual=True,
                                   seed=SEED_BASE + 400),
    "bf16_T65536_H5120_f32w": Workload("bf16_T65536_H5120_f32w", 65536, 5120, "bf16", "f32", seed=SEED_BASE + 500),
    "fp8_T8192_H4096": Workload("fp8_T8192_H4096", 8192, 4096, "bf16", "bf16", residual=True,
                                seed=SEED_BASE + 600),
    # the training pair with a residual stream (x, u, dy, g_residual all standard normal)
    "res_bf16_T8192_H4096": Workload("res_bf16_T8192_H4096", 8192, 4096, "bf16", "bf16", residual=True,
                                     g_residual=True, seed=SEED_BASE + 700),
    # per-head RMSNorm (QK-norm): a fused [T, 3 * 32 * 128] bf16 QKV projection output; the q and k
    # weights are w[:128] and w[128:256]
    "qk_bf16_T8192_32x128": Workload("qk_bf16_T8192_32x128", 8192, 3 * 32 * 128, "bf16", "bf16",
                                     seed=SEED_BASE + 800),
}
