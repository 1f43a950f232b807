"""Helpers shared by the GPU parity tests: host <-> device transfer of the
workload arrays, and the comparison rules.

Tolerances (the readings recorded in the design notes):
  fp32 y / dx           |gpu - oracle_fp64| <= 1e-5 (absolute)
  bf16 y / dx / normed  |gpu - oracle_fp64| <= 5e-2 (absolute), and, as a
                        quality check, within one bf16 spacing of the value
  rstd                  relative error <= 1e-5 (the Cake accuracy gate)
  dw                    every element within 1e-4 + 1e-4*|ref| of the FP64 sum
                        (miles-ext-kernels PR #15, Summary / Accuracy)
  residual, fp8 codes, block scales: bit-exact (codes and scales re-derived
                        by the oracle from the GPU's own bf16 normed values).
"""
import numpy as np
import torch

F32_TOL = 1e-5
BF16_TOL = 5e-2


def to_dev(a: np.ndarray) -> torch.Tensor:
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def to_host(t: torch.Tensor) -> np.ndarray:
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.float8_e4m3fn:
        return t.view(torch.uint8).numpy()
    return t.numpy()


def as_f64(a: np.ndarray) -> np.ndarray:
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def torch_dtype(a: np.ndarray):
    return torch.bfloat16 if a.dtype == np.uint16 else torch.float32


def check_values(name, got: np.ndarray, ref: np.ndarray, is_bf16: bool):
    """got: GPU output (uint16 bf16 bits or float32), ref: oracle FP64, same shape."""
    g = as_f64(got)
    err = np.abs(g - ref)
    if is_bf16:
        worst = float(err.max()) if err.size else 0.0
        assert worst <= BF16_TOL, "%s: max abs err %g > %g" % (name, worst, BF16_TOL)
        # quality: within one bf16 spacing of the exact value (rounding plus fp32 noise)
        scale = np.maximum(np.abs(ref), 1e-30)
        spacing = np.exp2(np.floor(np.log2(scale)) - 7)
        rowmax = np.max(np.abs(ref), axis=-1, keepdims=True) if ref.ndim == 2 else np.max(np.abs(ref))
        bad = err > spacing + 2.0 ** -20 * rowmax
        assert not bad.any(), "%s: %d values beyond one bf16 spacing (first at %s)" % (
            name, int(bad.sum()), np.argwhere(bad)[0])
    else:
        worst = float(err.max()) if err.size else 0.0
        assert worst <= F32_TOL, "%s: max abs err %g > %g" % (name, worst, F32_TOL)
    return worst


def check_rstd(got: np.ndarray, ref: np.ndarray):
    rel = np.abs(got.astype(np.float64) - ref) / np.abs(ref)
    worst = float(rel.max()) if rel.size else 0.0
    assert worst <= 1e-5, "rstd: max rel err %g" % worst
    return worst


def check_dw(got: np.ndarray, ref: np.ndarray):
    ratio = np.abs(got.astype(np.float64) - ref) / (1e-4 + 1e-4 * np.abs(ref))
    worst = float(ratio.max()) if ratio.size else 0.0
    assert worst <= 1.0, "dw: worst element at %g of the budget (index %d)" % (worst, int(np.argmax(ratio)))
    return worst


def sample_rows(T: int, n: int = 48, seed: int = 0):
    rng = np.random.default_rng(seed)
    rows = {0, T - 1, T // 2, max(T - 2, 0), min(1, T - 1)}
    rows.update(rng.choice(T, size=min(n, T), replace=False).tolist())
    return np.array(sorted(r for r in rows if 0 <= r < T), dtype=np.int64)


SENTINEL_BF16 = 0x7FBF      # a NaN pattern no kernel writes


def guarded_matrix(T, H, dtype, ld=None, guard=64):
    """A [T, ld] buffer plus guard elements on both sides, filled with a sentinel.
    Returns (full flat tensor, [T, H] view with row stride ld)."""
    ld = ld or H
    n = guard + T * ld + guard
    if dtype == torch.bfloat16:
        full = torch.full((n,), SENTINEL_BF16, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    elif dtype == torch.uint8:
        full = torch.full((n,), 0xA5, dtype=torch.uint8, device="cuda")
    else:
        full = torch.full((n,), float("nan"), dtype=dtype, device="cuda")
    view = full[guard: guard + T * ld].view(T, ld)[:, :H] if T > 0 else full[guard:guard].view(0, H)
    return full, view


def assert_guards(full: torch.Tensor, T, H, ld, guard=64, name="out"):
    """The guard bands (and the row padding beyond column H) still hold the sentinel."""
    h = to_host(full)
    if full.dtype == torch.bfloat16:
        sent = lambda a: a == SENTINEL_BF16
    elif full.dtype == torch.uint8:
        sent = lambda a: a == 0xA5
    else:
        sent = lambda a: np.isnan(a)
    assert sent(h[:guard]).all() and sent(h[guard + T * ld:]).all(), "%s: guard band overwritten" % name
    if ld > H and T > 0:
        body = h[guard: guard + T * ld].reshape(T, ld)
        assert sent(body[:, H:]).all(), "%s: row padding overwritten" % name
