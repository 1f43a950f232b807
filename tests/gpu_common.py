"""Helpers shared by the GPU parity tests: host <-> device transfer of the
workload arrays, and the comparison rules.

Tolerances (the readings recorded in the design notes):
  fp32 y / dx           |gpu - oracle_fp64| <= 1e-5 (absolute); in rows whose
                        largest |ref| is 10.5 or more (16 fp32 ulps of it exceed
                        1e-5) the bound is 16 ulps of that row maximum, 2^-20 * max
  bf16 y / dx / normed  |gpu - oracle_fp64| <= 5e-2 (absolute) where |ref| < 16;
                        from 16 on, where a correctly rounded bf16 value may
                        already be 0.0625 off, one bf16 spacing of the value;
                        and, as a quality check everywhere, within one bf16
                        spacing of the value plus 2^-20 of the row maximum
  rstd                  relative error <= 1e-5 (the Cake accuracy gate)
  dw                    every element within 1e-4 + 1e-4*|ref| of the FP64 sum
                        (miles-ext-kernels PR #15, Summary / Accuracy)
  residual, fp8 codes, block scales: bit-exact (codes and scales re-derived
                        by the oracle from the GPU's own bf16 normed values).
"""
import os
from concurrent.futures import ThreadPoolExecutor

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


BF16_ABS_RANGE = 16.0       # below it, 5e-2 is at least half a bf16 spacing
F32_ROW_ULPS = 2.0 ** -20   # 16 fp32 ulps of a row's largest magnitude


def check_values(name, got: np.ndarray, ref: np.ndarray, is_bf16: bool):
    """got: GPU output (uint16 bf16 bits or float32), ref: oracle FP64, same shape.
    Returns the largest absolute error."""
    g = as_f64(got)
    err = np.abs(g - ref)
    if not err.size:
        return 0.0
    absref = np.abs(ref)
    rowmax = np.max(absref, axis=-1, keepdims=True) if ref.ndim == 2 else np.max(absref)
    worst = float(err.max())
    if is_bf16:
        spacing = np.exp2(np.floor(np.log2(np.maximum(absref, 1e-30))) - 7)
        bound = np.where(absref < BF16_ABS_RANGE, BF16_TOL, spacing)
        over = err > bound
        assert not over.any(), "%s: %d values over the bound (first at %s: err %g, ref %g)" % (
            name, int(over.sum()), np.argwhere(over)[0], err[over][0], ref[over][0])
        # quality: within one bf16 spacing of the exact value (rounding plus fp32 noise)
        bad = err > spacing + 2.0 ** -20 * rowmax
        assert not bad.any(), "%s: %d values beyond one bf16 spacing (first at %s)" % (
            name, int(bad.sum()), np.argwhere(bad)[0])
    else:
        bound = np.maximum(F32_TOL, F32_ROW_ULPS * rowmax)
        over = err > bound
        assert not over.any(), "%s: %d values over the bound (first at %s: err %g, ref %g)" % (
            name, int(over.sum()), np.argwhere(over)[0], err[over][0], ref[over][0])
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


def worker_count() -> int:
    """Threads for host-side checking: the cores this process may run on, at most 16."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(n, 16))


def row_chunks(T: int, chunk: int):
    return [(lo, min(T, lo + chunk)) for lo in range(0, T, chunk)]


def over_row_chunks(T: int, chunk: int, fn):
    """fn(lo, hi) for consecutive row ranges covering [0, T), run on worker_count()
    threads (the oracle's C calls and numpy's array kernels release the GIL).
    Returns the results in row order."""
    with ThreadPoolExecutor(worker_count()) as ex:
        return list(ex.map(lambda c: fn(*c), row_chunks(T, chunk)))


def compare_all_rows(name, T, chunk, got_rows, ref_rows, is_bf16):
    """Every row of an output against the oracle: got_rows(lo, hi) is the GPU's rows,
    ref_rows(lo, hi) the oracle's FP64 values of the same rows.  Returns the largest
    absolute error."""
    def one(lo, hi):
        return check_values("%s rows %d..%d" % (name, lo, hi - 1), got_rows(lo, hi), ref_rows(lo, hi), is_bf16)
    return max(over_row_chunks(T, chunk, one), default=0.0)


def oracle_dw_chunked(oracle, dy, x, w, rstd64, chunk=8192):
    """The oracle's FP64 dw over all rows, computed on row chunks in parallel and summed
    over the chunks in row order (a different FP64 summation order than one sequential
    pass; both are within T * 2^-53 of the exact sum, far inside the dw budget)."""
    T = x.shape[0]

    def part(lo, hi):
        return oracle.rmsnorm_bwd(dy[lo:hi], x[lo:hi], w, rstd64[lo:hi], want_dx=False)[1]
    total = np.zeros(x.shape[1], np.float64)
    for p in over_row_chunks(T, chunk, part):
        total += p
    return total


def dw_budget_ratio(got: np.ndarray, ref: np.ndarray) -> float:
    """Worst element of |got - ref| / (1e-4 + 1e-4 |ref|)."""
    r = np.abs(got.astype(np.float64) - ref) / (1e-4 + 1e-4 * np.abs(ref))
    return float(r.max()) if r.size else 0.0


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


# ----------------------------------------------------------------------------
# edge rows for the backward (FlashInfer commit #5741 "cake_rmsnorm_train",
# Accuracy and tests: zero rows, a single extreme row, input scales 1e-3 and
# 1e3, strided rows)
# ----------------------------------------------------------------------------
EDGE_KINDS = ("zero", "const", "negconst", "tiny", "huge", "extreme", "sub_eps", "zero_dy", "big_dy")


def edge_inputs(T, H, seed, scale=1.0):
    """fp32 x and dy [T, H] ~ N(0,1) (x times `scale`) with edge rows planted at the
    first, middle and last rows, cycling through EDGE_KINDS:
      zero      x = 0 (rstd = 1/sqrt(eps), |dx| ~ 1e3)
      const     x = 3 (normalises to w)       negconst  x = -0.5
      tiny      x * 1e-3                      huge      x * 1e3
      extreme   one element of x set to 3e4   sub_eps   x * 1e-20 (mean square << eps)
      zero_dy   dy = 0 (dx = 0)               big_dy    dy * 1e3
    Returns (x, dy, {row: kind})."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, H), dtype=np.float32) * np.float32(scale)
    dy = rng.standard_normal((T, H), dtype=np.float32)
    where = sorted({0, 1, 2, 3, T // 3, T // 2, T // 2 + 1, T - 4, T - 3, T - 2, T - 1} & set(range(T)))
    kinds = {}
    for i, r in enumerate(where):
        k = EDGE_KINDS[i % len(EDGE_KINDS)]
        kinds[r] = k
        if k == "zero":
            x[r] = 0.0
        elif k == "const":
            x[r] = 3.0
        elif k == "negconst":
            x[r] = -0.5
        elif k == "tiny":
            x[r] *= np.float32(1e-3)
        elif k == "huge":
            x[r] *= np.float32(1e3)
        elif k == "extreme":
            x[r, 7 % H] = 3e4
        elif k == "sub_eps":
            x[r] *= np.float32(1e-20)
        elif k == "zero_dy":
            dy[r] = 0.0
        elif k == "big_dy":
            dy[r] *= np.float32(1e3)
    return x, dy, kinds


def strided_dev(a: np.ndarray, ld: int) -> torch.Tensor:
    """A host [T, H] array in a device buffer of row stride ld (elements); the padding
    holds a NaN pattern, so a kernel that read it would spoil its row.  Returns the
    [T, H] view."""
    T, H = a.shape
    dt = torch_dtype(a)
    if dt == torch.bfloat16:
        buf = torch.full((T, ld), SENTINEL_BF16, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    else:
        buf = torch.full((T, ld), float("nan"), dtype=dt, device="cuda")
    view = buf[:, :H]
    view.copy_(to_dev(a))
    return view
