"""Seeded random shapes through the C ABI against the oracle.

Row counts, row widths, dtypes and row padding are drawn at random within each
entry point's limits (one fixed seed per op, so the cases are the same on every
run and named by their shapes), beyond the hand-picked cases of the other parity
tests: every launch policy the shapes select runs, with the comparison rules and
the guard bands around every output that those tests use.
"""
import numpy as np
import pytest

from gpu_common import check_dw, check_rstd, check_values
from gpu_ops import (check_fp8, check_variant, gpu_bwd, gpu_bwd_res, gpu_fp8, gpu_fwd, gpu_fwd_res, lp16,
                     make_fused, run_heads, run_variant)
from workloads import Workload, generate, to_bf16_bits

pytestmark = pytest.mark.gpu

N_CASES = 24
ELEMENT_BUDGET = 6_000_000        # T * H per case, so that the oracle stays fast


def _rows(rng, H):
    """Half the draws log-uniform over [1, tmax] (few-row launches), half uniform over
    [tmax/4, tmax] (runs over many windows with a ragged last one)."""
    tmax = max(1, min(20000, ELEMENT_BUDGET // H))
    if rng.random() < 0.5:
        return max(1, int(np.exp(rng.uniform(0.0, np.log(tmax)))))
    return max(1, int(rng.integers(max(1, tmax // 4), tmax + 1)))


def _row_cases(op, seed):
    """(T, H, x dtype, w dtype, row padding in elements) for the forward or the backward."""
    rng = np.random.default_rng(seed)
    cases = []
    for _ in range(N_CASES):
        xd = "f32" if rng.random() < 0.25 else "bf16"
        wd = "f32" if xd == "f32" or rng.random() < 0.3 else "bf16"
        e = 4 if xd == "f32" else 8                    # elements per 16-byte vector
        hmax = {"fwd": {"bf16": 32768, "f32": 16384}, "bwd": {"bf16": 16384, "f32": 8192}}[op][xd]
        H = max(e, int(np.exp(rng.uniform(np.log(e), np.log(hmax)))) // e * e)
        pad = int(rng.choice([0, 0, 0, e, 2 * e, 64]))
        cases.append((_rows(rng, H), H, xd, wd, pad))
    return cases


def _fp8_cases(seed):
    """(T, H, row padding in elements) for the producer: H a multiple of 128; the padding
    is shared by the 1-byte codes, whose row stride must stay a 16-byte multiple."""
    rng = np.random.default_rng(seed)
    cases = []
    for _ in range(N_CASES):
        H = 128 * max(1, int(np.exp(rng.uniform(0.0, np.log(256)))))
        pad = int(rng.choice([0, 0, 16, 64]))
        cases.append((_rows(rng, H), H, pad))
    return cases


FWD_RANDOM = _row_cases("fwd", 71)
BWD_RANDOM = _row_cases("bwd", 72)
FP8_RANDOM = _fp8_cases(73)
FRES_RANDOM = _row_cases("fwd", 74)        # the residual pair has the plain ops' limits
BRES_RANDOM = _row_cases("bwd", 75)


def _heads_cases(seed):
    """(T, heads, head_dim, dtype, w dtype, head stride, band offset, token stride), strides and
    offsets in elements and 16-byte multiples; head_dim up to 128 vectors."""
    rng = np.random.default_rng(seed)
    cases = []
    for _ in range(N_CASES):
        xd = "f32" if rng.random() < 0.25 else "bf16"
        wd = "f32" if xd == "f32" or rng.random() < 0.3 else "bf16"
        e = 4 if xd == "f32" else 8
        D = max(e, int(np.exp(rng.uniform(np.log(e), np.log(128 * e)))) // e * e)
        nh = max(1, int(np.exp(rng.uniform(0.0, np.log(1000 if rng.random() < 0.15 else 64)))))
        ldh = D + e * int(rng.choice([0, 0, 1, 2]))
        off = e * int(rng.choice([0, 0, 1, 8]))
        ldt = off + (nh - 1) * ldh + D + e * int(rng.choice([0, 0, 1, 4]))
        T = _rows(rng, nh * D)
        cases.append((T, nh, D, xd, wd, ldh, off, ldt))
    return cases


HEADS_RANDOM = _heads_cases(76)


def _variant_cases(seed):
    """(T, H, row padding, row dtype, code format, per-tensor scale or None, normed written)."""
    rng = np.random.default_rng(seed)
    cases = []
    for (T, H, pad) in _fp8_cases(seed):
        dtype = str(rng.choice(["bf16", "f16"]))
        fmt = str(rng.choice(["e4m3", "e5m2"]))
        ts = None
        if rng.random() < 0.5:        # a given per-tensor scale, log-uniform around the codes' range
            top = 448.0 if fmt == "e4m3" else 57344.0
            ts = float(np.float32(np.exp2(rng.uniform(-4.0, 4.0)) * 4.0 / top))
        cases.append((T, H, pad, dtype, fmt, ts, bool(rng.random() < 0.7)))
    return cases


VARIANT_RANDOM = _variant_cases(77)


def _ids(cases):
    return ["T%d-H%d-%s" % (c[0], c[1], "-".join(str(v) for v in c[2:])) for c in cases]


@pytest.fixture(scope="module")
def rn():
    import bwd_fp8_block_amd as m
    return m


@pytest.mark.parametrize("T,H,xd,wd,pad", FWD_RANDOM, ids=_ids(FWD_RANDOM))
def test_fwd_random_shapes(rn, oracle, T, H, xd, wd, pad):
    d = generate(Workload("fwd", T, H, xd, wd, seed=7100 + T + H))
    y, rstd = gpu_fwd(rn, d["x"], d["w"], 1e-6, ld_pad=pad)
    yref, rref = oracle.rmsnorm_fwd(d["x"], d["w"], 1e-6)
    check_rstd(rstd, rref)
    check_values("y", y, yref, xd == "bf16")


@pytest.mark.parametrize("k", range(N_CASES), ids=_ids(BWD_RANDOM))
def test_bwd_random_shapes(rn, oracle, k):
    T, H, xd, wd, pad = BWD_RANDOM[k]
    d = generate(Workload("bwd", T, H, xd, wd, seed=7200 + T + H))
    _, rstd = gpu_fwd(rn, d["x"], d["w"], 1e-6)
    dx, dw = gpu_bwd(rn, d["dy"], d["x"], d["w"], rstd, k % 2 == 0, ld_pad=pad, poison=True)
    dxref, dwref = oracle.rmsnorm_bwd(d["dy"], d["x"], d["w"], rstd.astype(np.float64))
    check_values("dx", dx, dxref, xd == "bf16")
    check_dw(dw, dwref)


@pytest.mark.parametrize("T,H,pad", FP8_RANDOM, ids=_ids(FP8_RANDOM))
def test_fp8_random_shapes(rn, oracle, T, H, pad):
    d = generate(Workload("fp8", T, H, "bf16", "bf16", residual=True, seed=7300 + T + H))
    h, out, scale, normed = gpu_fp8(rn, d["x"], d["residual"], d["w"], 1e-6, ld_pad=pad, scale_pad=4)
    check_fp8(oracle, d["x"], d["residual"], d["w"], 1e-6, h, out, scale, normed)


@pytest.mark.parametrize("T,H,xd,wd,pad", FRES_RANDOM, ids=_ids(FRES_RANDOM))
def test_fwd_residual_random_shapes(rn, oracle, T, H, xd, wd, pad):
    d = generate(Workload("fres", T, H, xd, wd, residual=True, seed=7400 + T + H))
    y, h, rstd = gpu_fwd_res(rn, d["x"], d["residual"], d["w"], 1e-6, ld_pad=pad)
    yref, rref, href = oracle.rmsnorm_fwd_residual(d["x"], d["residual"], d["w"], 1e-6)
    assert np.array_equal(h, href), "h_new not bit-exact"
    check_rstd(rstd, rref)
    check_values("y", y, yref, xd == "bf16")


@pytest.mark.parametrize("T,H,xd,wd,pad", BRES_RANDOM, ids=_ids(BRES_RANDOM))
def test_bwd_residual_random_shapes(rn, oracle, T, H, xd, wd, pad):
    d = generate(Workload("bres", T, H, xd, wd, residual=True, g_residual=True, seed=7500 + T + H))
    _, h, rstd = gpu_fwd_res(rn, d["x"], d["residual"], d["w"], 1e-6)
    dx, dw = gpu_bwd_res(rn, d["dy"], h, d["w"], rstd, d["g_residual"], ld_pad=pad, poison=True)
    dxref, dwref = oracle.rmsnorm_bwd_residual(d["dy"], h, d["w"], rstd.astype(np.float64), d["g_residual"])
    check_values("dx_total", dx, dxref, xd == "bf16")
    check_dw(dw, dwref)


@pytest.mark.parametrize("T,nh,D,xd,wd,ldh,off,ldt", HEADS_RANDOM, ids=_ids(HEADS_RANDOM))
def test_heads_random_shapes(rn, oracle, T, nh, D, xd, wd, ldh, off, ldt):
    host = make_fused(T, ldt, xd, 7600 + T + nh + D)
    rng = np.random.default_rng(7700 + D)
    w = (1 + 0.1 * rng.standard_normal(D)).astype(np.float32)
    w = to_bf16_bits(w) if wd == "bf16" else w
    y, rstd, after = run_heads(rn, host, nh, D, ldh, off, w, 1e-6)
    assert np.array_equal(after, host), "input modified"
    yref, rref = oracle.rmsnorm_fwd_heads(np.ascontiguousarray(host[:, off:]), nh, D, w, 1e-6, ld_head=ldh)
    check_rstd(rstd.reshape(-1), rref.reshape(-1))
    check_values("y", y.reshape(T * nh, D), yref.reshape(T * nh, D), xd == "bf16")


@pytest.mark.parametrize("T,H,pad,dtype,fmt,ts,with_normed", VARIANT_RANDOM, ids=_ids(VARIANT_RANDOM))
def test_variant_random_shapes(rn, oracle, T, H, pad, dtype, fmt, ts, with_normed):
    rng = np.random.default_rng(7800 + T + H)
    x = lp16(rng.standard_normal((T, H)), dtype)
    res = lp16(rng.standard_normal((T, H)), dtype)
    w = lp16(1 + 0.1 * rng.standard_normal(H), dtype)
    h, out, scale, normed = run_variant(rn, x, res, w, dtype, fmt, ts, ld_pad=pad)
    check_variant(oracle, x, res, w, dtype, fmt, ts, h, out, scale, normed)
    if not with_normed:
        # without normed_out the codes and scales are those of the call that writes it
        h2, out2, scale2, n2 = run_variant(rn, x, res, w, dtype, fmt, ts, with_normed=False, ld_pad=pad)
        assert n2 is None and np.array_equal(h2, h) and np.array_equal(out2, out)
        if scale is not None:
            assert np.array_equal(scale2[:, :T].view(np.uint32), scale[:, :T].view(np.uint32))
