"""Pins of the oracle's training pair with a residual stream (forward that
stores and normalises h_new = x + u, backward that adds the residual-stream
gradient into dx), against the mathematics rather than against itself:

* hand-derived worked examples, including round-to-nearest-even ties of the
  sum in bf16 and in fp32 (tests/golden/hand_examples.json);
* the sum rounded by an independent route (IEEE fp32 addition in numpy, then
  an integer round-to-nearest-even onto bf16; correct because fp32 carries more
  than twice bf16's precision plus two bits) on random pairs with wide exponent
  gaps and on constructed ties;
* special cases: u = 0 reduces to the plain forward, the sum is symmetric in
  (x, u), g_residual = 0 reduces to the plain backward, dy = 0 gives
  dx_total = g_residual exactly and dw = 0;
* finite differences of L = sum g*y(x+u) + sum g_res*(x+u) with respect to x
  (inputs chosen so that every sum and perturbation is exact in fp32).

Definitions: FlashInfer commit #5741 'cake_rmsnorm_train' (quoted on the
FlashInfer PR #4480 page), API and Design: Forward / Backward."""
import json
import os

import numpy as np
import pytest

from workloads import to_bf16_bits

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_examples.json")


def _bits(vals, dtype):
    a = np.asarray(vals, np.float32).reshape(1, -1)
    return to_bf16_bits(a) if dtype == "bf16" else a


def _f64(a):
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def test_golden_forward_residual(oracle):
    for ex in json.load(open(GOLDEN))["fwd_residual"]:
        dt = ex["dtype"]
        x, u = _bits(ex["x"], dt), _bits(ex["u"], dt)
        assert np.array_equal(_f64(x)[0], np.asarray(ex["x"])), "example inputs must be exact in %s" % dt
        assert np.array_equal(_f64(u)[0], np.asarray(ex["u"])), "example inputs must be exact in %s" % dt
        w = _bits(ex["w"], dt)[0]
        y, rstd, h = oracle.rmsnorm_fwd_residual(x, u, w, ex["eps"])
        np.testing.assert_array_equal(_f64(h)[0], ex["h"])
        if "rstd" in ex:
            assert rstd[0] == pytest.approx(ex["rstd"], rel=1e-15, abs=0)
            np.testing.assert_allclose(y[0], ex["y"], rtol=1e-15, atol=1e-300)


def test_golden_backward_residual(oracle):
    for ex in json.load(open(GOLDEN))["bwd_residual"]:
        x, g, gr = (np.asarray(ex[k], np.float32).reshape(1, -1) for k in ("x", "g", "g_res"))
        w = np.asarray(ex["w"], np.float32)
        dx, dw = oracle.rmsnorm_bwd_residual(g, x, w, np.array([ex["rstd"]]), gr)
        np.testing.assert_allclose(dx[0], ex["dx"], rtol=1e-14, atol=1e-16)
        np.testing.assert_allclose(dw, ex["dw"], rtol=1e-14, atol=1e-16)


def _bf16_rne_from_f32(f):
    """Round fp32 values to bf16 bit patterns, ties to even, with integer arithmetic
    (finite inputs)."""
    u = np.ascontiguousarray(f, np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    return ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)


def test_bf16_sum_matches_fp32_add_then_round(oracle):
    rng = np.random.default_rng(21)
    n = 4096
    mag_x = rng.standard_normal(n) * np.exp2(rng.integers(-12, 12, n))
    mag_u = rng.standard_normal(n) * np.exp2(rng.integers(-30, 12, n))
    x = to_bf16_bits(mag_x.astype(np.float32)).reshape(64, 64)
    u = to_bf16_bits(mag_u.astype(np.float32)).reshape(64, 64)
    # constructed ties: x = 1 + k*2^-7, u = 2^-8 (sum halfway between two bf16 values)
    k = rng.integers(0, 127, 64)
    x[0] = to_bf16_bits((1 + k * 2.0 ** -7).astype(np.float32))
    u[0] = to_bf16_bits(np.full(64, 2.0 ** -8, np.float32))
    h = oracle.residual_add(x, u)
    ref = _bf16_rne_from_f32(_f64(x).astype(np.float32) + _f64(u).astype(np.float32))
    np.testing.assert_array_equal(h, ref)
    # the ties went to the even neighbour
    assert np.all((h[0] & 1) == 0)


def test_f32_sum_is_ieee_addition(oracle):
    rng = np.random.default_rng(22)
    x = (rng.standard_normal((32, 40)) * np.exp2(rng.integers(-20, 20, (32, 40)))).astype(np.float32)
    u = (rng.standard_normal((32, 40)) * np.exp2(rng.integers(-40, 20, (32, 40)))).astype(np.float32)
    h = oracle.residual_add(x, u)
    np.testing.assert_array_equal(h, x + u)


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_zero_residual_and_symmetry(oracle, dt):
    rng = np.random.default_rng(23)
    xf = rng.standard_normal((7, 48)).astype(np.float32)
    uf = rng.standard_normal((7, 48)).astype(np.float32)
    wf = (1 + 0.1 * rng.standard_normal(48)).astype(np.float32)
    conv = to_bf16_bits if dt == "bf16" else (lambda a: a)
    x, u, w = conv(xf), conv(uf), conv(wf)
    y0, r0 = oracle.rmsnorm_fwd(x, w, 1e-6)
    y1, r1, h1 = oracle.rmsnorm_fwd_residual(x, np.zeros_like(x), w, 1e-6)
    np.testing.assert_array_equal(h1, x)
    np.testing.assert_array_equal(y1, y0)
    np.testing.assert_array_equal(r1, r0)
    ya, ra, ha = oracle.rmsnorm_fwd_residual(x, u, w, 1e-6)
    yb, rb, hb = oracle.rmsnorm_fwd_residual(u, x, w, 1e-6)
    np.testing.assert_array_equal(ha, hb)
    np.testing.assert_array_equal(ya, yb)
    np.testing.assert_array_equal(ra, rb)
    # and the residual forward is the plain forward of the stored h_new
    yh, rh = oracle.rmsnorm_fwd(ha, w, 1e-6)
    np.testing.assert_array_equal(ya, yh)
    np.testing.assert_array_equal(ra, rh)


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_backward_residual_special_cases(oracle, dt):
    rng = np.random.default_rng(24)
    conv = to_bf16_bits if dt == "bf16" else (lambda a: a)
    h = conv(rng.standard_normal((9, 40)).astype(np.float32))
    g = conv(rng.standard_normal((9, 40)).astype(np.float32))
    gr = conv(rng.standard_normal((9, 40)).astype(np.float32))
    w = conv((1 + 0.1 * rng.standard_normal(40)).astype(np.float32))
    _, rstd = oracle.rmsnorm_fwd(h, w, 1e-6)
    dx0, dw0 = oracle.rmsnorm_bwd(g, h, w, rstd)
    dx1, dw1 = oracle.rmsnorm_bwd_residual(g, h, w, rstd, np.zeros_like(gr))
    np.testing.assert_array_equal(dx1, dx0)
    np.testing.assert_array_equal(dw1, dw0)
    dx2, dw2 = oracle.rmsnorm_bwd_residual(np.zeros_like(g), h, w, rstd, gr)
    np.testing.assert_array_equal(dx2, _f64(gr))
    np.testing.assert_array_equal(dw2, 0.0)
    dx3, dw3 = oracle.rmsnorm_bwd_residual(g, h, w, rstd, gr)
    np.testing.assert_array_equal(dw3, dw0)


def _richardson(fun, h):
    d1 = (fun(h) - fun(-h)) / (2 * h)
    d2 = (fun(h / 2) - fun(-h / 2)) / h
    return (4 * d2 - d1) / 3


def test_finite_differences_dx_total(oracle):
    """dx_total = dL/dx for L = sum g*y(x+u) + sum g_res*(x+u): the loss goes through the
    oracle's residual forward (rstd recomputed from the perturbed sum).  x and u are
    multiples of 2^-6 of modest size, so x + u and x +- h (h = 2^-8, 2^-9) are exact in fp32
    and h_new carries no rounding."""
    rng = np.random.default_rng(25)
    T, H, eps = 3, 6, 0.05
    x = (np.round(rng.standard_normal((T, H)) * 64) / 64).astype(np.float32)
    u = (np.round(rng.standard_normal((T, H)) * 64) / 64).astype(np.float32)
    w = (np.round((1 + 0.25 * rng.standard_normal(H)) * 64) / 64).astype(np.float32)
    g = rng.standard_normal((T, H)).astype(np.float32)
    gr = rng.standard_normal((T, H)).astype(np.float32)
    _, rstd, hnew = oracle.rmsnorm_fwd_residual(x, u, w, eps)
    np.testing.assert_array_equal(hnew.astype(np.float64), x.astype(np.float64) + u.astype(np.float64))
    dx, _ = oracle.rmsnorm_bwd_residual(g, hnew, w, rstd, gr)
    gd, grd = g.astype(np.float64), gr.astype(np.float64)

    def loss(xx):
        y, _, hh = oracle.rmsnorm_fwd_residual(xx, u, w, eps)
        return float((gd * y).sum() + (grd * hh.astype(np.float64)).sum())

    step = 2.0 ** -8
    for r in range(T):
        for j in range(H):
            def fx(d):
                xx = x.copy()
                xx[r, j] = np.float32(x[r, j] + d)
                assert float(xx[r, j]) == float(x[r, j]) + d
                return loss(xx)
            assert _richardson(fx, step) == pytest.approx(dx[r, j], rel=1e-7, abs=1e-9)


def test_strided_and_empty(oracle):
    rng = np.random.default_rng(26)
    bx = rng.standard_normal((4, 40)).astype(np.float32)
    bu = rng.standard_normal((4, 56)).astype(np.float32)
    w = np.ones(32, np.float32)
    yv, rv, hv = oracle.rmsnorm_fwd_residual(bx[:, 4:36], bu[:, 16:48], w, 1e-6)
    yc, rc, hc = oracle.rmsnorm_fwd_residual(np.ascontiguousarray(bx[:, 4:36]), np.ascontiguousarray(bu[:, 16:48]),
                                             w, 1e-6)
    np.testing.assert_array_equal(yv, yc)
    np.testing.assert_array_equal(hv, hc)
    y0, r0, h0 = oracle.rmsnorm_fwd_residual(np.zeros((0, 32), np.float32), np.zeros((0, 32), np.float32), w, 1e-6)
    assert y0.shape == (0, 32) and r0.shape == (0,) and h0.shape == (0, 32)
