"""Pins of the oracle's RMSNorm forward and backward against the mathematics,
not against itself:

* hand-derived worked examples (tests/golden/hand_examples.json);
* closed forms: constant rows normalise to sign(c)*w,
  H = 1 forward and backward in closed form;
* invariants: scale invariance at eps = 0, sum_j (y_j/w_j)^2 = H*ms/(ms+eps),
  sum_j dx_j*x_j = eps*rstd^3*sum_j g_j*w_j*x_j;
* finite differences (Richardson-extrapolated central differences of
  L = sum g*y computed through the oracle's own forward) for dx and dw;
* dW as an exactly rounded sum (math.fsum of products that are exact in FP64).

Definitions: FlashInfer commit #5741 'cake_rmsnorm_train' (quoted on the
FlashInfer PR #4480 page), Design: Forward and Backward, Accuracy (the eager
dw = (g*x*rstd).sum(0))."""
import json
import math
import os

import numpy as np
import pytest

from workloads import to_bf16_bits

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_examples.json")


def f32(a):
    return np.ascontiguousarray(np.asarray(a, dtype=np.float32).reshape(1, -1) if np.ndim(a) == 1 else a,
                                dtype=np.float32)


def test_golden_forward(oracle):
    for ex in json.load(open(GOLDEN))["fwd"]:
        x = f32(ex["x"])
        w = np.asarray(ex["w"], np.float32)
        y, rstd = oracle.rmsnorm_fwd(x, w, ex["eps"])
        assert rstd[0] == pytest.approx(ex["rstd"], rel=1e-15, abs=0)
        np.testing.assert_allclose(y[0], ex["y"], rtol=1e-15, atol=1e-300)


def test_golden_backward(oracle):
    for ex in json.load(open(GOLDEN))["bwd"]:
        x, g = f32(ex["x"]), f32(ex["g"])
        w = np.asarray(ex["w"], np.float32)
        dx, dw = oracle.rmsnorm_bwd(g, x, w, np.array([ex["rstd"]]))
        np.testing.assert_allclose(dx[0], ex["dx"], rtol=1e-14, atol=1e-16)
        np.testing.assert_allclose(dw, ex["dw"], rtol=1e-14, atol=1e-16)


@pytest.mark.parametrize("c", [1.0, -3.0, 1e-3, 250.0, -0.5])
@pytest.mark.parametrize("eps", [0.0, 1e-6, 0.5])
def test_constant_row_normalises_to_sign_times_w(oracle, c, eps):
    H = 24
    x = np.full((2, H), c, np.float32)
    w = (1 + 0.1 * np.random.default_rng(4).standard_normal(H)).astype(np.float32)
    y, rstd = oracle.rmsnorm_fwd(x, w, eps)
    cf = float(np.float32(c))
    r = 1.0 / math.sqrt(cf * cf + float(np.float32(eps)))
    np.testing.assert_allclose(rstd, r, rtol=1e-15)
    np.testing.assert_allclose(y, np.broadcast_to(cf * r * w.astype(np.float64), y.shape), rtol=1e-15)
    if eps == 0.0:
        np.testing.assert_allclose(y, np.broadcast_to(math.copysign(1.0, c) * w.astype(np.float64), y.shape),
                                   rtol=1e-15)


def test_h1_closed_forms(oracle):
    rng = np.random.default_rng(5)
    for _ in range(20):
        xv, wv, gv = (float(np.float32(v)) for v in rng.standard_normal(3))
        eps = float(np.float32(rng.uniform(1e-3, 1)))
        y, rstd = oracle.rmsnorm_fwd(f32([xv]), np.array([wv], np.float32), eps)
        assert y[0, 0] == pytest.approx(xv / math.sqrt(xv * xv + eps) * wv, rel=1e-14)
        dx, dw = oracle.rmsnorm_bwd(f32([gv]), f32([xv]), np.array([wv], np.float32), rstd)
        # d/dx [x (x^2+eps)^-1/2] = eps (x^2+eps)^-3/2
        assert dx[0, 0] == pytest.approx(gv * wv * eps * (xv * xv + eps) ** -1.5, rel=1e-12)
        assert dw[0] == pytest.approx(gv * xv / math.sqrt(xv * xv + eps), rel=1e-14)


def test_scale_invariance_at_eps0(oracle):
    rng = np.random.default_rng(6)
    x = rng.standard_normal((5, 40)).astype(np.float32)
    w = (1 + 0.1 * rng.standard_normal(40)).astype(np.float32)
    g = rng.standard_normal((5, 40)).astype(np.float32)
    y1, r1 = oracle.rmsnorm_fwd(x, w, 0.0)
    for a in (4.0, 0.125, 2.0 ** 20):      # powers of two: the scaled input is exact in fp32
        xa = (x * np.float32(a)).astype(np.float32)
        ya, ra = oracle.rmsnorm_fwd(xa, w, 0.0)
        np.testing.assert_allclose(ya, y1, rtol=1e-15)
        dx1, _ = oracle.rmsnorm_bwd(g, x, w, r1)
        dxa, _ = oracle.rmsnorm_bwd(g, xa, w, ra)
        np.testing.assert_allclose(dxa * a, dx1, rtol=1e-12, atol=1e-15)


def test_sum_of_squares_identity(oracle):
    rng = np.random.default_rng(7)
    for eps in (0.0, 1e-6, 0.3):
        x = rng.standard_normal((6, 33)).astype(np.float32)
        w = (1 + 0.1 * rng.standard_normal(33)).astype(np.float32)
        y, _ = oracle.rmsnorm_fwd(x, w, eps)
        ms = (x.astype(np.float64) ** 2).mean(axis=1)
        lhs = ((y / w.astype(np.float64)[None, :]) ** 2).sum(axis=1)
        np.testing.assert_allclose(lhs, 33 * ms / (ms + float(np.float32(eps))), rtol=1e-13)


def test_dx_orthogonality_invariant(oracle):
    rng = np.random.default_rng(8)
    for eps in (0.0, 1e-6, 0.7):
        x = rng.standard_normal((4, 16)).astype(np.float32)
        w = (1 + 0.1 * rng.standard_normal(16)).astype(np.float32)
        g = rng.standard_normal((4, 16)).astype(np.float32)
        _, rstd = oracle.rmsnorm_fwd(x, w, eps)
        dx, _ = oracle.rmsnorm_bwd(g, x, w, rstd)
        xd, gd, wd = x.astype(np.float64), g.astype(np.float64), w.astype(np.float64)
        lhs = (dx * xd).sum(axis=1)
        rhs = float(np.float32(eps)) * rstd ** 3 * (gd * wd[None, :] * xd).sum(axis=1)
        np.testing.assert_allclose(lhs, rhs, rtol=1e-9, atol=1e-13)


def _richardson(fun, h):
    d1 = (fun(h) - fun(-h)) / (2 * h)
    d2 = (fun(h / 2) - fun(-h / 2)) / h
    return (4 * d2 - d1) / 3


def test_finite_differences_dx_dw(oracle):
    """dx and dw equal dL/dx and dL/dw of L = sum g*y, with y from the oracle's forward
    (rstd recomputed from the perturbed x).  Inputs are multiples of 2^-6 so every
    perturbation x +- h (h = 2^-8, 2^-9) is exact in fp32."""
    rng = np.random.default_rng(9)
    T, H, eps = 3, 7, 0.05
    x = (np.round(rng.standard_normal((T, H)) * 64) / 64).astype(np.float32)
    w = (np.round((1 + 0.25 * rng.standard_normal(H)) * 64) / 64).astype(np.float32)
    g = rng.standard_normal((T, H)).astype(np.float32)
    _, rstd = oracle.rmsnorm_fwd(x, w, eps)
    dx, dw = oracle.rmsnorm_bwd(g, x, w, rstd)
    gd = g.astype(np.float64)

    def loss(xx, ww):
        y, _ = oracle.rmsnorm_fwd(xx, ww, eps)
        return float((gd * y).sum())

    h = 2.0 ** -8
    for r in range(T):
        for j in range(H):
            def fx(d):
                xx = x.copy()
                xx[r, j] = np.float32(x[r, j] + d)
                assert float(xx[r, j]) == float(x[r, j]) + d
                return loss(xx, w)
            assert _richardson(fx, h) == pytest.approx(dx[r, j], rel=1e-7, abs=1e-9)
    for j in range(H):
        def fw(d):
            ww = w.copy()
            ww[j] = np.float32(w[j] + d)
            assert float(ww[j]) == float(w[j]) + d
            return loss(x, ww)
        assert _richardson(fw, h) == pytest.approx(dw[j], rel=1e-9, abs=1e-12)


def test_dw_is_exactly_rounded_sum_for_bf16(oracle):
    """For bf16 g, x and fp32 rstd every product g*x*rstd is exact in FP64
    (8 + 8 + 24 significant bits), so math.fsum gives the correctly rounded dw."""
    rng = np.random.default_rng(10)
    T, H = 300, 24
    xb = to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32) * 3)
    gb = to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    w = to_bf16_bits((1 + 0.1 * rng.standard_normal(H)).astype(np.float32))
    _, rstd64 = oracle.rmsnorm_fwd(xb, w, 1e-6)
    rstd = rstd64.astype(np.float32).astype(np.float64)          # the fp32 rstd a kernel stores
    _, dw = oracle.rmsnorm_bwd(gb, xb, w, rstd, want_dx=False)
    xv = xb.astype(np.uint32) << 16
    gv = gb.astype(np.uint32) << 16
    xf = xv.view(np.float32).astype(np.float64)
    gf = gv.view(np.float32).astype(np.float64)
    for j in range(H):
        terms = gf[:, j] * xf[:, j] * rstd
        assert np.all(terms == gf[:, j] * xf[:, j] * rstd)
        # recursive summation bound: |err| <= (T-1) * 2^-53 * sum |terms|
        bound = (T - 1) * 2.0 ** -53 * float(np.abs(terms).sum())
        assert abs(dw[j] - math.fsum(terms)) <= bound


def test_strided_rows_and_empty(oracle):
    rng = np.random.default_rng(11)
    base = rng.standard_normal((5, 48)).astype(np.float32)
    w = np.ones(32, np.float32)
    y_view, r_view = oracle.rmsnorm_fwd(base[:, 8:40], w, 1e-6)
    y_copy, r_copy = oracle.rmsnorm_fwd(np.ascontiguousarray(base[:, 8:40]), w, 1e-6)
    np.testing.assert_array_equal(y_view, y_copy)
    np.testing.assert_array_equal(r_view, r_copy)
    y0, r0 = oracle.rmsnorm_fwd(np.zeros((0, 32), np.float32), w, 1e-6)
    assert y0.shape == (0, 32) and r0.shape == (0,)
    _, dw0 = oracle.rmsnorm_bwd(np.zeros((0, 32), np.float32), np.zeros((0, 32), np.float32), w,
                                np.zeros(0))
    np.testing.assert_array_equal(dw0, 0.0)
