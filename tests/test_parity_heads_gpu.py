"""Parity of the per-head RMSNorm (QK-norm, rmsnorm_fwd_heads) through the
C ABI against the FP64 CPU oracle: the q and k bands of a fused QKV
projection, padded head strides, in-place use on the fused buffer (every
value outside the normalised band must come back unchanged), optional rstd,
and the bf16 T=8192, 32 heads x 128 workload at full size."""
import numpy as np
import pytest
import torch

from gpu_common import as_f64, check_rstd, check_values, compare_all_rows, to_dev, to_host
from gpu_ops import heads_view, make_fused, run_heads
from workloads import CONFIGS, generate, to_bf16_bits

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def rn():
    import bwd_fp8_block_amd as m
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return m



HEADS_CASES = [
    # T, heads, head_dim, dtype, w dtype, head stride, band offset (elements), token stride
    (37, 32, 128, "bf16", "bf16", 128, 0, 3 * 32 * 128),            # q band of a fused projection
    (37, 8, 128, "bf16", "bf16", 128, 32 * 128, 48 * 128),          # k band (GQA: 32 q, 8 k, 8 v heads)
    (5, 4, 64, "f32", "f32", 80, 16, 4 * 80 + 32),                  # padded heads, offset band
    (300, 16, 256, "bf16", "f32", 256, 0, 16 * 256),
    (9, 3, 512, "bf16", "bf16", 520, 8, 3 * 520 + 8),
    (7, 2, 1024, "bf16", "bf16", 1024, 0, 2048),
    (64, 24, 8, "bf16", "bf16", 8, 0, 24 * 8),
    (1, 1, 64, "bf16", "bf16", 64, 0, 64),
    (3000, 2, 120, "bf16", "bf16", 128, 0, 256),
    (11, 6, 512, "f32", "f32", 512, 0, 3072),
    (4099, 7, 128, "bf16", "bf16", 128, 0, 7 * 128),                # many rows: token = row / heads
    (1500, 40, 128, "bf16", "bf16", 136, 64, 40 * 136 + 64),
    # the widest heads (1024 bf16 / 512 fp32 values) and the narrowest, over many rows
    (2000, 4, 1024, "bf16", "bf16", 1024, 0, 4 * 1024), (1700, 3, 512, "f32", "f32", 520, 4, 3 * 520 + 8),
    (3001, 48, 8, "bf16", "f32", 8, 0, 48 * 8),
    # many heads per token (the token of a row is found by a multiply and a shift)
    (50, 1000, 8, "bf16", "bf16", 8, 0, 8000), (301, 127, 16, "bf16", "bf16", 24, 8, 127 * 24 + 8),
]


@pytest.mark.parametrize("T,nh,D,xd,wd,ldh,off,ldt", HEADS_CASES)
def test_heads_parity(rn, oracle, T, nh, D, xd, wd, ldh, off, ldt):
    host = make_fused(T, ldt, xd, 6000 + T + nh + D)
    rng = np.random.default_rng(6100 + D)
    w = (1 + 0.1 * rng.standard_normal(D)).astype(np.float32)
    w = to_bf16_bits(w) if wd == "bf16" else w
    y, rstd, after = run_heads(rn, host, nh, D, ldh, off, w, 1e-6)
    assert np.array_equal(after, host), "input modified"
    yref, rref = oracle.rmsnorm_fwd_heads(np.ascontiguousarray(host[:, off:]), nh, D, w, 1e-6, ld_head=ldh)
    check_rstd(rstd.reshape(-1), rref.reshape(-1))
    check_values("y", y.reshape(T * nh, D), yref.reshape(T * nh, D), xd == "bf16")


@pytest.mark.parametrize("band", [0, 1])
def test_heads_in_place_on_fused_buffer(rn, oracle, band):
    """Normalise the q (or k) band of a fused [T, 3*heads*128] buffer in place: the band
    matches the out-of-place result bit for bit and nothing else in the buffer changes."""
    T, nh, D = 33, 8, 128
    ldt = 3 * nh * D
    host = make_fused(T, ldt, "bf16", 6200 + band)
    w = to_bf16_bits((1 + 0.1 * np.random.default_rng(6201).standard_normal(D)).astype(np.float32))
    off = band * nh * D
    y0, r0, _ = run_heads(rn, host, nh, D, D, off, w, 1e-6)
    y1, r1, after = run_heads(rn, host, nh, D, D, off, w, 1e-6, in_place=True)
    assert np.array_equal(y1, y0) and np.array_equal(r1, r0)
    outside = np.ones(host.shape, bool)
    outside[:, off: off + nh * D] = False
    assert np.array_equal(after[outside], host[outside]), "values outside the band changed"
    assert np.array_equal(after[:, off: off + nh * D].reshape(T, nh, D), y0)


def test_heads_edge_rows(rn, oracle):
    """Heads of zeros (rstd = 1/sqrt(eps), y = 0), constant heads (y = sign * w), heads scaled by
    1e-3 and 1e3, a head below eps and one extreme element, spread over tokens and head slots."""
    T, nh, D = 40, 8, 128
    rng = np.random.default_rng(6400)
    a = rng.standard_normal((T, nh, D)).astype(np.float32)
    a[0, 0] = 0.0
    a[1, 7] = 2.5
    a[2, 3] = -0.75
    a[3, 1] *= 1e-3
    a[T - 1, 5] *= 1e3
    a[T // 2, 2] *= 1e-20
    a[T // 2 + 1, 6, 17] = 3e4
    host = to_bf16_bits(a.reshape(T, nh * D))
    w = to_bf16_bits((1 + 0.1 * rng.standard_normal(D)).astype(np.float32))
    y, rstd, _ = run_heads(rn, host, nh, D, D, 0, w, 1e-6)
    yref, rref = oracle.rmsnorm_fwd_heads(host, nh, D, w, 1e-6)
    check_rstd(rstd.reshape(-1), rref.reshape(-1))
    check_values("y", y.reshape(T * nh, D), yref.reshape(T * nh, D), True)
    y3 = y.reshape(T, nh, D)
    assert np.all((y3[0, 0] & 0x7FFF) == 0)
    np.testing.assert_allclose(as_f64(y3[1, 7]), as_f64(w), rtol=2 ** -7)


def test_heads_without_rstd(rn, oracle):
    T, nh, D = 19, 4, 128
    host = make_fused(T, nh * D, "bf16", 6300)
    w = to_bf16_bits(np.ones(D, np.float32))
    y, _, _ = run_heads(rn, host, nh, D, D, 0, w, 1e-6, with_rstd=False)
    yref, _ = oracle.rmsnorm_fwd_heads(host, nh, D, w, 1e-6)
    check_values("y", y.reshape(-1, D), yref.reshape(-1, D), True)


def test_heads_empty(rn):
    x = torch.empty(0, 4, 128, dtype=torch.bfloat16, device="cuda")
    rn.rmsnorm_fwd_heads(x, torch.ones(128, dtype=torch.bfloat16, device="cuda"), torch.empty_like(x), None, 1e-6)


def test_config_qk_norm(rn, oracle):
    """bf16 T=8192 tokens of a fused [T, 3*32*128] projection: the q band and the k band
    (separate weights) at full size; rstd and every token's y in full."""
    wl = CONFIGS["qk_bf16_T8192_32x128"]
    d = generate(wl)
    T, D = wl.T, 128
    nh = wl.H // D // 3
    full = to_dev(d["x"])
    for band in (0, 1):
        w = np.ascontiguousarray(d["w"][band * D:(band + 1) * D])
        x = heads_view(full, T, nh, D, wl.H, D, band * nh * D)
        y = torch.empty(T, nh, D, dtype=torch.bfloat16, device="cuda")
        rstd = torch.empty(T * nh, dtype=torch.float32, device="cuda")
        rn.rmsnorm_fwd_heads(x, to_dev(w), y, rstd, wl.eps)
        band_host = np.ascontiguousarray(d["x"][:, band * nh * D:(band + 1) * nh * D])
        _, rref = oracle.rmsnorm_fwd_heads(band_host, nh, D, w, wl.eps, want_y=False)
        check_rstd(to_host(rstd), rref.reshape(-1))
        yh = to_host(y)
        compare_all_rows("y band %d" % band, T, 1024, lambda lo, hi: yh[lo:hi].reshape(-1, D),
                         lambda lo, hi: oracle.rmsnorm_fwd_heads(band_host[lo:hi], nh, D, w, wl.eps)[0].reshape(-1, D),
                         True)
