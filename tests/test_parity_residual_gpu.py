"""Parity of the training pair with a residual stream (rmsnorm_fwd_residual,
rmsnorm_bwd_residual) through the C ABI against the FP64 CPU oracle.

h_new is compared bit for bit; y, dx_total, rstd and dw to the same
tolerances as the plain pair.  In-place forms (h_out = x, h_out = u,
g_residual = dx) must give the same bits as the out-of-place calls.  The
bf16 T=8192 H=4096 workload is checked at full size, every row, in the launch
configuration the benchmark times."""
import numpy as np
import pytest
import torch

from gpu_common import (as_f64, assert_guards, check_dw, check_rstd, check_values, compare_all_rows, edge_inputs,
                        guarded_matrix, strided_dev, to_dev, to_host, torch_dtype)
from gpu_ops import gpu_bwd_res, gpu_fwd_res
from workloads import CONFIGS, Workload, generate, to_bf16_bits

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def rn():
    import bwd_fp8_block_amd as m
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return m



RES_FWD_CASES = [
    # T, H, x dtype, w dtype, row padding (elements)
    (64, 256, "f32", "f32", 0), (1, 8, "bf16", "bf16", 0), (7, 120, "bf16", "bf16", 8), (63, 512, "bf16", "f32", 0),
    (65, 1000, "bf16", "bf16", 64), (129, 2048, "bf16", "f32", 0), (257, 4096, "bf16", "bf16", 0),
    (33, 5120, "bf16", "f32", 16), (17, 7168, "bf16", "bf16", 0), (9, 8200, "bf16", "bf16", 0),
    (5, 16384, "bf16", "bf16", 0), (3, 16384, "f32", "f32", 0), (2, 32768, "bf16", "bf16", 0),
    (1000, 128, "bf16", "bf16", 0), (300, 3072, "bf16", "bf16", 0),
    # the widest rows over many windows
    (1200, 32768, "bf16", "bf16", 0), (700, 16384, "f32", "f32", 0),
]


@pytest.mark.parametrize("T,H,xd,wd,pad", RES_FWD_CASES)
def test_fwd_residual_parity(rn, oracle, T, H, xd, wd, pad):
    d = generate(Workload("fres", T, H, xd, wd, residual=True, seed=4000 + T + H))
    y, h, rstd = gpu_fwd_res(rn, d["x"], d["residual"], d["w"], 1e-6, ld_pad=pad)
    yref, rref, href = oracle.rmsnorm_fwd_residual(d["x"], d["residual"], d["w"], 1e-6)
    assert np.array_equal(h, href), "h_new not bit-exact"
    check_rstd(rstd, rref)
    check_values("y", y, yref, xd == "bf16")


@pytest.mark.parametrize("where", ["x", "u"])
@pytest.mark.parametrize("T,H,xd,wd", [(37, 1024, "bf16", "bf16"), (19, 768, "f32", "f32")])
def test_fwd_residual_in_place(rn, T, H, xd, wd, where):
    d = generate(Workload("fres_ip", T, H, xd, wd, residual=True, seed=4100 + T))
    y0, h0, r0 = gpu_fwd_res(rn, d["x"], d["residual"], d["w"], 1e-6)
    y1, h1, r1 = gpu_fwd_res(rn, d["x"], d["residual"], d["w"], 1e-6, inplace=where)
    assert np.array_equal(h1, h0) and np.array_equal(y1, y0)
    assert np.array_equal(r1.view(np.uint32), r0.view(np.uint32))


def test_fwd_residual_cancelling_rows(rn, oracle):
    """u = -x gives h_new = 0 and y = 0 exactly; u = 0 gives the plain forward's bits."""
    from workloads import to_bf16_bits
    T, H = 6, 2048
    rng = np.random.default_rng(41)
    x = to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    w = to_bf16_bits((1 + 0.1 * rng.standard_normal(H)).astype(np.float32))
    u = x ^ np.uint16(0x8000)
    u[3:] = 0
    y, h, rstd = gpu_fwd_res(rn, x, u, w, 1e-6)
    assert np.all((h[:3] & 0x7FFF) == 0) and np.all((y[:3] & 0x7FFF) == 0)
    xd, wd = to_dev(x[3:]), to_dev(w)
    yp = torch.empty_like(xd)
    rp = torch.empty(T - 3, dtype=torch.float32, device="cuda")
    rn.rmsnorm_fwd(xd, wd, yp, rp, 1e-6)
    assert np.array_equal(to_host(yp), y[3:]) and np.array_equal(to_host(rp), rstd[3:])
    yref, rref, href = oracle.rmsnorm_fwd_residual(x, u, w, 1e-6)
    assert np.array_equal(h, href)
    check_rstd(rstd, rref)
    check_values("y", y, yref, True)


RES_BWD_CASES = [
    (64, 256, "f32", "f32", 0), (1, 8, "bf16", "bf16", 0), (7, 120, "bf16", "bf16", 8), (63, 512, "bf16", "f32", 0),
    (65, 1000, "bf16", "bf16", 64), (127, 1024, "f32", "f32", 0), (129, 2048, "bf16", "f32", 0),
    (257, 4096, "bf16", "bf16", 0), (300, 5120, "bf16", "f32", 16), (31, 7168, "bf16", "bf16", 0),
    (5, 16384, "bf16", "bf16", 0), (4, 8192, "f32", "f32", 0), (2000, 256, "bf16", "bf16", 0),
    # rows of 513 .. 1024 chunks: two vectors per lane, three row buffers, many windows
    (3001, 7168, "bf16", "bf16", 0), (2003, 4096, "f32", "f32", 8),
    # rows wider than 1024 chunks over many windows
    (2500, 16384, "bf16", "bf16", 0), (1000, 8192, "f32", "f32", 0),
]


@pytest.mark.parametrize("T,H,xd,wd,pad", RES_BWD_CASES)
def test_bwd_residual_parity(rn, oracle, T, H, xd, wd, pad):
    d = generate(Workload("bres", T, H, xd, wd, residual=True, g_residual=True, seed=5000 + T + H))
    _, h, rstd = gpu_fwd_res(rn, d["x"], d["residual"], d["w"], 1e-6)
    dx, dw = gpu_bwd_res(rn, d["dy"], h, d["w"], rstd, d["g_residual"], ld_pad=pad)
    dxref, dwref = oracle.rmsnorm_bwd_residual(d["dy"], h, d["w"], rstd.astype(np.float64), d["g_residual"])
    check_values("dx_total", dx, dxref, xd == "bf16")
    check_dw(dw, dwref)


@pytest.mark.parametrize("T,H,xd,wd", [(300, 2048, "bf16", "f32"), (33, 1024, "f32", "f32")])
def test_bwd_residual_in_place_and_plain_dw(rn, T, H, xd, wd):
    """g_residual = dx in place gives the same bits; dw equals the plain backward's bits."""
    d = generate(Workload("bres_ip", T, H, xd, wd, residual=True, g_residual=True, seed=5100 + T))
    _, h, rstd = gpu_fwd_res(rn, d["x"], d["residual"], d["w"], 1e-6)
    dx0, dw0 = gpu_bwd_res(rn, d["dy"], h, d["w"], rstd, d["g_residual"])
    dx1, dw1 = gpu_bwd_res(rn, d["dy"], h, d["w"], rstd, d["g_residual"], inplace=True, poison=True)
    assert np.array_equal(dx1, dx0)
    assert np.array_equal(dw1.view(np.uint32), dw0.view(np.uint32))
    dyd, hd, wdev = to_dev(d["dy"]), to_dev(h), to_dev(d["w"])
    rd = torch.from_numpy(np.ascontiguousarray(rstd)).cuda()
    dxp = torch.empty_like(hd)
    dwp = torch.empty(H, dtype=torch.float32, device="cuda")
    ws = torch.empty(rn.rmsnorm_bwd_workspace_bytes(T, H) // 4, dtype=torch.float32, device="cuda")
    rn.rmsnorm_bwd(dyd, hd, wdev, rd, dxp, dwp, deterministic=True, workspace=ws)
    assert np.array_equal(to_host(dwp).view(np.uint32), dw0.view(np.uint32))


@pytest.mark.parametrize("T,H,xd,wd,ld,in_place", [
    (128, 4096, "bf16", "bf16", 8192, False), (255, 1024, "f32", "f32", 2048, True),
    (16231, 2048, "bf16", "f32", 2048, True), (16172, 7168, "bf16", "bf16", 7168, False),
    (4, 4096, "bf16", "bf16", 4096, False)])
def test_bwd_residual_edge_rows(rn, oracle, T, H, xd, wd, ld, in_place):
    """The residual backward over the edge rows of h_new (zero, constant, x * 1e-3 / 1e3, below
    eps, one extreme element, dy = 0, dy * 1e3), strided rows, g_residual with its own zero and
    huge rows, out of place and accumulating in place into dx; every row and dw element."""
    seed = 5900 + T + H
    h32, dy32, kinds = edge_inputs(T, H, seed)
    rng = np.random.default_rng(seed + 2)
    g32 = rng.standard_normal((T, H), dtype=np.float32)
    g32[T // 2] = 0.0
    g32[T - 1] *= np.float32(1e3)
    w = (1 + 0.1 * rng.standard_normal(H)).astype(np.float32)
    cast = to_bf16_bits if xd == "bf16" else (lambda a: a)
    h, dy, g = cast(h32), cast(dy32), cast(g32)
    w = to_bf16_bits(w) if wd == "bf16" else w
    hdev, dydev, wdev = strided_dev(h, ld), strided_dev(dy, ld), to_dev(w)
    dt = torch_dtype(h)
    rstd = torch.empty(T, dtype=torch.float32, device="cuda")
    rn.rmsnorm_fwd(hdev, wdev, torch.empty(T, H, dtype=dt, device="cuda"), rstd, 1e-6)
    rh = to_host(rstd)
    dxfull, dx = guarded_matrix(T, H, dt, ld)
    if in_place:
        dx.copy_(to_dev(g))
        gdev = dx
    else:
        gdev = strided_dev(g, ld)
    dw = torch.empty(H, dtype=torch.float32, device="cuda")
    nbytes = rn.rmsnorm_bwd_workspace_bytes(T, H)
    ws = torch.full((max(nbytes // 4, 1),), float("nan"), device="cuda") if nbytes else None
    rn.rmsnorm_bwd_residual(dydev, hdev, wdev, rstd, gdev, dx, dw, deterministic=True, workspace=ws)
    torch.cuda.synchronize()
    assert_guards(dxfull, T, H, ld, name="dx")
    dxh = to_host(dx)
    r64 = rh.astype(np.float64)
    compare_all_rows("dx_total", T, 2048, lambda lo, hi: dxh[lo:hi],
                     lambda lo, hi: oracle.rmsnorm_bwd_residual(dy[lo:hi], h[lo:hi], w, r64[lo:hi], g[lo:hi],
                                                                want_dw=False)[0], xd == "bf16")
    _, dwref = oracle.rmsnorm_bwd(dy, h, w, r64, want_dx=False)
    check_dw(to_host(dw), dwref)
    for r, k in kinds.items():
        if k == "zero_dy":                          # dx_total is g_residual, exactly
            assert np.array_equal(as_f64(dxh[r]), as_f64(g[r])), "dy = 0 must give dx_total = g_residual"


def test_residual_empty(rn):
    H = 256
    e = torch.empty(0, H, dtype=torch.bfloat16, device="cuda")
    w = torch.ones(H, dtype=torch.bfloat16, device="cuda")
    r0 = torch.empty(0, dtype=torch.float32, device="cuda")
    rn.rmsnorm_fwd_residual(e, e.clone(), w, e.clone(), e.clone(), r0, 1e-6)
    dw = torch.full((H,), 7.0, device="cuda")
    rn.rmsnorm_bwd_residual(e, e.clone(), w, r0, e.clone(), e.clone(), dw, deterministic=True, workspace=None)
    torch.cuda.synchronize()
    assert torch.all(dw == 0)


def test_residual_validation(rn):
    T, H = 4, 256
    x = torch.randn(T, H, device="cuda").to(torch.bfloat16)
    u = torch.randn(T, H, device="cuda").to(torch.bfloat16)
    w = torch.ones(H, dtype=torch.bfloat16, device="cuda")
    y = torch.full((T, H), 3.0, dtype=torch.bfloat16, device="cuda")
    rstd = torch.full((T,), 5.0, device="cuda")
    big = torch.zeros(2 * T * H, dtype=torch.bfloat16, device="cuda")
    xa = big[:T * H].view(T, H)
    ha = big[8 * 64: 8 * 64 + T * H].view(T, H)            # overlaps x without being x
    xa.copy_(x)
    with pytest.raises(rn.RNError) as e:
        rn.rmsnorm_fwd_residual(xa, u, w, y, ha, rstd, 1e-6)
    assert e.value.status == 7
    with pytest.raises(rn.RNError) as e:                    # h_out overlaps y
        rn.rmsnorm_fwd_residual(x, u, w, y, y, rstd, 1e-6)
    assert e.value.status == 7
    torch.cuda.synchronize()
    assert torch.all(y == 3.0) and torch.all(rstd == 5.0)
    dx = torch.zeros_like(x)
    dw = torch.full((H,), 9.0, device="cuda")
    ws = torch.empty(rn.rmsnorm_bwd_workspace_bytes(T, H) // 4, dtype=torch.float32, device="cuda")
    gpart = big[64: 64 + T * H].view(T, H)
    dxa = big[:T * H].view(T, H)
    with pytest.raises(rn.RNError) as e:                    # g_residual overlaps dx without being dx
        rn.rmsnorm_bwd_residual(x, u, w, rstd, gpart, dxa, dw, deterministic=True, workspace=ws)
    assert e.value.status == 7
    torch.cuda.synchronize()
    assert torch.all(dw == 9.0)


def test_config_residual_pair(rn, oracle):
    """The bf16 T=8192 H=4096 training pair with a residual at full size: h_new in full
    (bit-exact), rstd and dw in full, every row of y and dx_total; dw repeatable."""
    wl = CONFIGS["res_bf16_T8192_H4096"]
    d = generate(wl)
    T, H = wl.T, wl.H
    xd, ud, wd = to_dev(d["x"]), to_dev(d["residual"]), to_dev(d["w"])
    y = torch.empty_like(xd)
    h = torch.empty_like(xd)
    rstd = torch.empty(T, dtype=torch.float32, device="cuda")
    rn.rmsnorm_fwd_residual(xd, ud, wd, y, h, rstd, wl.eps)
    hh, rh = to_host(h), to_host(rstd)
    assert np.array_equal(hh, oracle.residual_add(d["x"], d["residual"])), "h_new not bit-exact"
    _, rref = oracle.rmsnorm_fwd(hh, d["w"], wl.eps, want_y=False)
    check_rstd(rh, rref)
    yh = to_host(y)
    compare_all_rows("y", T, 2048, lambda lo, hi: yh[lo:hi],
                     lambda lo, hi: oracle.rmsnorm_fwd(hh[lo:hi], d["w"], wl.eps)[0], True)
    del y, yh, xd, ud

    dyd, gd = to_dev(d["dy"]), to_dev(d["g_residual"])
    dx = torch.empty_like(h)
    dw = torch.empty(H, dtype=torch.float32, device="cuda")
    ws = torch.empty(rn.rmsnorm_bwd_workspace_bytes(T, H) // 4, dtype=torch.float32, device="cuda")
    _, dwref = oracle.rmsnorm_bwd(d["dy"], hh, d["w"], rh.astype(np.float64), want_dx=False)
    dws = []
    for rep in range(2):
        ws.fill_(float("nan"))
        rn.rmsnorm_bwd_residual(dyd, h, wd, rstd, gd, dx, dw, deterministic=True, workspace=ws)
        dws.append(to_host(dw).copy())
    check_dw(dws[0], dwref)
    assert np.array_equal(dws[1].view(np.uint32), dws[0].view(np.uint32))
    dxh = to_host(dx)
    r64 = rh.astype(np.float64)
    compare_all_rows("dx_total", T, 2048, lambda lo, hi: dxh[lo:hi],
                     lambda lo, hi: oracle.rmsnorm_bwd_residual(d["dy"][lo:hi], hh[lo:hi], d["w"], r64[lo:hi],
                                                                d["g_residual"][lo:hi], want_dw=False)[0], True)
