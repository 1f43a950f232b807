"""Device calls and result checks shared by the GPU parity tests: each helper runs one
entry point through the C ABI on host (numpy) inputs with guard bands around every
output, or compares an op's outputs with the oracle's under the parity rules of
gpu_common."""
import numpy as np
import torch

from gpu_common import assert_guards, check_values, guarded_matrix, to_dev, to_host, torch_dtype
from workloads import to_bf16_bits


def gpu_fwd(rn, x: np.ndarray, w: np.ndarray, eps: float, ld_pad=0):
    T, H = x.shape
    xd, wd = to_dev(x), to_dev(w)
    ld = H + ld_pad
    yfull, y = guarded_matrix(T, H, torch_dtype(x), ld)
    rfull, rstd = guarded_matrix(1, T, torch.float32)
    rstd = rstd.view(T)
    rn.rmsnorm_fwd(xd, wd, y, rstd, eps)
    torch.cuda.synchronize()
    assert_guards(yfull, T, H, ld, name="y")
    assert_guards(rfull, 1, T, T, name="rstd")
    return to_host(y) if T else np.zeros((0, H), x.dtype), to_host(rstd)


def gpu_bwd(rn, dy, x, w, rstd, det, ld_pad=0, poison=False):
    T, H = x.shape
    dyd, xd, wd = to_dev(dy), to_dev(x), to_dev(w)
    rd = torch.from_numpy(np.ascontiguousarray(rstd, dtype=np.float32)).cuda()
    ld = H + ld_pad
    dxfull, dx = guarded_matrix(T, H, torch_dtype(x), ld)
    dwfull, dw = guarded_matrix(1, H, torch.float32)
    dw = dw.view(H)
    nbytes = rn.rmsnorm_bwd_workspace_bytes(T, H)
    ws = torch.empty(max(nbytes // 4, 1), dtype=torch.float32, device="cuda")
    if poison:
        ws.fill_(float("nan"))
    rn.rmsnorm_bwd(dyd, xd, wd, rd, dx, dw, deterministic=det, workspace=ws)
    torch.cuda.synchronize()
    assert_guards(dxfull, T, H, ld, name="dx")
    assert_guards(dwfull, 1, H, H, name="dw")
    return to_host(dx) if T else np.zeros((0, H), x.dtype), to_host(dw)


def gpu_fp8(rn, x, res, w, eps, ld_pad=0, scale_pad=0):
    T, H = x.shape
    ld = H + ld_pad
    xd, wd = to_dev(x), to_dev(w)
    rfull, r = guarded_matrix(T, H, torch.bfloat16, ld)
    if T:
        r.copy_(to_dev(res))
    ofull, o = guarded_matrix(T, H, torch.uint8, ld)
    nfull, n = guarded_matrix(T, H, torch.bfloat16, ld)
    sld = (T + 3) // 4 * 4 + scale_pad
    sfull, s = guarded_matrix(H // 128, sld, torch.float32)
    rn.add_rmsnorm_fp8_block_quant(xd, r, wd, o, s, n, eps)
    torch.cuda.synchronize()
    assert_guards(rfull, T, H, ld, name="residual")
    assert_guards(ofull, T, H, ld, name="out")
    assert_guards(nfull, T, H, ld, name="normed")
    sh = to_host(s)
    assert np.all(np.isnan(sh[:, T:])), "scale padding rows were written"
    assert_guards(sfull, H // 128, sld, sld, name="block_scale")
    return to_host(r), to_host(o), sh, to_host(n)


def check_fp8(oracle, x, res, w, eps, h, out, scale, normed):
    T = x.shape[0]
    ref = oracle.add_rmsnorm_fp8(x, res, w, eps)
    assert np.array_equal(h, ref["h"]), "residual not bit-exact"
    check_values("normed", normed, ref["normed"], True)
    sref, cref = oracle.block_quant_e4m3(normed, scale_ld=scale.shape[1])
    assert np.array_equal(scale[:, :T].view(np.uint32), sref[:, :T].view(np.uint32)), "block scales not bit-exact"
    bad = np.argwhere(out != cref)
    assert bad.size == 0, "fp8 codes differ at %s (gpu 0x%02x, oracle 0x%02x)" % (
        bad[0], out[tuple(bad[0])], cref[tuple(bad[0])])
    # the oracle's own end-to-end codes: equal wherever its bf16 normed equals the GPU's
    same = ref["normed_bf16"] == normed
    assert np.array_equal(ref["codes"][same & np.repeat(
        (ref["scale"][:, :T].T == scale[:, :T].T), 128, axis=1)], out[same & np.repeat(
            (ref["scale"][:, :T].T == scale[:, :T].T), 128, axis=1)])
    return float(same.mean())


def gpu_fwd_res(rn, x, u, w, eps, ld_pad=0, inplace=None):
    """Runs rmsnorm_fwd_residual; inplace in (None, "x", "u") writes h_new over that input."""
    T, H = x.shape
    ld = H + ld_pad
    dt = torch_dtype(x)
    xfull, xd = guarded_matrix(T, H, dt, ld)
    ufull, ud = guarded_matrix(T, H, dt, ld)
    if T:
        xd.copy_(to_dev(x))
        ud.copy_(to_dev(u))
    yfull, y = guarded_matrix(T, H, dt, ld)
    if inplace == "x":
        hfull, h = xfull, xd
    elif inplace == "u":
        hfull, h = ufull, ud
    else:
        hfull, h = guarded_matrix(T, H, dt, ld)
    rfull, rstd = guarded_matrix(1, T, torch.float32)
    rstd = rstd.view(T)
    rn.rmsnorm_fwd_residual(xd, ud, to_dev(w), y, h, rstd, eps)
    torch.cuda.synchronize()
    for f, n in ((xfull, "x"), (ufull, "u"), (yfull, "y"), (hfull, "h_out")):
        assert_guards(f, T, H, ld, name=n)
    assert_guards(rfull, 1, T, T, name="rstd")
    empty = np.zeros((0, H), x.dtype)
    return (to_host(y) if T else empty), (to_host(h) if T else empty), to_host(rstd)


def gpu_bwd_res(rn, dy, h, w, rstd, gres, ld_pad=0, inplace=False, poison=False):
    T, H = h.shape
    ld = H + ld_pad
    dt = torch_dtype(h)
    rd = torch.from_numpy(np.ascontiguousarray(rstd, dtype=np.float32)).cuda()
    dxfull, dx = guarded_matrix(T, H, dt, ld)
    if inplace:
        if T:
            dx.copy_(to_dev(gres))
        g, gfull = dx, None
    else:
        gfull, g = guarded_matrix(T, H, dt, ld)
        if T:
            g.copy_(to_dev(gres))
    dwfull, dw = guarded_matrix(1, H, torch.float32)
    dw = dw.view(H)
    ws = torch.empty(max(rn.rmsnorm_bwd_workspace_bytes(T, H) // 4, 1), dtype=torch.float32, device="cuda")
    if poison:
        ws.fill_(float("nan"))
    rn.rmsnorm_bwd_residual(to_dev(dy), to_dev(h), to_dev(w), rd, g, dx, dw, deterministic=True, workspace=ws)
    torch.cuda.synchronize()
    assert_guards(dxfull, T, H, ld, name="dx")
    if gfull is not None:
        assert_guards(gfull, T, H, ld, name="g_residual")
        if T:
            assert np.array_equal(to_host(g), gres), "g_residual was modified"
    assert_guards(dwfull, 1, H, H, name="dw")
    return (to_host(dx) if T else np.zeros((0, H), h.dtype)), to_host(dw)


def make_fused(T, ld_t, dt, seed):
    rng = np.random.default_rng(seed)
    a = rng.standard_normal((T, ld_t)).astype(np.float32)
    return to_bf16_bits(a) if dt == "bf16" else a


def heads_view(dev_full, T, nh, D, ld_t, ld_h, off):
    return torch.as_strided(dev_full, (T, nh, D), (ld_t, ld_h, 1), storage_offset=off)


def run_heads(rn, host_full, nh, D, ld_h, off, w, eps, with_rstd=True, in_place=False):
    T, ld_t = host_full.shape
    dt = torch.bfloat16 if host_full.dtype == np.uint16 else torch.float32
    full = to_dev(host_full)
    x = heads_view(full, T, nh, D, ld_t, ld_h, off)
    if in_place:
        y, yfull = x, None
    else:
        yfull, y2 = guarded_matrix(T, nh * D, dt)
        y = y2.view(T, nh, D) if T else y2.view(0, nh, D)
    rfull, rstd = guarded_matrix(1, T * nh, torch.float32)
    rstd = rstd.view(T * nh)
    rn.rmsnorm_fwd_heads(x, to_dev(w), y, rstd if with_rstd else None, eps)
    torch.cuda.synchronize()
    if yfull is not None:
        assert_guards(yfull, T, nh * D, nh * D, name="y")
    assert_guards(rfull, 1, T * nh, T * nh, name="rstd")
    r = to_host(rstd).reshape(T, nh)
    if not with_rstd:
        assert np.all(np.isnan(r)), "rstd written although not requested"
    return to_host(y.contiguous()), r, to_host(full)


def lp16(a, dtype):
    a = np.asarray(a, np.float32)
    if dtype == "bf16":
        return to_bf16_bits(a)
    return a.astype(np.float16).view(np.uint16)


def dev16(bits, dtype):
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda()
    return t.view(torch.bfloat16 if dtype == "bf16" else torch.float16)


def host16(t):
    return t.detach().cpu().view(torch.int16).numpy().view(np.uint16)


def dec16(b, dtype):
    if dtype == "bf16":
        return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return b.view(np.float16).astype(np.float64)


def check_normed(normed, ref, dtype):
    if dtype == "bf16":
        return check_values("normed", normed, ref, True)
    g = dec16(normed, "f16")
    err = np.abs(g - ref)
    assert err.max() <= 5e-2
    spacing = np.exp2(np.floor(np.log2(np.maximum(np.abs(ref), 2.0 ** -14))) - 10)
    bad = err > spacing + 2.0 ** -20 * np.max(np.abs(ref), axis=-1, keepdims=True)
    assert not bad.any(), "normed: %d values beyond one fp16 spacing" % int(bad.sum())


def run_variant(rn, x, res, w, dtype, fmt, tensor_scale=None, with_normed=True, ld_pad=0, scale_pad=4, eps=1e-6):
    T, H = x.shape
    ld = H + ld_pad
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float16
    xd, wd = dev16(x, dtype), dev16(w, dtype)
    rfull, r = guarded_matrix(T, H, torch.bfloat16, ld)
    rfull, r = rfull.view(tdt), r.view(tdt)
    if T:
        r.copy_(dev16(res, dtype))
    ofull, o = guarded_matrix(T, H, torch.uint8, ld)
    nfull = n = None
    if with_normed:
        nfull, n = guarded_matrix(T, H, torch.bfloat16, ld)
        nfull, n = nfull.view(tdt), n.view(tdt)
    sfull = s = ts = None
    if tensor_scale is None:
        sld = (T + 3) // 4 * 4 + scale_pad
        sfull, s = guarded_matrix(H // 128, sld, torch.float32)
    else:
        ts = torch.tensor([tensor_scale], dtype=torch.float32, device="cuda")
    rn.add_rmsnorm_fp8_quant(xd, r, wd, o, eps, out_format=fmt, block_scale=s, tensor_scale=ts, normed_out=n)
    torch.cuda.synchronize()
    assert_guards(rfull.view(torch.bfloat16), T, H, ld, name="residual")
    assert_guards(ofull, T, H, ld, name="out")
    if nfull is not None:
        assert_guards(nfull.view(torch.bfloat16), T, H, ld, name="normed")
    sh = None
    if sfull is not None:
        sh = to_host(s)
        assert np.all(np.isnan(sh[:, T:])), "scale padding rows were written"
        assert_guards(sfull, H // 128, s.shape[1], s.shape[1], name="block_scale")
    return host16(r), to_host(o), sh, (host16(n) if n is not None else None)


def check_variant(oracle, x, res, w, dtype, fmt, tensor_scale, h, out, scale, normed, eps=1e-6):
    T = x.shape[0]
    ref = oracle.add_rmsnorm_quant(x, res, w, eps, dtype, fmt, tensor_scale or 0.0)
    assert np.array_equal(h, ref["h"]), "residual not bit-exact"
    if normed is None:
        normed = ref["normed_lp"]                     # codes then checked where the oracle's normed is exact
    else:
        check_normed(normed, ref["normed"], dtype)
    sref, cref = oracle.quant_lp(normed, dtype, fmt, tensor_scale or 0.0,
                                 scale_ld=scale.shape[1] if scale is not None else None)
    if scale is not None:
        assert np.array_equal(scale[:, :T].view(np.uint32), sref[:, :T].view(np.uint32)), "block scales differ"
    bad = np.argwhere(out != cref)
    assert bad.size == 0, "codes differ at %s (gpu 0x%02x, oracle 0x%02x)" % (
        bad[0], out[tuple(bad[0])], cref[tuple(bad[0])])
