"""MI355X (gfx950) RMSNorm: forward, fused dX+dW backward, the fused
residual-add + RMSNorm + FP8 e4m3 1x128 block-quant producer, and the
training pair with a residual stream.

Thin ctypes binding over ``librmsnorm_gfx950.so``, whose C ABI is declared in
``include/rmsnorm_gfx950.h``.  Each function here only marshals arguments:
it checks that the torch tensors live on the current GPU with contiguous
columns, passes raw device pointers, row strides and torch's current HIP
stream to the C entry point of the same name, and raises ``RNError`` on a
non-zero status.  All arithmetic runs in the library's HIP kernels; there is
no other code path, and importing this package fails loudly when the library
has not been built.
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = [
    "RNError", "RN_F32", "RN_BF16", "RN_MAX_H", "lib", "library_path",
    "rmsnorm_fwd", "rmsnorm_bwd", "rmsnorm_bwd_workspace_bytes", "add_rmsnorm_fp8_block_quant",
    "rn_query_policy", "rn_bwd_workspace_bytes_for", "rn_status_string", "rn_version",
    "rn_selftest_quant", "rn_selftest_cvt_e4m3",
    "plan_rmsnorm_fwd", "plan_rmsnorm_bwd", "plan_add_rmsnorm_fp8_block_quant",
    "rmsnorm_fwd_residual", "rmsnorm_bwd_residual", "plan_rmsnorm_fwd_residual", "plan_rmsnorm_bwd_residual",
    "rmsnorm_fwd_heads", "plan_rmsnorm_fwd_heads", "RN_HEADS_MAX_VECTORS",
    "RN_F16", "RN_E4M3", "RN_E5M2", "add_rmsnorm_fp8_quant", "plan_add_rmsnorm_fp8_quant",
    "rn_selftest_cvt_e5m2", "rn_selftest_quotient", "rmsnorm_bwd_noalloc",
]

RN_F32 = 0
RN_BF16 = 1
RN_F16 = 2
RN_E4M3 = 0
RN_E5M2 = 1
RN_MAX_H = 32768
RN_HEADS_MAX_VECTORS = 128

_HERE = os.path.dirname(os.path.abspath(__file__))
library_path = os.path.join(_HERE, "librmsnorm_gfx950.so")

if not os.path.exists(library_path):
    raise ImportError(
        "bwd_fp8_block_amd: %s is missing; build it with `python bwd_fp8_block_amd/build.py` "
        "(or __graft_entry__.build())" % library_path)

# torch is imported first so that its HIP runtime is the one the library binds to.
lib = ctypes.CDLL(library_path)

_i64, _i32, _f32, _vp, _sz = ctypes.c_int64, ctypes.c_int, ctypes.c_float, ctypes.c_void_p, ctypes.c_size_t
lib.rn_status_string.argtypes = [_i32]
lib.rn_status_string.restype = ctypes.c_char_p
lib.rn_version.argtypes = []
lib.rn_version.restype = _i32
lib.rmsnorm_fwd.argtypes = [_vp, _i64, _i32, _vp, _i32, _vp, _i64, _vp, _i64, _i64, _f32, _vp]
lib.rmsnorm_fwd.restype = _i32
lib.rmsnorm_bwd_workspace_bytes.argtypes = [_i64, _i64, _i32]
lib.rmsnorm_bwd_workspace_bytes.restype = _sz
lib.rmsnorm_bwd.argtypes = [_vp, _i64, _vp, _i64, _i32, _vp, _i32, _vp, _vp, _i64, _vp,
                            _i64, _i64, _i32, _vp, _sz, _vp]
lib.rmsnorm_bwd.restype = _i32
lib.rmsnorm_bwd_noalloc.argtypes = [_vp, _i64, _vp, _i64, _i32, _vp, _i32, _vp, _vp, _i64, _vp, _i64, _i64, _i32, _vp]
lib.rmsnorm_bwd_noalloc.restype = _i32
lib.add_rmsnorm_fp8_block_quant.argtypes = [_vp, _i64, _vp, _i64, _vp, _vp, _i64, _vp, _i64, _vp, _i64,
                                            _i64, _i64, _f32, _vp]
lib.add_rmsnorm_fp8_block_quant.restype = _i32
lib.rmsnorm_fwd_residual.argtypes = [_vp, _i64, _vp, _i64, _i32, _vp, _i32, _vp, _i64, _vp, _i64, _vp,
                                     _i64, _i64, _f32, _vp]
lib.rmsnorm_fwd_residual.restype = _i32
lib.rmsnorm_bwd_residual.argtypes = [_vp, _i64, _vp, _i64, _i32, _vp, _i32, _vp, _vp, _i64, _vp, _i64, _vp,
                                     _i64, _i64, _i32, _vp, _sz, _vp]
lib.rmsnorm_bwd_residual.restype = _i32
lib.rmsnorm_fwd_heads.argtypes = [_vp, _i64, _i64, _i32, _vp, _i32, _vp, _i64, _i64, _vp, _i64, _i64, _i64,
                                  _f32, _vp]
lib.rmsnorm_fwd_heads.restype = _i32
lib.add_rmsnorm_fp8_quant.argtypes = [_vp, _i64, _vp, _i64, _vp, _i32, _vp, _i64, _i32, _vp, _i64, _vp, _vp, _i64,
                                      _i64, _i64, _f32, _vp]
lib.add_rmsnorm_fp8_quant.restype = _i32
lib.rn_selftest_cvt_e5m2.argtypes = [_vp, _vp, _i64, _vp]
lib.rn_selftest_cvt_e5m2.restype = _i32
lib.rn_selftest_quotient.argtypes = [_i32, _i32, ctypes.c_uint32, ctypes.c_uint32, _vp, _i64, _vp, _vp, _vp]
lib.rn_selftest_quotient.restype = _i32
lib.rn_query_policy.argtypes = [_i32, _i64, _i64, _i32, _i32, _i32, ctypes.POINTER(ctypes.c_int32)]
lib.rn_query_policy.restype = _i32
lib.rn_bwd_workspace_bytes_for.argtypes = [_i64, _i64, _i32]
lib.rn_bwd_workspace_bytes_for.restype = _sz
lib.rn_selftest_quant.argtypes = [ctypes.c_uint32, ctypes.c_uint32, _vp, _vp, _vp]
lib.rn_selftest_quant.restype = _i32
lib.rn_selftest_cvt_e4m3.argtypes = [_vp, _vp, _i64, _vp]
lib.rn_selftest_cvt_e4m3.restype = _i32

_SIZE_MAX = ctypes.c_size_t(-1).value


class RNError(RuntimeError):
    """A non-zero rn_status returned by the library."""

    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__("%s: %s (status %d)" % (fn, rn_status_string(status), status))


def rn_status_string(status: int) -> str:
    return lib.rn_status_string(int(status)).decode()


def rn_version() -> int:
    return int(lib.rn_version())


def _check(fn: str, st: int) -> None:
    if st != 0:
        raise RNError(fn, st)


def _dt(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return RN_BF16
    if t.dtype == torch.float32:
        return RN_F32
    raise TypeError("unsupported dtype %s (float32 or bfloat16)" % t.dtype)


def _dev(tensors) -> torch.device:
    dev = None
    for t in tensors:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError("all tensors must be on the GPU (got %s)" % t.device)
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError("tensors are on different devices")
    return dev


def _mat(t: torch.Tensor, name: str):
    """(pointer, row stride in elements) of a 2-D tensor with contiguous columns."""
    if t.dim() != 2:
        raise ValueError("%s must be 2-D [T, H]" % name)
    if t.shape[0] > 0 and t.shape[1] > 1 and t.stride(1) != 1:
        raise ValueError("%s must have contiguous columns" % name)
    ld = t.stride(0) if t.shape[0] > 1 else t.shape[1]
    return t.data_ptr(), ld


def _vec(t: torch.Tensor, name: str):
    if t.dim() != 1 or (t.numel() > 1 and t.stride(0) != 1):
        raise ValueError("%s must be a contiguous 1-D tensor" % name)
    return t.data_ptr()


def _stream(dev: torch.device):
    return torch.cuda.current_stream(dev).cuda_stream


class _NoSwitch:
    def __enter__(self):
        return None

    def __exit__(self, *a):
        return False


_NOSWITCH = _NoSwitch()


def _on(dev: torch.device):
    """Make `dev` current for the call (a no-op when it already is)."""
    return _NOSWITCH if dev.index == torch.cuda.current_device() else torch.cuda.device(dev)


def _prep_fwd(x, w, y, rstd, eps):
    dev = _dev((x, w, y, rstd))
    T, H = x.shape
    if y.shape != x.shape or y.dtype != x.dtype or w.shape != (H,) or rstd.shape != (T,) or rstd.dtype != torch.float32:
        raise ValueError("rmsnorm_fwd: shape or dtype mismatch")
    px, ldx = _mat(x, "x")
    py, ldy = _mat(y, "y")
    with _on(dev):
        args = (px, ldx, _dt(x), _vec(w, "w"), _dt(w), py, ldy, _vec(rstd, "rstd"), T, H, float(eps), _stream(dev))
    return dev, lib.rmsnorm_fwd, args


def rmsnorm_fwd(x: torch.Tensor, w: torch.Tensor, y: torch.Tensor, rstd: torch.Tensor, eps: float) -> None:
    """y = x * rstd * w with rstd = 1/sqrt(mean(x^2) + eps); writes y [T,H] and rstd [T] (fp32)."""
    dev, fn, args = _prep_fwd(x, w, y, rstd, eps)
    with _on(dev):
        st = fn(*args)
    _check("rmsnorm_fwd", st)


def rmsnorm_bwd_workspace_bytes(T: int, H: int, device=None) -> int:
    """Workspace bytes rmsnorm_bwd needs for (T, H) on `device`."""
    if device is None:
        device = torch.cuda.current_device()
    idx = torch.device(device).index if not isinstance(device, int) else device
    if idx is None:
        idx = torch.cuda.current_device()
    n = lib.rmsnorm_bwd_workspace_bytes(int(T), int(H), int(idx))
    if n == _SIZE_MAX:
        raise RNError("rmsnorm_bwd_workspace_bytes", 2)
    return int(n)


def rmsnorm_bwd(dy: torch.Tensor, x: torch.Tensor, w: torch.Tensor, rstd: torch.Tensor,
                dx: torch.Tensor, dw: torch.Tensor, deterministic: bool = True,
                workspace: torch.Tensor | None = None) -> None:
    """dx [T,H] and dw [H] (fp32, overwritten) from dy, x, w and the forward's rstd.
    `workspace`: a device tensor of at least rmsnorm_bwd_workspace_bytes(T, H) bytes
    (may be None when that size is 0; its content does not matter)."""
    dev, fn, args = _prep_bwd(dy, x, w, rstd, dx, dw, deterministic, workspace)
    with _on(dev):
        st = fn(*args)
    _check("rmsnorm_bwd", st)


def rmsnorm_bwd_noalloc(dy: torch.Tensor, x: torch.Tensor, w: torch.Tensor, rstd: torch.Tensor,
                        dx: torch.Tensor, dw: torch.Tensor, deterministic: bool = True) -> None:
    """rmsnorm_bwd with the library's own per-device scratch instead of a workspace
    (nothing is allocated; calls that overlap on one device race on the scratch)."""
    dev, _, a = _prep_bwd(dy, x, w, rstd, dx, dw, deterministic, None)
    with _on(dev):
        st = lib.rmsnorm_bwd_noalloc(*(a[:14] + a[16:]))
    _check("rmsnorm_bwd_noalloc", st)


def _prep_bwd(dy, x, w, rstd, dx, dw, deterministic, workspace):
    dev = _dev((dy, x, w, rstd, dx, dw, workspace))
    T, H = x.shape
    if dy.shape != x.shape or dx.shape != x.shape or dy.dtype != x.dtype or dx.dtype != x.dtype:
        raise ValueError("rmsnorm_bwd: dy/x/dx shape or dtype mismatch")
    if w.shape != (H,) or rstd.shape != (T,) or dw.shape != (H,) or dw.dtype != torch.float32:
        raise ValueError("rmsnorm_bwd: w/rstd/dw shape or dtype mismatch")
    pdy, lddy = _mat(dy, "dy")
    px, ldx = _mat(x, "x")
    pdx, lddx = _mat(dx, "dx")
    wsp, wsb = None, 0
    if workspace is not None:
        if not workspace.is_contiguous():
            raise ValueError("workspace must be contiguous")
        wsp, wsb = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    with _on(dev):
        args = (pdy, lddy, px, ldx, _dt(x), _vec(w, "w"), _dt(w), _vec(rstd, "rstd"),
                pdx, lddx, _vec(dw, "dw"), T, H, 1 if deterministic else 0, wsp, wsb, _stream(dev))
    return dev, lib.rmsnorm_bwd, args


def add_rmsnorm_fp8_block_quant(x: torch.Tensor, residual: torch.Tensor, w: torch.Tensor,
                                out: torch.Tensor, block_scale: torch.Tensor, normed_out: torch.Tensor,
                                eps: float) -> None:
    """residual <- bf16(x + residual); normed_out = bf16 RMSNorm(residual) * w;
    out = e4m3 codes [T,H] (uint8 or float8_e4m3fn); block_scale [H/128, ld] fp32 with
    entry (k, m) the scale of row m, block k (ld = block_scale.stride(0) >= T)."""
    dev, fn, args = _prep_fp8(x, residual, w, out, block_scale, normed_out, eps)
    with _on(dev):
        st = fn(*args)
    _check("add_rmsnorm_fp8_block_quant", st)


def _prep_fp8(x, residual, w, out, block_scale, normed_out, eps):
    dev = _dev((x, residual, w, out, block_scale, normed_out))
    T, H = x.shape
    for t, n in ((x, "x"), (residual, "residual"), (w, "w"), (normed_out, "normed_out")):
        if t.dtype != torch.bfloat16:
            raise ValueError("%s must be bfloat16" % n)
    if out.dtype not in (torch.uint8, torch.float8_e4m3fn):
        raise ValueError("out must be uint8 or float8_e4m3fn")
    if residual.shape != x.shape or normed_out.shape != x.shape or out.shape != x.shape or w.shape != (H,):
        raise ValueError("add_rmsnorm_fp8_block_quant: shape mismatch")
    if block_scale.dtype != torch.float32 or block_scale.dim() != 2 or block_scale.shape[0] != H // 128:
        raise ValueError("block_scale must be float32 [H/128, >= T]")
    if block_scale.shape[1] < T or (block_scale.numel() > 1 and block_scale.stride(1) != 1):
        raise ValueError("block_scale must be [H/128, ld >= T] with the row index contiguous")
    scale_ld = block_scale.stride(0) if block_scale.shape[0] > 1 else block_scale.shape[1]
    px, ldx = _mat(x, "x")
    pr, ldr = _mat(residual, "residual")
    po, ldo = _mat(out, "out")
    pn, ldn = _mat(normed_out, "normed_out")
    with _on(dev):
        args = (px, ldx, pr, ldr, _vec(w, "w"), po, ldo, block_scale.data_ptr(), scale_ld, pn, ldn,
                T, H, float(eps), _stream(dev))
    return dev, lib.add_rmsnorm_fp8_block_quant, args


def _prep_fwd_residual(x, u, w, y, h_out, rstd, eps):
    dev = _dev((x, u, w, y, h_out, rstd))
    T, H = x.shape
    for t in (u, y, h_out):
        if t.shape != x.shape or t.dtype != x.dtype:
            raise ValueError("rmsnorm_fwd_residual: u, y and h_out must match x in shape and dtype")
    if w.shape != (H,) or rstd.shape != (T,) or rstd.dtype != torch.float32:
        raise ValueError("rmsnorm_fwd_residual: w/rstd shape or dtype mismatch")
    px, ldx = _mat(x, "x")
    pu, ldu = _mat(u, "u")
    py, ldy = _mat(y, "y")
    ph, ldh = _mat(h_out, "h_out")
    with _on(dev):
        args = (px, ldx, pu, ldu, _dt(x), _vec(w, "w"), _dt(w), py, ldy, ph, ldh, _vec(rstd, "rstd"),
                T, H, float(eps), _stream(dev))
    return dev, lib.rmsnorm_fwd_residual, args


def rmsnorm_fwd_residual(x: torch.Tensor, u: torch.Tensor, w: torch.Tensor, y: torch.Tensor,
                         h_out: torch.Tensor, rstd: torch.Tensor, eps: float) -> None:
    """h_out = round(x + u); y = h_out * rstd * w with rstd = 1/sqrt(mean(h_out^2) + eps).
    h_out may be x or u itself (in-place update of the residual stream)."""
    dev, fn, args = _prep_fwd_residual(x, u, w, y, h_out, rstd, eps)
    with _on(dev):
        st = fn(*args)
    _check("rmsnorm_fwd_residual", st)


def _prep_bwd_residual(dy, x, w, rstd, g_residual, dx, dw, deterministic, workspace):
    dev, _, a = _prep_bwd(dy, x, w, rstd, dx, dw, deterministic, workspace)
    if g_residual.shape != x.shape or g_residual.dtype != x.dtype or g_residual.device != dev:
        raise ValueError("rmsnorm_bwd_residual: g_residual must match x in shape, dtype and device")
    pg, ldg = _mat(g_residual, "g_residual")
    args = a[:8] + (pg, ldg) + a[8:]
    return dev, lib.rmsnorm_bwd_residual, args


def rmsnorm_bwd_residual(dy: torch.Tensor, x: torch.Tensor, w: torch.Tensor, rstd: torch.Tensor,
                         g_residual: torch.Tensor, dx: torch.Tensor, dw: torch.Tensor,
                         deterministic: bool = True, workspace: torch.Tensor | None = None) -> None:
    """Backward of rmsnorm_fwd_residual: dx = (the rmsnorm_bwd dx at x = h_out) + g_residual,
    dw as in rmsnorm_bwd.  g_residual may be dx itself (in-place accumulation)."""
    dev, fn, args = _prep_bwd_residual(dy, x, w, rstd, g_residual, dx, dw, deterministic, workspace)
    with _on(dev):
        st = fn(*args)
    _check("rmsnorm_bwd_residual", st)


def _heads(t: torch.Tensor, name: str):
    """(pointer, token stride, head stride) of a [T, heads, head_dim] view with contiguous head_dim."""
    if t.dim() != 3:
        raise ValueError("%s must be 3-D [T, heads, head_dim]" % name)
    T, nh, D = t.shape
    if T > 0 and D > 1 and t.stride(2) != 1:
        raise ValueError("%s must have a contiguous head_dim" % name)
    ld_h = t.stride(1) if nh > 1 else D
    ld_t = t.stride(0) if T > 1 else (nh - 1) * ld_h + D
    return t.data_ptr(), ld_t, ld_h


def _prep_fwd_heads(x, w, y, rstd, eps):
    dev = _dev((x, w, y, rstd))
    if y.shape != x.shape or y.dtype != x.dtype:
        raise ValueError("rmsnorm_fwd_heads: y must match x in shape and dtype")
    T, nh, D = x.shape
    if w.shape != (D,):
        raise ValueError("rmsnorm_fwd_heads: w must be [head_dim]")
    pr = None
    if rstd is not None:
        if rstd.dtype != torch.float32 or rstd.numel() != T * nh or not rstd.is_contiguous():
            raise ValueError("rmsnorm_fwd_heads: rstd must be contiguous float32 with T*heads elements")
        pr = rstd.data_ptr()
    px, ldt, ldh = _heads(x, "x")
    py, ldyt, ldyh = _heads(y, "y")
    with _on(dev):
        args = (px, ldt, ldh, _dt(x), _vec(w, "w"), _dt(w), py, ldyt, ldyh, pr, T, nh, D, float(eps), _stream(dev))
    return dev, lib.rmsnorm_fwd_heads, args


def rmsnorm_fwd_heads(x: torch.Tensor, w: torch.Tensor, y: torch.Tensor, rstd: torch.Tensor | None,
                      eps: float) -> None:
    """Per-head RMSNorm over x viewed as [T, heads, head_dim] (any token and head strides, contiguous
    head_dim), shared weight w [head_dim]; y has the same shape and may be x itself (in place).
    rstd: float32 with T*heads elements (token-major) or None."""
    dev, fn, args = _prep_fwd_heads(x, w, y, rstd, eps)
    with _on(dev):
        st = fn(*args)
    _check("rmsnorm_fwd_heads", st)


_FP8_OUT = {torch.uint8: None, torch.float8_e4m3fn: RN_E4M3, torch.float8_e5m2: RN_E5M2}


def _prep_fp8_quant(x, residual, w, out, block_scale, tensor_scale, normed_out, eps, out_format):
    dev = _dev((x, residual, w, out, block_scale, tensor_scale, normed_out))
    T, H = x.shape
    if x.dtype == torch.bfloat16:
        dt = RN_BF16
    elif x.dtype == torch.float16:
        dt = RN_F16
    else:
        raise ValueError("add_rmsnorm_fp8_quant: x must be bfloat16 or float16")
    for t, n in ((residual, "residual"), (w, "w"), (normed_out, "normed_out")):
        if t is not None and t.dtype != x.dtype:
            raise ValueError("%s must have x's dtype" % n)
    if out.dtype not in _FP8_OUT:
        raise ValueError("out must be uint8, float8_e4m3fn or float8_e5m2")
    fmt = {"e4m3": RN_E4M3, "e5m2": RN_E5M2}[out_format] if isinstance(out_format, str) else int(out_format)
    if _FP8_OUT[out.dtype] is not None and _FP8_OUT[out.dtype] != fmt:
        raise ValueError("out's dtype does not match out_format")
    if residual.shape != x.shape or out.shape != x.shape or w.shape != (H,) or \
            (normed_out is not None and normed_out.shape != x.shape):
        raise ValueError("add_rmsnorm_fp8_quant: shape mismatch")
    if (block_scale is None) == (tensor_scale is None):
        raise ValueError("give exactly one of block_scale and tensor_scale")
    ps, sld, pt = None, 0, None
    if block_scale is not None:
        if block_scale.dtype != torch.float32 or block_scale.dim() != 2 or block_scale.shape[0] != H // 128:
            raise ValueError("block_scale must be float32 [H/128, >= T]")
        if block_scale.shape[1] < T or (block_scale.numel() > 1 and block_scale.stride(1) != 1):
            raise ValueError("block_scale must be [H/128, ld >= T] with the row index contiguous")
        ps = block_scale.data_ptr()
        sld = block_scale.stride(0) if block_scale.shape[0] > 1 else block_scale.shape[1]
    else:
        if tensor_scale.dtype != torch.float32 or tensor_scale.numel() != 1:
            raise ValueError("tensor_scale must be a one-element float32 device tensor")
        pt = tensor_scale.data_ptr()
    px, ldx = _mat(x, "x")
    pr, ldr = _mat(residual, "residual")
    po, ldo = _mat(out, "out")
    pn, ldn = _mat(normed_out, "normed_out") if normed_out is not None else (None, 0)
    with _on(dev):
        args = (px, ldx, pr, ldr, _vec(w, "w"), dt, po, ldo, fmt, ps, sld, pt, pn, ldn, T, H, float(eps),
                _stream(dev))
    return dev, lib.add_rmsnorm_fp8_quant, args


def add_rmsnorm_fp8_quant(x: torch.Tensor, residual: torch.Tensor, w: torch.Tensor, out: torch.Tensor,
                          eps: float, out_format="e4m3", block_scale: torch.Tensor | None = None,
                          tensor_scale: torch.Tensor | None = None, normed_out: torch.Tensor | None = None) -> None:
    """Producer variants: bf16 or fp16 rows (x's dtype), e4m3 or e5m2 codes, and either
    per-1x128-block scales (block_scale [H/128, ld]) or one given scale (tensor_scale, a
    one-element float32 device tensor).  normed_out is optional."""
    dev, fn, args = _prep_fp8_quant(x, residual, w, out, block_scale, tensor_scale, normed_out, eps, out_format)
    with _on(dev):
        st = fn(*args)
    _check("add_rmsnorm_fp8_quant", st)


def _plan(name, prep):
    dev, fn, args = prep
    cur = torch.cuda.current_device

    def call() -> None:
        if dev.index != cur():
            raise RuntimeError("%s: planned for %s, current device differs" % (name, dev))
        st = fn(*args)
        if st:
            raise RNError(name, st)
    return call


def plan_rmsnorm_fwd(x, w, y, rstd, eps):
    """A zero-argument callable that runs rmsnorm_fwd on these tensors and torch's current
    stream at plan time (arguments marshalled once; for launch-bound loops)."""
    return _plan("rmsnorm_fwd", _prep_fwd(x, w, y, rstd, eps))


def plan_rmsnorm_bwd(dy, x, w, rstd, dx, dw, deterministic=True, workspace=None):
    """Planned rmsnorm_bwd (see plan_rmsnorm_fwd)."""
    return _plan("rmsnorm_bwd", _prep_bwd(dy, x, w, rstd, dx, dw, deterministic, workspace))


def plan_add_rmsnorm_fp8_block_quant(x, residual, w, out, block_scale, normed_out, eps):
    """Planned add_rmsnorm_fp8_block_quant (see plan_rmsnorm_fwd)."""
    return _plan("add_rmsnorm_fp8_block_quant", _prep_fp8(x, residual, w, out, block_scale, normed_out, eps))


def plan_rmsnorm_fwd_residual(x, u, w, y, h_out, rstd, eps):
    """Planned rmsnorm_fwd_residual (see plan_rmsnorm_fwd)."""
    return _plan("rmsnorm_fwd_residual", _prep_fwd_residual(x, u, w, y, h_out, rstd, eps))


def plan_rmsnorm_bwd_residual(dy, x, w, rstd, g_residual, dx, dw, deterministic=True, workspace=None):
    """Planned rmsnorm_bwd_residual (see plan_rmsnorm_fwd)."""
    return _plan("rmsnorm_bwd_residual",
                 _prep_bwd_residual(dy, x, w, rstd, g_residual, dx, dw, deterministic, workspace))


def plan_rmsnorm_fwd_heads(x, w, y, rstd, eps):
    """Planned rmsnorm_fwd_heads (see plan_rmsnorm_fwd)."""
    return _plan("rmsnorm_fwd_heads", _prep_fwd_heads(x, w, y, rstd, eps))


def plan_add_rmsnorm_fp8_quant(x, residual, w, out, eps, out_format="e4m3", block_scale=None, tensor_scale=None,
                               normed_out=None):
    """Planned add_rmsnorm_fp8_quant (see plan_rmsnorm_fwd)."""
    return _plan("add_rmsnorm_fp8_quant", _prep_fp8_quant(x, residual, w, out, block_scale, tensor_scale,
                                                          normed_out, eps, out_format))


def rn_query_policy(op: int, T: int, H: int, x_dtype: int, w_dtype: int, cu_count: int) -> dict:
    """Host-only launch policy (no GPU needed)."""
    out = (ctypes.c_int32 * 7)()
    _check("rn_query_policy", lib.rn_query_policy(op, T, H, x_dtype, w_dtype, cu_count, out))
    return dict(lpr=out[0], nv=out[1], wgs=out[2], grid=out[3], gpw=out[4], kernel=out[5], flags=out[6])


def rn_bwd_workspace_bytes_for(T: int, H: int, cu_count: int) -> int:
    n = lib.rn_bwd_workspace_bytes_for(int(T), int(H), int(cu_count))
    if n == _SIZE_MAX:
        raise RNError("rn_bwd_workspace_bytes_for", 2)
    return int(n)


def rn_selftest_quant(a_lo: int, a_hi: int, mismatches: torch.Tensor, first_bad: torch.Tensor) -> None:
    """Exhaustive check of the producer's quantisation step (see the C header)."""
    dev = _dev((mismatches, first_bad))
    with _on(dev):
        st = lib.rn_selftest_quant(a_lo, a_hi, mismatches.data_ptr(), first_bad.data_ptr(), _stream(dev))
    _check("rn_selftest_quant", st)


def rn_selftest_cvt_e4m3(x: torch.Tensor, out: torch.Tensor) -> None:
    """out[i] = e4m3 code of float32 x[i], via the producer's conversion instruction."""
    dev = _dev((x, out))
    if x.dtype != torch.float32 or out.dtype != torch.uint8 or x.numel() != out.numel():
        raise ValueError("rn_selftest_cvt_e4m3: float32 in, uint8 out, same size")
    with _on(dev):
        st = lib.rn_selftest_cvt_e4m3(x.data_ptr(), out.data_ptr(), x.numel(), _stream(dev))
    _check("rn_selftest_cvt_e4m3", st)


def rn_selftest_cvt_e5m2(x: torch.Tensor, out: torch.Tensor) -> None:
    """out[i] = e5m2 code of float32 x[i], via the producer's conversion instruction."""
    dev = _dev((x, out))
    if x.dtype != torch.float32 or out.dtype != torch.uint8 or x.numel() != out.numel():
        raise ValueError("rn_selftest_cvt_e5m2: float32 in, uint8 out, same size")
    with _on(dev):
        st = lib.rn_selftest_cvt_e5m2(x.data_ptr(), out.data_ptr(), x.numel(), _stream(dev))
    _check("rn_selftest_cvt_e5m2", st)


def rn_selftest_quotient(dtype: int, out_format: int, mismatches: torch.Tensor, first_bad: torch.Tensor,
                         a_lo: int = 0, a_hi: int = 0, scales: torch.Tensor | None = None) -> None:
    """The producer's quotient against the IEEE division (see the C header)."""
    dev = _dev((mismatches, first_bad, scales))
    ps, ns = (scales.data_ptr(), scales.numel()) if scales is not None else (None, 0)
    with _on(dev):
        st = lib.rn_selftest_quotient(dtype, out_format, a_lo, a_hi, ps, ns, mismatches.data_ptr(),
                                      first_bad.data_ptr(), _stream(dev))
    _check("rn_selftest_quotient", st)
