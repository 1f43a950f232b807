"""CPU FP64 oracle for RMSNorm forward / backward and the fused
add-RMSNorm-FP8 1x128 block-quant producer.

TEST INFRASTRUCTURE ONLY: imported by the test suite, the smoke check and the
benchmark's CPU-baseline leg, never by the product package.  The arithmetic is
in ``oracle.c`` (plain sequential C, FP64, no fast-math); this module only
compiles it with gcc and marshals numpy arrays through ctypes.

Parity status of each function (what pins it, independently of itself) is
stated in the test files ``tests/test_oracle_*.py``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

F32 = 0
BF16 = 1
F16 = 2
E4M3 = 0
E5M2 = 1

_lib = None


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so (gcc, -O2, no fast-math, no FP contraction)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c11", "-Wall", "-Wextra", "-fno-fast-math",
               "-ffp-contract=off", "-fPIC", "-shared", _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB):
        build(force=True)
    lib = ctypes.CDLL(_LIB)
    i64, i32, f32 = ctypes.c_int64, ctypes.c_int, ctypes.c_float
    vp = ctypes.c_void_p
    lib.rno_bf16_to_double.argtypes = [ctypes.c_uint16]
    lib.rno_bf16_to_double.restype = ctypes.c_double
    lib.rno_double_to_bf16.argtypes = [ctypes.c_double]
    lib.rno_double_to_bf16.restype = ctypes.c_uint16
    lib.rno_e4m3_to_double.argtypes = [ctypes.c_uint8]
    lib.rno_e4m3_to_double.restype = ctypes.c_double
    lib.rno_float_to_e4m3.argtypes = [ctypes.c_float]
    lib.rno_float_to_e4m3.restype = ctypes.c_uint8
    lib.rno_rmsnorm_fwd.argtypes = [vp, i64, i32, vp, i32, i64, i64, f32, vp, i64, vp]
    lib.rno_rmsnorm_fwd.restype = i32
    lib.rno_rmsnorm_bwd.argtypes = [vp, i64, vp, i64, i32, vp, i32, vp, i64, i64, vp, i64, vp]
    lib.rno_rmsnorm_bwd.restype = i32
    lib.rno_block_quant_e4m3.argtypes = [vp, i64, i64, i64, vp, i64, vp, i64]
    lib.rno_block_quant_e4m3.restype = i32
    lib.rno_add_rmsnorm_fp8.argtypes = [vp, i64, vp, i64, vp, i64, i64, f32,
                                        vp, i64, vp, vp, i64, vp, i64, vp, i64, vp, i64]
    lib.rno_add_rmsnorm_fp8.restype = i32
    lib.rno_residual_add.argtypes = [vp, i64, vp, i64, i32, i64, i64, vp, i64]
    lib.rno_residual_add.restype = i32
    lib.rno_rmsnorm_fwd_residual.argtypes = [vp, i64, vp, i64, i32, vp, i32, i64, i64, f32, vp, i64, vp, i64, vp]
    lib.rno_rmsnorm_fwd_residual.restype = i32
    lib.rno_rmsnorm_bwd_residual.argtypes = [vp, i64, vp, i64, i32, vp, i32, vp, vp, i64, i64, i64, vp, i64, vp]
    lib.rno_rmsnorm_bwd_residual.restype = i32
    lib.rno_rmsnorm_fwd_heads.argtypes = [vp, i64, i64, i32, vp, i32, i64, i64, i64, f32, vp, vp]
    lib.rno_rmsnorm_fwd_heads.restype = i32
    lib.rno_f16_to_double.argtypes = [ctypes.c_uint16]
    lib.rno_f16_to_double.restype = ctypes.c_double
    lib.rno_double_to_f16.argtypes = [ctypes.c_double]
    lib.rno_double_to_f16.restype = ctypes.c_uint16
    lib.rno_e5m2_to_double.argtypes = [ctypes.c_uint8]
    lib.rno_e5m2_to_double.restype = ctypes.c_double
    lib.rno_float_to_e5m2.argtypes = [ctypes.c_float]
    lib.rno_float_to_e5m2.restype = ctypes.c_uint8
    lib.rno_quant_lp.argtypes = [vp, i64, i32, i32, i64, i64, f32, vp, i64, vp, i64]
    lib.rno_quant_lp.restype = i32
    lib.rno_add_rmsnorm_quant.argtypes = [vp, i64, vp, i64, vp, i32, i32, i64, i64, f32, f32,
                                          vp, i64, vp, vp, i64, vp, i64, vp, i64, vp, i64]
    lib.rno_add_rmsnorm_quant.restype = i32
    _lib = lib
    return lib


# --------------------------------------------------------------------------
# helpers: arrays are numpy; bf16 tensors travel as uint16 bit patterns
# --------------------------------------------------------------------------

def _dtype_code(a: np.ndarray) -> int:
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.uint16:
        return BF16
    raise TypeError("oracle inputs are float32 arrays or uint16 bf16 bit patterns, got %s" % a.dtype)


def _ptr(a):
    return None if a is None else a.ctypes.data


def _row_stride(a: np.ndarray) -> int:
    assert a.ndim == 2 and a.strides[1] == a.itemsize, "rows must be contiguous"
    return a.strides[0] // a.itemsize


def bf16_to_double(b: int) -> float:
    return _load().rno_bf16_to_double(int(b))


def double_to_bf16(v: float) -> int:
    return int(_load().rno_double_to_bf16(float(v)))


def e4m3_to_double(c: int) -> float:
    return _load().rno_e4m3_to_double(int(c))


def float_to_e4m3(v) -> int:
    return int(_load().rno_float_to_e4m3(float(np.float32(v))))


def bf16_decode_array(a: np.ndarray) -> np.ndarray:
    """Vectorised exact decode of bf16 bit patterns (uint16) to float64."""
    lib = _load()
    flat = np.ascontiguousarray(a).ravel()
    out = np.fromiter((lib.rno_bf16_to_double(int(v)) for v in flat), dtype=np.float64, count=flat.size)
    return out.reshape(a.shape)


def rmsnorm_fwd(x: np.ndarray, w: np.ndarray, eps: float, want_y: bool = True):
    """FP64 forward: returns (y unrounded [T,H] float64 or None, rstd [T] float64)."""
    lib = _load()
    T, H = x.shape
    y = np.empty((T, H), dtype=np.float64) if want_y else None
    rstd = np.empty((T,), dtype=np.float64)
    rc = lib.rno_rmsnorm_fwd(_ptr(x), _row_stride(x) if T else H, _dtype_code(x),
                             _ptr(w), _dtype_code(w), T, H, np.float32(eps),
                             _ptr(y), H, _ptr(rstd))
    if rc:
        raise ValueError("oracle rmsnorm_fwd rejected the arguments (%d)" % rc)
    return y, rstd


def rmsnorm_bwd(dy: np.ndarray, x: np.ndarray, w: np.ndarray, rstd: np.ndarray,
                want_dx: bool = True, want_dw: bool = True):
    """FP64 backward at the given rstd: returns (dx [T,H] float64 or None, dw [H] float64 or None)."""
    lib = _load()
    assert dy.dtype == x.dtype and dy.shape == x.shape
    T, H = x.shape
    rstd = np.ascontiguousarray(rstd, dtype=np.float64)
    dx = np.empty((T, H), dtype=np.float64) if want_dx else None
    dw = np.empty((H,), dtype=np.float64) if want_dw else None
    rc = lib.rno_rmsnorm_bwd(_ptr(dy), _row_stride(dy) if T else H, _ptr(x), _row_stride(x) if T else H,
                             _dtype_code(x), _ptr(w), _dtype_code(w), _ptr(rstd), T, H,
                             _ptr(dx), H, _ptr(dw))
    if rc:
        raise ValueError("oracle rmsnorm_bwd rejected the arguments (%d)" % rc)
    return dx, dw


def block_quant_e4m3(normed_bf16: np.ndarray, scale_ld: int | None = None):
    """Quantise bf16 normed values (uint16 [T,H]) per 1x128 block.

    Returns (scale [H/128, scale_ld] float32 with padding rows left NaN, codes [T,H] uint8)."""
    lib = _load()
    T, H = normed_bf16.shape
    if scale_ld is None:
        scale_ld = (T + 3) // 4 * 4
    scale = np.full((H // 128, scale_ld), np.nan, dtype=np.float32)
    codes = np.empty((T, H), dtype=np.uint8)
    rc = lib.rno_block_quant_e4m3(_ptr(normed_bf16), _row_stride(normed_bf16) if T else H, T, H,
                                  _ptr(scale), scale_ld, _ptr(codes), H)
    if rc:
        raise ValueError("oracle block_quant_e4m3 rejected the arguments (%d)" % rc)
    return scale, codes


def add_rmsnorm_fp8(x: np.ndarray, res: np.ndarray, w: np.ndarray, eps: float,
                    scale_ld: int | None = None):
    """Full FP64 fused producer.

    Returns dict with h (uint16 bf16 [T,H]), rstd (float64 [T]), normed (float64 [T,H],
    unrounded), normed_bf16 (uint16 [T,H]), scale (float32 [H/128, scale_ld], NaN padding),
    codes (uint8 [T,H]) -- scale and codes quantised from the oracle's own normed_bf16."""
    lib = _load()
    T, H = x.shape
    if scale_ld is None:
        scale_ld = (T + 3) // 4 * 4
    h = np.empty((T, H), dtype=np.uint16)
    rstd = np.empty((T,), dtype=np.float64)
    normed = np.empty((T, H), dtype=np.float64)
    nb = np.empty((T, H), dtype=np.uint16)
    scale = np.full((H // 128, scale_ld), np.nan, dtype=np.float32)
    codes = np.empty((T, H), dtype=np.uint8)
    rc = lib.rno_add_rmsnorm_fp8(_ptr(x), _row_stride(x) if T else H, _ptr(res), _row_stride(res) if T else H,
                                 _ptr(w), T, H, np.float32(eps),
                                 _ptr(h), H, _ptr(rstd), _ptr(normed), H, _ptr(nb), H,
                                 _ptr(scale), scale_ld, _ptr(codes), H)
    if rc:
        raise ValueError("oracle add_rmsnorm_fp8 rejected the arguments (%d)" % rc)
    return dict(h=h, rstd=rstd, normed=normed, normed_bf16=nb, scale=scale, codes=codes)


def residual_add(x: np.ndarray, u: np.ndarray) -> np.ndarray:
    """h = x + u rounded once into x's dtype (uint16 bf16 bits or float32)."""
    lib = _load()
    assert x.dtype == u.dtype and x.shape == u.shape
    T, H = x.shape
    h = np.empty((T, H), dtype=x.dtype)
    rc = lib.rno_residual_add(_ptr(x), _row_stride(x) if T else H, _ptr(u), _row_stride(u) if T else H,
                              _dtype_code(x), T, H, _ptr(h), H)
    if rc:
        raise ValueError("oracle residual_add rejected the arguments (%d)" % rc)
    return h


def rmsnorm_fwd_residual(x: np.ndarray, u: np.ndarray, w: np.ndarray, eps: float, want_y: bool = True):
    """Training forward with a residual: returns (y unrounded float64 or None, rstd float64 [T],
    h_new [T,H] in x's dtype)."""
    lib = _load()
    assert x.dtype == u.dtype and x.shape == u.shape
    T, H = x.shape
    h = np.empty((T, H), dtype=x.dtype)
    y = np.empty((T, H), dtype=np.float64) if want_y else None
    rstd = np.empty((T,), dtype=np.float64)
    rc = lib.rno_rmsnorm_fwd_residual(_ptr(x), _row_stride(x) if T else H, _ptr(u), _row_stride(u) if T else H,
                                      _dtype_code(x), _ptr(w), _dtype_code(w), T, H, np.float32(eps),
                                      _ptr(h), H, _ptr(y), H, _ptr(rstd))
    if rc:
        raise ValueError("oracle rmsnorm_fwd_residual rejected the arguments (%d)" % rc)
    return y, rstd, h


def rmsnorm_bwd_residual(dy: np.ndarray, h: np.ndarray, w: np.ndarray, rstd: np.ndarray, g_res: np.ndarray,
                         want_dx: bool = True, want_dw: bool = True):
    """Training backward with a residual-stream gradient: returns (dx_total = dx + g_res unrounded
    float64 or None, dw float64 or None)."""
    lib = _load()
    assert dy.dtype == h.dtype == g_res.dtype and dy.shape == h.shape == g_res.shape
    T, H = h.shape
    rstd = np.ascontiguousarray(rstd, dtype=np.float64)
    dx = np.empty((T, H), dtype=np.float64) if want_dx else None
    dw = np.empty((H,), dtype=np.float64) if want_dw else None
    rc = lib.rno_rmsnorm_bwd_residual(_ptr(dy), _row_stride(dy) if T else H, _ptr(h), _row_stride(h) if T else H,
                                      _dtype_code(h), _ptr(w), _dtype_code(w), _ptr(rstd),
                                      _ptr(g_res), _row_stride(g_res) if T else H, T, H, _ptr(dx), H, _ptr(dw))
    if rc:
        raise ValueError("oracle rmsnorm_bwd_residual rejected the arguments (%d)" % rc)
    return dx, dw


def rmsnorm_fwd_heads(x: np.ndarray, heads: int, head_dim: int, w: np.ndarray, eps: float,
                      ld_head: int | None = None, want_y: bool = True):
    """Per-head RMSNorm over a [T, >= (heads-1)*ld_head + head_dim] array (float32 or uint16 bf16
    bits, contiguous columns): row (t, h) is x[t, h*ld_head : h*ld_head + head_dim].
    Returns (y [T, heads, head_dim] float64 unrounded or None, rstd [T, heads] float64)."""
    lib = _load()
    T = x.shape[0]
    ld_head = head_dim if ld_head is None else ld_head
    assert x.ndim == 2 and x.shape[1] >= (heads - 1) * ld_head + head_dim
    y = np.empty((T, heads, head_dim), dtype=np.float64) if want_y else None
    rstd = np.empty((T, heads), dtype=np.float64)
    rc = lib.rno_rmsnorm_fwd_heads(_ptr(x), _row_stride(x) if T else x.shape[1], ld_head, _dtype_code(x),
                                   _ptr(w), _dtype_code(w), T, heads, head_dim, np.float32(eps),
                                   _ptr(y), _ptr(rstd))
    if rc:
        raise ValueError("oracle rmsnorm_fwd_heads rejected the arguments (%d)" % rc)
    return y, rstd


def f16_to_double(b: int) -> float:
    return _load().rno_f16_to_double(int(b))


def double_to_f16(v: float) -> int:
    return int(_load().rno_double_to_f16(float(v)))


def e5m2_to_double(c: int) -> float:
    return _load().rno_e5m2_to_double(int(c))


def float_to_e5m2(v) -> int:
    return int(_load().rno_float_to_e5m2(float(np.float32(v))))


_FMT = {"e4m3": E4M3, "e5m2": E5M2}
_LP = {"bf16": BF16, "f16": F16}


def quant_lp(normed: np.ndarray, dtype: str, fmt: str, tensor_scale: float = 0.0, scale_ld: int | None = None):
    """Codes of low-precision normed values (uint16 bits of bf16 or fp16, [T,H]).
    tensor_scale > 0: that scale for every element (scale returned as None);
    0: per-1x128-block scales amax/MAX (returned [H/128, scale_ld] float32, NaN padding)."""
    lib = _load()
    T, H = normed.shape
    if scale_ld is None:
        scale_ld = (T + 3) // 4 * 4
    scale = None if tensor_scale else np.full((H // 128, scale_ld), np.nan, dtype=np.float32)
    codes = np.empty((T, H), dtype=np.uint8)
    rc = lib.rno_quant_lp(_ptr(normed), _row_stride(normed) if T else H, _LP[dtype], _FMT[fmt], T, H,
                          np.float32(tensor_scale), _ptr(scale), scale_ld, _ptr(codes), H)
    if rc:
        raise ValueError("oracle quant_lp rejected the arguments (%d)" % rc)
    return scale, codes


def add_rmsnorm_quant(x: np.ndarray, res: np.ndarray, w: np.ndarray, eps: float, dtype: str, fmt: str,
                      tensor_scale: float = 0.0, scale_ld: int | None = None):
    """The producer variants (bf16 / fp16 rows as uint16 bits; e4m3 / e5m2 codes; block or given
    per-tensor scale).  Returns dict h, rstd, normed (float64 unrounded), normed_lp (uint16 bits),
    scale (None for a per-tensor scale), codes."""
    lib = _load()
    T, H = x.shape
    if scale_ld is None:
        scale_ld = (T + 3) // 4 * 4
    h = np.empty((T, H), dtype=np.uint16)
    rstd = np.empty((T,), dtype=np.float64)
    normed = np.empty((T, H), dtype=np.float64)
    nl = np.empty((T, H), dtype=np.uint16)
    scale = None if tensor_scale else np.full((H // 128, scale_ld), np.nan, dtype=np.float32)
    codes = np.empty((T, H), dtype=np.uint8)
    rc = lib.rno_add_rmsnorm_quant(_ptr(x), _row_stride(x) if T else H, _ptr(res), _row_stride(res) if T else H,
                                   _ptr(w), _LP[dtype], _FMT[fmt], T, H, np.float32(eps), np.float32(tensor_scale),
                                   _ptr(h), H, _ptr(rstd), _ptr(normed), H, _ptr(nl), H,
                                   _ptr(scale), scale_ld, _ptr(codes), H)
    if rc:
        raise ValueError("oracle add_rmsnorm_quant rejected the arguments (%d)" % rc)
    return dict(h=h, rstd=rstd, normed=normed, normed_lp=nl, scale=scale, codes=codes)
