"""Host-side checks of the C-ABI library (no GPU needed, no kernel launched).

* the shared library loads and exports every function declared in
  include/rmsnorm_gfx950.h;
* status strings, version;
* the launch policy (a pure host function) for the workload shapes;
* argument validation: each call below carries an argument error that the
  library must reject before it touches the device, so no pointer passed here
  is ever dereferenced.
"""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "rmsnorm_gfx950.h")


@pytest.fixture(scope="module")
def rn():
    lib_path = os.path.join(ROOT, "bwd_fp8_block_amd", "librmsnorm_gfx950.so")
    if not os.path.exists(lib_path):
        import importlib.util
        spec = importlib.util.spec_from_file_location(
            "bwd_fp8_block_amd_build", os.path.join(ROOT, "bwd_fp8_block_amd", "build.py"))
        b = importlib.util.module_from_spec(spec)
        spec.loader.exec_module(b)      # by path: the package __init__ needs the library
        b.build()
    import bwd_fp8_block_amd as m
    return m


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\**\s+\**([a-z_][a-z0-9_]*)\s*\(", src, flags=re.M)
    return sorted(set(names))


def test_exports_every_declared_symbol(rn):
    names = declared_functions()
    assert {"rmsnorm_fwd", "rmsnorm_bwd", "add_rmsnorm_fp8_block_quant", "rmsnorm_bwd_workspace_bytes"} <= set(names)
    lib = ctypes.CDLL(rn.library_path)
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings_and_version(rn):
    for code, text in [(0, "ok"), (1, "null pointer"), (2, "unsupported shape"), (3, "unsupported dtype"),
                       (4, "misaligned pointer"), (5, "bad row stride"), (6, "workspace missing or too small"),
                       (7, "overlapping buffers"), (8, "no gfx950 device"), (9, "kernel launch failed")]:
        assert rn.rn_status_string(code) == text
    assert rn.rn_status_string(99) == "unknown status"
    assert rn.rn_version() >= 10000


CU = 256


@pytest.mark.parametrize("op,T,H,xd,wd", [
    (0, 64, 256, 0, 0), (1, 64, 256, 0, 0),
    (0, 8192, 4096, 1, 1), (1, 8192, 4096, 1, 1),
    (1, 58497, 2048, 1, 0), (0, 65536, 5120, 1, 0), (1, 65536, 5120, 1, 0),
    (2, 4096, 7168, 1, 1), (2, 8192, 4096, 1, 1), (2, 3, 1152, 1, 1), (2, 1, 128, 1, 1),
    (2, 8192, 2048, 1, 1), (2, 32768, 2048, 1, 1), (2, 16384, 5120, 1, 1), (2, 1000, 1024, 1, 1),
    (2, 5, 1152, 1, 1), (2, 8192, 8192, 1, 1),
    (0, 5, 8, 1, 1), (1, 5, 8, 1, 1), (0, 100, 32768, 1, 1), (1, 9, 16384, 1, 1), (2, 9, 32768, 1, 1),
    (0, 7, 17408, 1, 1), (2, 7, 17408, 1, 1), (0, 7, 9216, 0, 0), (2, 7, 9216, 1, 1), (0, 3, 20480, 1, 0),
    (3, 8192, 4096, 1, 1), (3, 64, 256, 0, 0), (3, 5, 8, 1, 1), (3, 100, 120, 1, 1), (3, 33, 5120, 1, 0),
    (3, 17, 7168, 1, 1), (3, 9, 8200, 1, 1), (3, 5, 16384, 1, 1), (3, 3, 16384, 0, 0), (3, 2, 32768, 1, 1),
    (3, 1000, 128, 1, 1), (3, 300, 3072, 1, 1), (3, 7, 17408, 1, 1),
    (0, 1 << 21, 128, 1, 1), (0, 65536, 256, 1, 1), (0, 262144, 512, 1, 1), (0, 65536, 1024, 1, 1),
    (0, 65536, 64, 0, 0), (0, 9, 32, 0, 0), (0, 4096, 7168, 1, 1), (0, 8192, 8192, 1, 1), (3, 65536, 7168, 1, 1),
    (0, 3001, 5120, 1, 0),
])
def test_policy_invariants(rn, op, T, H, xd, wd):
    p = rn.rn_query_policy(op, T, H, xd, wd, CU)
    E = 8 if xd == 1 else 4
    nch = H // E
    assert p["lpr"] in ((8, 16, 32) if op in (0, 3) else (16, 32)) or p["lpr"] % 64 == 0
    assert p["lpr"] * p["nv"] >= nch                         # every chunk owned by a lane
    assert p["lpr"] * (p["nv"] - 1) < nch                    # no fully idle vector slot
    assert p["wgs"] % p["lpr"] == 0 and p["wgs"] <= 1024 and p["gpw"] == p["wgs"] // p["lpr"]
    assert 1 <= p["grid"] <= max(1, -(-T // p["gpw"]))       # no work-group without rows
    if op == 2:
        assert p["lpr"] % 16 == 0                            # 1x128 block = 16 lanes
    # a compiled variant serves it: the same check the library applies to overrides
    lprc = min(p["lpr"], 64)
    if op in (0, 3):
        assert (lprc, p["nv"]) in {(4, 4), (8, 1), (8, 2), (8, 4), (16, 1), (16, 2), (16, 4), (32, 1), (32, 2),
                                   (32, 4)} or \
            (lprc == 64 and (p["wgs"] <= 256 and 1 <= p["nv"] <= 8 or p["wgs"] <= 512 and 5 <= p["nv"] <= 8))
    elif op == 2:
        assert (lprc, p["nv"]) in {(16, 1), (32, 1)} or \
            (lprc == 64 and (p["wgs"] <= 256 and 1 <= p["nv"] <= 8 or p["wgs"] <= 512 and 2 <= p["nv"] <= 8))
    else:
        assert (lprc, p["nv"]) in {(16, 1), (32, 1), (64, 1), (64, 2)}
    if op == 1:
        assert p["grid"] <= CU                               # one row strip per CU at most


def test_policy_shapes_of_the_workloads(rn):
    f = rn.rn_query_policy(0, 8192, 4096, 1, 1, CU)
    assert f["lpr"] == 128 and f["nv"] == 4 and f["grid"] == 1024 and f["flags"] & 3 == 3
    b = rn.rn_query_policy(1, 8192, 4096, 1, 1, CU)
    assert b["nv"] == 1 and b["lpr"] == 512 and b["grid"] == 256
    # forward rows of 5-8 vectors per 128-lane group: 512-thread work-groups, one per CU on long
    # runs; the residual form keeps 256-thread groups
    f5 = rn.rn_query_policy(0, 65536, 5120, 1, 0, CU)
    assert f5["lpr"] == 128 and f5["nv"] == 5 and f5["wgs"] == 512 and f5["grid"] == CU
    assert rn.rn_query_policy(0, 4096, 5120, 1, 1, CU)["grid"] == 2 * CU
    assert rn.rn_query_policy(0, 4096, 7168, 1, 1, CU)["grid"] == CU
    r5 = rn.rn_query_policy(3, 65536, 5120, 1, 0, CU)
    assert r5["wgs"] == 256 and r5["gpw"] == 2 and r5["grid"] == CU
    q = rn.rn_query_policy(2, 4096, 7168, 1, 1, CU)
    assert q["lpr"] == 128 and q["nv"] == 7 and q["wgs"] == 512 and q["grid"] == 256
    # the producer: four 128-lane groups per work-group, one work-group per CU for long runs
    # and two for short ones; rows of 4 vectors switch from 32768 chunks per CU, as do rows of
    # 1024 chunks in 256-lane groups
    q2 = rn.rn_query_policy(2, 8192, 4096, 1, 1, CU)
    assert q2["lpr"] == 128 and q2["nv"] == 4 and q2["wgs"] == 256 and q2["grid"] == 2 * CU
    q5 = rn.rn_query_policy(2, 16384, 4096, 1, 1, CU)
    assert q5["lpr"] == 128 and q5["nv"] == 4 and q5["wgs"] == 512 and q5["grid"] == CU
    q3 = rn.rn_query_policy(2, 8192, 2048, 1, 1, CU)
    assert q3["wgs"] == 512 and q3["grid"] == 2 * CU
    q4 = rn.rn_query_policy(2, 8192, 8192, 1, 1, CU)               # rows of 1024 chunks: 256 lanes x 4
    assert q4["lpr"] == 256 and q4["nv"] == 4 and q4["wgs"] == 512 and q4["grid"] == CU
    q6 = rn.rn_query_policy(2, 4096, 8192, 1, 1, CU)
    assert q6["lpr"] == 256 and q6["wgs"] == 512 and q6["grid"] == 2 * CU
    r = rn.rn_query_policy(3, 8192, 4096, 1, 1, CU)
    assert r["lpr"] == 128 and r["nv"] == 4 and r["grid"] == 512 and r["flags"] & 3 == 3
    assert rn.rn_query_policy(0, 65536, 4096, 1, 1, CU)["grid"] == 512
    qk = rn.rn_query_policy(0, 8192 * 32, 128, 1, 1, CU)           # per-head rows of 128 bf16
    assert qk["lpr"] == 8 and qk["nv"] == 2 and qk["grid"] == 2048
    assert rn.rn_query_policy(3, 65536, 4096, 1, 1, CU)["grid"] == 256
    # streaming backward: 512-thread strips with three row buffers; rows of 513 .. 1024 chunks take
    # two vectors per lane in one group of at most 512 lanes; wider rows two vectors per lane in
    # groups of more than 512 lanes with two buffers
    assert b["wgs"] == 512 and (b["flags"] >> 4) & 7 == 3
    # the residual form streams with two row buffers in the steady form (flag 8) where the plain one takes three
    br = rn.rn_query_policy(4, 8192, 4096, 1, 1, CU)
    assert {k: br[k] for k in ("lpr", "nv", "wgs", "grid")} == {k: b[k] for k in ("lpr", "nv", "wgs", "grid")}
    assert (br["flags"] >> 4) & 7 == 2 and br["flags"] & 8 and br["flags"] & 3 == b["flags"] & 3
    for H in (128, 256):                                            # short rows: the same streaming form
        sb = rn.rn_query_policy(1, 65536, H, 1, 1, CU)
        assert sb["wgs"] == 512 and (sb["flags"] >> 4) & 7 == 3 and sb["grid"] == CU
    w = rn.rn_query_policy(1, 8192, 7168, 1, 1, CU)
    wr = rn.rn_query_policy(4, 8192, 7168, 1, 1, CU)
    assert w["lpr"] == 448 and w["nv"] == 2 and w["wgs"] == 448 and (w["flags"] >> 4) & 7 == 3
    assert {k: wr[k] for k in ("lpr", "nv", "wgs", "grid")} == {k: w[k] for k in ("lpr", "nv", "wgs", "grid")}
    assert (wr["flags"] >> 4) & 7 == 2 and wr["flags"] & 8
    c5 = rn.rn_query_policy(1, 65536, 5120, 1, 0, CU)
    assert c5["lpr"] == 320 and c5["nv"] == 2 and c5["wgs"] == 320 and c5["grid"] == CU
    x = rn.rn_query_policy(1, 8192, 12288, 1, 1, CU)                # beyond 1024 chunks
    assert x["nv"] == 2 and x["lpr"] == 768 and (x["flags"] >> 4) & 7 == 0


def test_policy_rejects_out_of_range(rn):
    with pytest.raises(rn.RNError):
        rn.rn_query_policy(0, 10, 65536, 1, 1, CU)
    with pytest.raises(rn.RNError):
        rn.rn_query_policy(1, 10, 32768, 1, 1, CU)          # bwd bf16 rows up to 16384
    with pytest.raises(rn.RNError):
        rn.rn_query_policy(2, 10, 1000, 1, 1, CU)           # fp8 needs H % 128 == 0
    with pytest.raises(rn.RNError):
        rn.rn_query_policy(2, 10, 1024, 0, 0, CU)           # fp8 is bf16-only
    with pytest.raises(rn.RNError):
        rn.rn_query_policy(0, 10, 1024, 0, 1, CU)           # (f32 x, bf16 w) not a valid pair


def test_workspace_bytes_monotone_and_reusable(rn):
    assert rn.rn_bwd_workspace_bytes_for(0, 4096, CU) == 0
    prev = 0
    for T in (1, 2, 3, 7, 64, 255, 1000, 8192, 58497, 65536, 10 ** 6):
        b = rn.rn_bwd_workspace_bytes_for(T, 4096, CU)
        assert b >= prev and b % 256 == 0
        prev = b
    assert rn.rn_bwd_workspace_bytes_for(8192, 4096, CU) == 256 * 4096 * 4
    with pytest.raises(rn.RNError):
        rn.rn_bwd_workspace_bytes_for(10, 4097, CU)


# --- validation-only calls: every one carries an error caught before any device work.
# The pointers are fake, so these run only where no GPU is visible: on a GPU
# machine the same paths are exercised with real buffers in test_parity_gpu.py.
no_gpu = pytest.mark.skipif(__import__("torch").cuda.is_available(),
                            reason="fake-pointer validation tests run only without a GPU")
A = 0x10000          # a 16-byte aligned address that is never dereferenced
B = 0x20000000
C = 0x40000000


@no_gpu
def test_fwd_validation(rn):
    lib = rn.lib
    f = lib.rmsnorm_fwd
    # bad dtype pair
    assert f(A, 256, 0, B, 1, C, 256, C + 4096, 4, 256, 1e-6, None) == 3
    assert f(A, 256, 7, B, 1, C, 256, C + 4096, 4, 256, 1e-6, None) == 3
    # H not a multiple of the vector width / out of range
    assert f(A, 256, 1, B, 1, C, 256, C + 4096, 4, 250, 1e-6, None) == 2
    assert f(A, 40000, 1, B, 1, C, 40000, C + 4096, 4, 40000, 1e-6, None) == 2
    assert f(A, 256, 1, B, 1, C, 256, C + 4096, -1, 256, 1e-6, None) == 2
    # T == 0: nothing to do, nothing touched (null pointers allowed)
    assert f(None, 256, 1, None, 1, None, 256, None, 0, 256, 1e-6, None) == 0
    # null pointers
    assert f(None, 256, 1, B, 1, C, 256, C + 4096, 4, 256, 1e-6, None) == 1
    assert f(A, 256, 1, B, 1, C, 256, None, 4, 256, 1e-6, None) == 1
    # misaligned
    assert f(A + 2, 256, 1, B, 1, C, 256, C + 4096, 4, 256, 1e-6, None) == 4
    assert f(A, 256, 1, B + 8, 1, C, 256, C + 4096, 4, 256, 1e-6, None) == 4
    assert f(A, 256, 1, B, 1, C, 256, C + 4098, 4, 256, 1e-6, None) == 4
    # strides
    assert f(A, 255, 1, B, 1, C, 256, C + 4096, 4, 256, 1e-6, None) == 5
    assert f(A, 260, 1, B, 1, C, 256, C + 4096, 4, 256, 1e-6, None) == 5      # 520 B, not 16-B multiple
    # aliasing: y overlaps x; rstd inside y
    assert f(A, 256, 1, B, 1, A + 512, 256, C, 4, 256, 1e-6, None) == 7
    assert f(A, 256, 1, B, 1, C, 256, C + 16, 4, 256, 1e-6, None) == 7


@no_gpu
def test_bwd_validation(rn):
    f = rn.lib.rmsnorm_bwd
    args = dict(dy=A, lddy=256, x=A + 0x100000, ldx=256, xd=1, w=B, wd=1, rstd=B + 0x1000,
                dx=C, lddx=256, dw=C + 0x100000, T=4, H=256, det=1, ws=C + 0x200000, wsb=1 << 20)

    def call(**kw):
        a = dict(args)
        a.update(kw)
        return f(a["dy"], a["lddy"], a["x"], a["ldx"], a["xd"], a["w"], a["wd"], a["rstd"], a["dx"],
                 a["lddx"], a["dw"], a["T"], a["H"], a["det"], a["ws"], a["wsb"], None)

    assert call(xd=0, wd=1) == 3
    assert call(H=252) == 2
    assert call(H=16392) == 2                      # beyond the backward's range for bf16 rows
    assert call(dw=None) == 1
    assert call(dy=None) == 1
    assert call(dw=C + 0x100002) == 4
    assert call(x=A + 0x100008) == 4
    assert call(lddx=100) == 5
    assert call(dx=A + 64) == 7                    # dx overlaps dy
    assert call(dw=A + 64) == 7                    # dw inside dy
    # T = 4 rows of 256 fit one strip: no workspace is used, so none is required (the call then
    # gets as far as the device query, which fails without a GPU)
    assert rn.rn_bwd_workspace_bytes_for(4, 256, CU) == 0
    assert call(ws=None, wsb=0) == 8
    assert call(ws=None, wsb=0, det=0) == 8
    assert call(ws=C + 0x200008) == 8              # an unused workspace is not inspected
    # T = 2048 rows take several strips: the partial sums need the workspace, whatever the flag
    big = dict(x=A + 0x400000, dx=C, dw=C + 0x400000, T=2048, ws=C + 0x800000)
    assert rn.rn_bwd_workspace_bytes_for(2048, 256, CU) > 0
    assert call(**dict(big, ws=None)) == 6
    assert call(**dict(big, ws=None, det=0)) == 6
    assert call(**dict(big, ws=C + 0x800008)) == 4
    assert call(**big) == 8                        # valid arguments: reaches the device query


@no_gpu
def test_fp8_validation(rn):
    f = rn.lib.add_rmsnorm_fp8_block_quant
    args = dict(x=A, ldx=256, r=A + 0x100000, ldr=256, w=B, out=C, ldo=256, sc=C + 0x100000, sld=8,
                n=C + 0x200000, ldn=256, T=4, H=256)

    def call(**kw):
        a = dict(args)
        a.update(kw)
        return f(a["x"], a["ldx"], a["r"], a["ldr"], a["w"], a["out"], a["ldo"], a["sc"], a["sld"], a["n"],
                 a["ldn"], a["T"], a["H"], 1e-6, None)

    assert call(H=200) == 2                        # not a multiple of 128
    assert call(H=1000) == 2
    assert call(T=-1) == 2
    assert call(T=0, x=None, r=None, w=None, out=None, sc=None, n=None) == 0
    assert call(out=None) == 1
    assert call(out=C + 8) == 4
    assert call(sc=C + 0x100002) == 4
    assert call(ldo=200) == 5
    assert call(sld=3) == 5                        # scale_ld < T
    assert call(sld=6) == 5                        # scale_ld % 4 != 0
    assert call(n=A + 16) == 7                     # normed overlaps x
    assert call(sc=C + 64) == 7                    # scales inside out
    assert call(r=A) == 7                          # residual is x


@no_gpu
def test_fwd_residual_validation(rn):
    f = rn.lib.rmsnorm_fwd_residual
    args = dict(x=A, ldx=256, u=A + 0x100000, ldu=256, xd=1, w=B, wd=1, y=C, ldy=256, h=C + 0x100000, ldh=256,
                r=C + 0x200000, T=4, H=256)

    def call(**kw):
        a = dict(args)
        a.update(kw)
        return f(a["x"], a["ldx"], a["u"], a["ldu"], a["xd"], a["w"], a["wd"], a["y"], a["ldy"], a["h"], a["ldh"],
                 a["r"], a["T"], a["H"], 1e-6, None)

    assert call(xd=0, wd=1) == 3
    assert call(H=250) == 2
    assert call(T=0, x=None, u=None, w=None, y=None, h=None, r=None) == 0
    assert call(u=None) == 1
    assert call(h=None) == 1
    assert call(u=A + 0x100008) == 4
    assert call(ldh=250) == 5
    assert call(h=A + 64) == 7                     # h_out overlaps x without being x
    assert call(h=A + 0x100000 + 64) == 7          # h_out overlaps u without being u
    assert call(h=A, ldh=264) == 7                 # x itself but another stride
    assert call(y=A + 0x100000) == 7               # y overlaps u
    assert call(h=C + 16) == 7                     # h_out overlaps y


@no_gpu
def test_bwd_residual_validation(rn):
    f = rn.lib.rmsnorm_bwd_residual
    args = dict(dy=A, lddy=256, x=A + 0x100000, ldx=256, xd=1, w=B, wd=1, rstd=B + 0x1000, g=A + 0x200000,
                ldg=256, dx=C, lddx=256, dw=C + 0x100000, T=4, H=256, ws=C + 0x200000, wsb=1 << 20)

    def call(**kw):
        a = dict(args)
        a.update(kw)
        return f(a["dy"], a["lddy"], a["x"], a["ldx"], a["xd"], a["w"], a["wd"], a["rstd"], a["g"], a["ldg"],
                 a["dx"], a["lddx"], a["dw"], a["T"], a["H"], 1, a["ws"], a["wsb"], None)

    assert call(g=None) == 1
    assert call(g=A + 0x200008) == 4
    assert call(ldg=100) == 5
    assert call(g=C + 64) == 7                     # g_residual overlaps dx without being dx
    assert call(g=C, ldg=264) == 7                 # dx itself but another stride
    assert call(dw=A + 0x200000 + 64) == 7         # dw inside g_residual


@no_gpu
def test_fwd_heads_validation(rn):
    f = rn.lib.rmsnorm_fwd_heads
    # fused [T, 3*32*128] bf16 projection: q band at A, token stride 12288, head stride 128
    args = dict(x=A, ldt=12288, ldh=128, xd=1, w=B, wd=1, y=C, ldyt=4096, ldyh=128, r=C + 0x1000000, T=4,
                nh=32, D=128)

    def call(**kw):
        a = dict(args)
        a.update(kw)
        return f(a["x"], a["ldt"], a["ldh"], a["xd"], a["w"], a["wd"], a["y"], a["ldyt"], a["ldyh"], a["r"],
                 a["T"], a["nh"], a["D"], 1e-6, None)

    assert call(xd=0, wd=1) == 3
    assert call(D=100) == 2                        # not a vector multiple
    assert call(D=2048) == 2                       # beyond 128 vectors
    assert call(nh=0) == 2
    assert call(T=1 << 26, nh=64) == 2             # T*heads beyond 2^31
    assert call(T=0, x=None, w=None, y=None, r=None) == 0
    assert call(y=None) == 1
    assert call(x=A + 2) == 4
    assert call(r=C + 0x1000002) == 4
    assert call(ldh=100) == 5                      # heads overlap each other
    assert call(ldh=132) == 5                      # 264 B: not a 16-byte multiple
    assert call(ldt=4000) == 5                     # heads spill past the token stride
    assert call(y=A + 16) == 7                     # y overlaps x without being x
    assert call(y=A, ldyt=12288, ldyh=256) == 7    # x itself but other strides
    assert call(r=C + 64) == 7                     # rstd inside y


@no_gpu
def test_fp8_quant_validation(rn):
    f = rn.lib.add_rmsnorm_fp8_quant
    args = dict(x=A, ldx=256, r=A + 0x100000, ldr=256, w=B, dt=2, out=C, ldo=256, fmt=1, sc=C + 0x100000, sld=8,
                ts=None, n=C + 0x200000, ldn=256, T=4, H=256)

    def call(**kw):
        a = dict(args)
        a.update(kw)
        return f(a["x"], a["ldx"], a["r"], a["ldr"], a["w"], a["dt"], a["out"], a["ldo"], a["fmt"], a["sc"],
                 a["sld"], a["ts"], a["n"], a["ldn"], a["T"], a["H"], 1e-6, None)

    assert call(dt=0) == 3                         # fp32 rows are not a producer dtype
    assert call(dt=7) == 3
    assert call(fmt=2) == 3
    assert call(H=200) == 2
    assert call(T=0, x=None, r=None, w=None, out=None, sc=None, n=None) == 0
    assert call(ts=B + 0x1000) == 1                # both scale forms
    assert call(sc=None) == 1                      # neither
    assert call(sc=None, ts=B + 0x1002) == 4       # misaligned per-tensor scale
    assert call(sc=None, ts=C + 64) == 7           # per-tensor scale inside out
    assert call(sld=3) == 5
    assert call(n=A + 16) == 7


def test_small_t_backward_is_one_strip_on_any_device(rn):
    """Few rows: one row strip (one kernel, dw written directly), whatever the CU count, so
    the bits of dw do not depend on the device; more rows: several strips."""
    for T, H, d in ((1, 4096, 1), (4, 4096, 1), (8, 2048, 1), (64, 256, 0), (2, 7168, 1), (1, 16384, 1)):
        grids = {rn.rn_query_policy(1, T, H, d, d, cu)["grid"] for cu in (8, 32, 80, 256, 304)}
        assert grids == {1}, (T, H, grids)
    for T, H, d in ((8, 4096, 1), (128, 256, 0), (300, 2048, 1)):
        g = rn.rn_query_policy(1, T, H, d, d, 256)
        assert g["grid"] > 1 and g["grid"] == rn.rn_query_policy(1, T, H, d, d, 304)["grid"]


@no_gpu
def test_bwd_noalloc_validation(rn):
    """The no-workspace backward runs the same argument checks as rmsnorm_bwd; valid
    arguments get as far as the device query (which fails without a GPU)."""
    f = rn.lib.rmsnorm_bwd_noalloc
    args = dict(dy=A, lddy=256, x=A + 0x400000, ldx=256, xd=1, w=B, wd=1, rstd=B + 0x1000,
                dx=C, lddx=256, dw=C + 0x400000, T=2048, H=256, det=1)

    def call(**kw):
        a = dict(args)
        a.update(kw)
        return f(a["dy"], a["lddy"], a["x"], a["ldx"], a["xd"], a["w"], a["wd"], a["rstd"], a["dx"],
                 a["lddx"], a["dw"], a["T"], a["H"], a["det"], None)

    assert call(xd=0, wd=1) == 3
    assert call(H=252) == 2
    assert call(dw=None) == 1
    assert call(x=A + 0x400008) == 4
    assert call(lddx=100) == 5
    assert call(dx=A + 64) == 7
    assert call() == 8                             # no workspace argument is needed
    assert call(det=0) == 8



def test_per_head_token_index_multiply_shift():
    """The per-head forward finds the token of row r as (r * m) >> (31 + l) with
    l = ceil(log2 heads) and m = ceil(2^(31+l) / heads) (division by an invariant
    integer, Granlund and Montgomery 1994).  For every head count the host accepts
    (1 .. 65535), m fits 32 bits and the quotient equals r // heads at the rows
    where an error would show first: just below and at every multiple of heads up
    to a bound, and the largest rows below 2^31."""
    import numpy as np
    top = (1 << 31) - 1
    for d in range(1, 65536):
        l = (d - 1).bit_length()
        m = ((1 << (31 + l)) + d - 1) // d
        assert m < (1 << 32)
        q = np.arange(1, 64, dtype=np.uint64)
        a = q * np.uint64(d)
        n = np.concatenate([a, a - np.uint64(1), np.arange(top - 2 * d, top + 1, dtype=np.uint64)[-64:]])
        n = n[n <= top]
        got = (n * np.uint64(m)) >> np.uint64(31 + l)
        assert np.array_equal(got, n // np.uint64(d)), d
