"""Parity of the producer variants (add_rmsnorm_fp8_quant: fp16 rows, e5m2
codes, a given per-tensor scale) through the C ABI against the FP64 CPU
oracle, and the quotient / conversion self-tests they rely on.

Residual and codes are bit-exact; codes (and block scales) are re-derived by
the oracle from the GPU's own normed values; normed is within the bf16 rule
for bf16 rows and the same rule at fp16 spacing for fp16 rows."""
import numpy as np
import pytest
import torch

from gpu_common import to_host
from gpu_ops import check_variant, dec16, dev16, host16, lp16, run_variant
from workloads import CONFIGS, Workload, generate

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def rn():
    import bwd_fp8_block_amd as m
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return m


# ----------------------------------------------------------------------------
# self-tests: the quotient, bit for bit, and the e5m2 conversion
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("fmt", [0, 1], ids=["e4m3", "e5m2"])
@pytest.mark.parametrize("dtype", [1, 2], ids=["bf16", "f16"])
def test_quotient_block_scales_exhaustive(rn, dtype, fmt):
    """Every amax pattern of the dtype and every n with |n| <= amax: the corrected product
    equals the IEEE quotient n / (amax / MAX) bit for bit."""
    mism = torch.zeros(1, dtype=torch.int64, device="cuda")
    first = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    top = 0x7f7f if dtype == 1 else 0x7bff
    for lo in range(1, top + 1, 8192):
        rn.rn_selftest_quotient(dtype, fmt, mism, first, a_lo=lo, a_hi=min(lo + 8191, top))
    torch.cuda.synchronize()
    assert int(mism.item()) == 0, "first mismatch at 0x%08x" % (int(first.item()) & 0xFFFFFFFF)


@pytest.mark.parametrize("fmt", [0, 1], ids=["e4m3", "e5m2"])
@pytest.mark.parametrize("dtype", [1, 2], ids=["bf16", "f16"])
def test_quotient_tensor_scale(rn, dtype, fmt):
    """Per-tensor scales: 4096 log-uniform scales in [2^-90, 2^90] plus edge values, against
    every finite n of the dtype (both signs)."""
    rng = np.random.default_rng(80 + dtype + fmt)
    s = np.exp2(rng.uniform(-90, 90, 4000)).astype(np.float32)
    edge = [1.0, 2.0, 0.5, 1 / 3, 448.0, 57344.0, 1 / 448, 1 / 57344, 2.0 ** -100, 2.0 ** 100, 3e-5, 7.0,
            np.nextafter(np.float32(1), np.float32(2)), np.nextafter(np.float32(1), np.float32(0))]
    s = np.concatenate([s, np.array(edge, np.float32)])
    s = s[s >= np.float32(2.0 ** -100)]
    mism = torch.zeros(1, dtype=torch.int64, device="cuda")
    first = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    rn.rn_selftest_quotient(dtype, fmt, mism, first, scales=torch.from_numpy(s).cuda())
    torch.cuda.synchronize()
    assert int(mism.item()) == 0, "first mismatch at 0x%08x" % (int(first.item()) & 0xFFFFFFFF)


def test_cvt_e5m2_matches_oracle_encoder(rn, oracle):
    mags = sorted({abs(oracle.e5m2_to_double(c)) for c in range(0x7C)})
    pts = []
    for lo, hi in zip(mags[:-1], mags[1:]):
        m = np.float32((lo + hi) / 2)
        pts += [m, np.nextafter(m, np.float32(0)), np.nextafter(m, np.float32(1e9)), np.float32(lo)]
    pts += [np.float32(57344.0) * np.float32(1 + k * 2.0 ** -23) for k in range(16)]
    pts += [np.float32(2.0 ** -17), np.float32(0.0), np.float32(1e-30), np.float32(57400.0)]
    rng = np.random.default_rng(81)
    rnd = (rng.uniform(-1, 1, 200000) * np.exp2(rng.integers(-18, 17, 200000))).astype(np.float32)
    v = np.concatenate([np.array(pts, np.float32), -np.array(pts, np.float32), rnd])
    v = v[np.abs(v) <= 57344.0 * 1.001]
    out = torch.empty(v.size, dtype=torch.uint8, device="cuda")
    rn.rn_selftest_cvt_e5m2(torch.from_numpy(v).cuda(), out)
    got = to_host(out)
    ref = np.array([oracle.float_to_e5m2(x) for x in v], np.uint8)
    bad = np.flatnonzero(got != ref)
    assert bad.size == 0, "first mismatch: value %r gpu 0x%02x oracle 0x%02x" % (v[bad[0]], got[bad[0]], ref[bad[0]])


# ----------------------------------------------------------------------------
# the producer variants
# ----------------------------------------------------------------------------

VARIANT_CASES = [(1, 128, 0), (3, 256, 16), (64, 1152, 0), (129, 2048, 128), (7, 4096, 0), (33, 7168, 0),
                 (3, 16384, 0), (2, 32768, 0), (300, 1024, 0),
                 # long runs over many windows (ragged last window), and the widest rows
                 (4099, 5120, 64), (1201, 32768, 0)]


@pytest.mark.parametrize("mode", ["block", "tensor"])
@pytest.mark.parametrize("dtype,fmt", [("f16", "e4m3"), ("bf16", "e5m2"), ("f16", "e5m2"), ("bf16", "e4m3")])
@pytest.mark.parametrize("T,H,pad", VARIANT_CASES)
def test_variant_parity(rn, oracle, T, H, pad, dtype, fmt, mode):
    rng = np.random.default_rng(9000 + T + H)
    x = lp16(rng.standard_normal((T, H)), dtype)
    res = lp16(rng.standard_normal((T, H)), dtype)
    w = lp16(1 + 0.1 * rng.standard_normal(H), dtype)
    ts = None if mode == "block" else float(np.float32(0.01 if fmt == "e4m3" else 2.0 ** -12))
    h, out, scale, normed = run_variant(rn, x, res, w, dtype, fmt, ts, ld_pad=pad)
    check_variant(oracle, x, res, w, dtype, fmt, ts, h, out, scale, normed)


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_tensor_scale_saturation_and_signs(rn, oracle, fmt):
    """A per-tensor scale small enough that most quotients saturate at +-MAX, one large
    enough that most round to (signed) zero, and a row that cancels to zero."""
    T, H = 6, 512
    rng = np.random.default_rng(82)
    x = lp16(rng.standard_normal((T, H)), "bf16")
    res = lp16(rng.standard_normal((T, H)), "bf16")
    res[0] = x[0] ^ 0x8000
    w = lp16(1 + 0.1 * rng.standard_normal(H), "bf16")
    for ts in (1e-6, 1e3, 2.0 ** -100, 3.0e38):
        h, out, _, normed = run_variant(rn, x, res, w, "bf16", fmt, float(np.float32(ts)))
        check_variant(oracle, x, res, w, "bf16", fmt, float(np.float32(ts)), h, out, None, normed)


def test_variant_without_normed_matches(rn, oracle):
    T, H = 17, 2048
    rng = np.random.default_rng(83)
    x = lp16(rng.standard_normal((T, H)), "f16")
    res = lp16(rng.standard_normal((T, H)), "f16")
    w = lp16(1 + 0.1 * rng.standard_normal(H), "f16")
    for ts in (None, 0.004):
        _, o1, s1, n1 = run_variant(rn, x, res, w, "f16", "e5m2", ts)
        _, o2, s2, n2 = run_variant(rn, x, res, w, "f16", "e5m2", ts, with_normed=False)
        assert n2 is None and np.array_equal(o1, o2)
        if s1 is not None:
            assert np.array_equal(s1[:, :T], s2[:, :T])


def test_variant_base_form_is_the_block_quant_entry(rn):
    """bf16 / e4m3 / block scales through the general entry point gives the same bits as
    add_rmsnorm_fp8_block_quant."""
    T, H = 40, 1024
    d = generate(Workload("v", T, H, "bf16", "bf16", residual=True, seed=84))
    h1, o1, s1, n1 = run_variant(rn, d["x"], d["residual"], d["w"], "bf16", "e4m3")
    xd, wd = dev16(d["x"], "bf16"), dev16(d["w"], "bf16")
    r = dev16(d["residual"], "bf16").clone()
    o = torch.empty(T, H, dtype=torch.uint8, device="cuda")
    s = torch.full((H // 128, (T + 3) // 4 * 4 + 4), float("nan"), device="cuda")
    n = torch.empty(T, H, dtype=torch.bfloat16, device="cuda")
    rn.add_rmsnorm_fp8_block_quant(xd, r, wd, o, s, n, 1e-6)
    torch.cuda.synchronize()
    assert np.array_equal(host16(r), h1) and np.array_equal(to_host(o), o1)
    assert np.array_equal(host16(n), n1) and np.array_equal(to_host(s)[:, :T], s1[:, :T])


def test_variant_validation(rn):
    T, H = 4, 256
    x = torch.randn(T, H, device="cuda").to(torch.float16)
    r = torch.randn(T, H, device="cuda").to(torch.float16)
    w = torch.ones(H, dtype=torch.float16, device="cuda")
    o = torch.zeros(T, H, dtype=torch.uint8, device="cuda")
    s = torch.full((H // 128, 4), 5.0, device="cuda")
    ts = torch.tensor([0.5], device="cuda")
    f = rn.lib.add_rmsnorm_fp8_quant
    st = rn._stream(x.device)
    base = [x.data_ptr(), H, r.data_ptr(), H, w.data_ptr(), 2, o.data_ptr(), H, 1]
    tail = [None, 0, T, H, 1e-6, st]
    assert f(*base, s.data_ptr(), 4, ts.data_ptr(), *tail) == 1         # both scale forms
    assert f(*base, None, 0, None, *tail) == 1                           # neither
    assert f(*(base[:5] + [3] + base[6:]), s.data_ptr(), 4, None, *tail) == 3     # unknown dtype
    assert f(*(base[:8] + [2]), s.data_ptr(), 4, None, *tail) == 3                # unknown format
    assert f(*base, None, 0, o.data_ptr(), *tail) == 7                  # tensor scale inside out
    torch.cuda.synchronize()
    assert torch.all(o == 0) and torch.all(s == 5.0)


@pytest.mark.parametrize("name,dtype,fmt,ts", [("fp8_T4096_H7168", "f16", "e5m2", None),
                                               ("fp8_T8192_H4096", "bf16", "e4m3", 0.0125),
                                               ("fp8_T8192_H4096", "f16", "e4m3", None)])
def test_config_variants(rn, oracle, name, dtype, fmt, ts):
    wl = CONFIGS[name]
    d = generate(wl)
    if dtype == "f16":            # the same draws, rounded to fp16 instead of bf16
        conv = lambda b: lp16(dec16(b, "bf16"), "f16")
        x, res, w = conv(d["x"]), conv(d["residual"]), conv(d["w"])
    else:
        x, res, w = d["x"], d["residual"], d["w"]
    h, out, scale, normed = run_variant(rn, x, res, w, dtype, fmt, ts, eps=wl.eps)
    check_variant(oracle, x, res, w, dtype, fmt, ts, h, out, scale, normed, eps=wl.eps)
