"""Pins of the oracle's producer variants: fp16 rows, e5m2 codes, and a given
per-tensor scale (FlashInfer PR #4480: description, test matrix over fp16 and
bf16 inputs, review thread on the bound tied to the output type).

* fp16 codec: every pattern against numpy's float16, rounding against numpy
  on random values and on constructed ties;
* E5M2 codec: every pattern against torch's float8_e5m2, rounding against
  torch wherever torch does not overflow to infinity, hand-derived codes
  (ties, subnormals, saturation);
* the general producer reduces, for bf16 rows, e4m3 codes and block scales,
  to the already pinned fused producer, bit for bit;
* fp16 rows: h against IEEE fp32 addition then numpy's rounding to fp16;
  normed against the pinned forward on the decoded h;
* per-tensor scale: a hand-derived row; scaling n and s by a power of two
  leaves the codes unchanged; codes against a brute-force nearest search;
* e5m2 block scales: scale = amax / 57344 against numpy's fp32 division, the
  block maximum always encodes to +-57344."""
import json
import math
import os

import numpy as np
import pytest
import torch

from workloads import to_bf16_bits

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_examples.json")


def test_f16_decode_all_patterns(oracle):
    pats = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = pats.view(np.float16).astype(np.float64)
    got = np.array([oracle.f16_to_double(int(p)) for p in pats])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])


def test_f16_encode_against_numpy(oracle):
    rng = np.random.default_rng(71)
    v = rng.standard_normal(20000) * np.exp2(rng.integers(-28, 17, 20000))
    # exact midpoints between neighbouring fp16 values (ties) and their neighbours in double
    a = np.sort(np.abs(rng.standard_normal(2000) * 100).astype(np.float16)).astype(np.float64)
    b = np.nextafter(a.astype(np.float16), np.float16(np.inf)).astype(np.float64)
    mids = (a + b) / 2
    v = np.concatenate([v, mids, -mids, np.nextafter(mids, 0), np.nextafter(mids, np.inf), [0.0, -0.0, 65504.0]])
    v = v[np.abs(v) < 65504.0]
    got = np.array([oracle.double_to_f16(x) for x in v], dtype=np.uint16)
    ref = v.astype(np.float16).view(np.uint16)
    assert np.array_equal(got, ref)


def test_e5m2_decode_all_patterns(oracle):
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e5m2).to(torch.float64).numpy()
    got = np.array([oracle.e5m2_to_double(c) for c in range(256)])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])


def test_e5m2_encode_against_torch_and_by_hand(oracle):
    rng = np.random.default_rng(72)
    v = (rng.standard_normal(50000) * np.exp2(rng.integers(-20, 16, 50000))).astype(np.float32)
    grid = np.array([abs(oracle.e5m2_to_double(c)) for c in range(0x7C)])
    mids = ((grid[:-1] + grid[1:]) / 2).astype(np.float32)
    v = np.concatenate([v, mids, -mids, np.nextafter(mids, np.float32(0)), np.nextafter(mids, np.float32(1e9))])
    v = v[np.abs(v) < 61440.0]                      # beyond, torch overflows to infinity
    got = np.array([oracle.float_to_e5m2(x) for x in v], dtype=np.uint8)
    ref = torch.from_numpy(v).to(torch.float8_e5m2).view(torch.uint8).numpy()
    assert np.array_equal(got, ref)
    for ex in json.load(open(GOLDEN))["e5m2"]:
        got = [oracle.float_to_e5m2(x) for x in ex["values"]]
        assert got == ex["codes"]
    assert oracle.float_to_e5m2(np.float32(np.inf)) == 0x7B and oracle.float_to_e5m2(np.float32(-np.inf)) == 0xFB


def _bits(a, dtype):
    a = np.asarray(a, np.float32)
    return to_bf16_bits(a) if dtype == "bf16" else a.astype(np.float16).view(np.uint16)


def _dec(b, dtype):
    if dtype == "bf16":
        return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return b.view(np.float16).astype(np.float64)


def test_general_producer_reduces_to_the_pinned_one(oracle):
    rng = np.random.default_rng(73)
    T, H = 6, 384
    x = _bits(rng.standard_normal((T, H)), "bf16")
    r = _bits(rng.standard_normal((T, H)), "bf16")
    w = _bits(1 + 0.1 * rng.standard_normal(H), "bf16")
    a = oracle.add_rmsnorm_fp8(x, r, w, 1e-6)
    b = oracle.add_rmsnorm_quant(x, r, w, 1e-6, "bf16", "e4m3")
    assert np.array_equal(a["h"], b["h"]) and np.array_equal(a["normed_bf16"], b["normed_lp"])
    assert np.array_equal(a["rstd"], b["rstd"]) and np.array_equal(a["normed"], b["normed"])
    assert np.array_equal(a["scale"][:, :T], b["scale"][:, :T]) and np.array_equal(a["codes"], b["codes"])


def test_f16_producer_h_and_normed(oracle):
    rng = np.random.default_rng(74)
    T, H = 5, 256
    x = _bits(rng.standard_normal((T, H)) * 4, "f16")
    r = _bits(rng.standard_normal((T, H)) * np.exp2(rng.integers(-14, 3, (T, H))), "f16")
    w = _bits(1 + 0.1 * rng.standard_normal(H), "f16")
    out = oracle.add_rmsnorm_quant(x, r, w, 1e-6, "f16", "e4m3")
    # IEEE fp32 addition then rounding to fp16 (fp32 carries more than 2*11+2 bits)
    href = (x.view(np.float16).astype(np.float32) + r.view(np.float16).astype(np.float32)).astype(np.float16)
    assert np.array_equal(out["h"], href.view(np.uint16))
    y, rstd = oracle.rmsnorm_fwd(_dec(out["h"], "f16").astype(np.float32), _dec(w, "f16").astype(np.float32), 1e-6)
    assert np.array_equal(out["normed"], y) and np.array_equal(out["rstd"], rstd)
    assert np.array_equal(out["normed_lp"], y.astype(np.float16).view(np.uint16))


def test_tensor_scale_hand_example(oracle):
    ex = json.load(open(GOLDEN))["tensor_quant"][0]
    row = np.zeros(128, np.float32)
    row[:len(ex["normed_head"])] = ex["normed_head"]
    nb = to_bf16_bits(row).reshape(1, 128)
    assert np.array_equal(_dec(nb, "bf16")[0], row.astype(np.float64)), "example values must be exact in bf16"
    scale, codes = oracle.quant_lp(nb, "bf16", "e4m3", tensor_scale=ex["scale"])
    assert scale is None
    assert codes[0, :len(ex["codes_head"])].tolist() == ex["codes_head"]
    assert np.all(codes[0, len(ex["codes_head"]):] == 0)


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_tensor_scale_invariance_and_brute_force(oracle, fmt, dtype):
    rng = np.random.default_rng(75)
    T, H = 4, 256
    n = _bits(rng.standard_normal((T, H)) * 3, dtype)
    s = np.float32(0.0137)
    _, c1 = oracle.quant_lp(n, dtype, fmt, tensor_scale=float(s))
    n4 = _bits(_dec(n, dtype) * 4, dtype)                  # exact: power of two, in range
    assert np.array_equal(_dec(n4, dtype), _dec(n, dtype) * 4)
    _, c4 = oracle.quant_lp(n4, dtype, fmt, tensor_scale=float(s * np.float32(4)))
    assert np.array_equal(c1, c4)
    # brute force: the code is the nearest grid value to the fp32 quotient, ties to even, saturated
    dec = oracle.e4m3_to_double if fmt == "e4m3" else oracle.e5m2_to_double
    mx = 448.0 if fmt == "e4m3" else 57344.0
    grid = np.array([dec(c) for c in range(0x80)])
    ok = ~np.isnan(grid) & (np.abs(grid) <= mx)
    cand = np.flatnonzero(ok)
    q = (_dec(n, dtype).astype(np.float32) / s).astype(np.float64)
    for qi, ci in zip(q.ravel()[:300], c1.ravel()[:300]):
        a = min(abs(qi), mx)
        d = np.abs(grid[cand] - a)
        best = cand[d == d.min()]
        exp = best[0] if len(best) == 1 else best[best % 2 == 0][0]
        assert (ci & 0x7F) == exp and (ci >> 7) == (1 if math.copysign(1, qi) < 0 else 0)


def test_e5m2_block_scales(oracle):
    rng = np.random.default_rng(76)
    T, H = 7, 512
    for dtype in ("bf16", "f16"):
        x = _bits(rng.standard_normal((T, H)), dtype)
        r = _bits(rng.standard_normal((T, H)), dtype)
        w = _bits(1 + 0.1 * rng.standard_normal(H), dtype)
        out = oracle.add_rmsnorm_quant(x, r, w, 1e-6, dtype, "e5m2")
        nl = _dec(out["normed_lp"], dtype)
        amax = np.abs(nl).reshape(T, H // 128, 128).max(axis=2).astype(np.float32)
        assert np.array_equal(out["scale"][:, :T].T, amax / np.float32(57344.0))
        blocks = out["codes"].reshape(T, H // 128, 128)
        arg = np.abs(nl).reshape(T, H // 128, 128).argmax(axis=2)
        top = np.take_along_axis(blocks, arg[..., None], axis=2)[..., 0]
        assert np.all((top & 0x7F) == 0x7B)
