"""Pins of the oracle's bf16 and E4M3FN codecs against things other than itself:
torch's dtype conversions (library routines), exhaustive round trips, a
brute-force nearest-value search written here from the formats' definitions,
and hand-derived edge values.

The codecs implement the storage formats the pages name: bf16 activations and
weights, and fp8 e4m3 codes (FlashInfer PR #4480 'Add FusedAddRMSNormFP8BlockQuant',
description and review thread: e4m3 only, largest finite 448)."""
import math

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.filterwarnings("ignore")


def all_bf16_values():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    vals = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    return bits, vals


def test_bf16_decode_exhaustive(oracle):
    bits, ref = all_bf16_values()
    got = np.array([oracle.bf16_to_double(int(b)) for b in bits])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    # sign of zero is kept
    assert math.copysign(1.0, oracle.bf16_to_double(0x8000)) == -1.0


def test_bf16_encode_matches_torch_on_fp32(oracle):
    rng = np.random.default_rng(1)
    # wide exponent range, plus values exactly halfway between bf16 neighbours
    v = (rng.standard_normal(20000) * np.exp2(rng.integers(-130, 120, 20000))).astype(np.float32)
    ties = (np.arange(5000, dtype=np.uint32) << 16 | 0x8000).view(np.float32)   # bf16 bits + half ulp
    v = np.concatenate([v, ties[np.isfinite(ties)], np.array([0.0, -0.0, 1.0, -1.0], np.float32)])
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = np.array([oracle.double_to_bf16(float(x)) for x in v], dtype=np.uint16)
    assert np.array_equal(got, ref)


def nearest_bf16_bruteforce(v, pos_vals, pos_bits):
    """Nearest bf16 (ties to the even pattern) by search over all finite values."""
    a = abs(v)
    i = np.searchsorted(pos_vals, a)
    cands = [j for j in (i - 1, i) if 0 <= j < len(pos_vals)]
    best = min(cands, key=lambda j: (abs(pos_vals[j] - a), pos_bits[j] & 1))
    b = int(pos_bits[best])
    return b | (0x8000 if math.copysign(1.0, v) < 0 else 0)


def test_bf16_encode_from_double_bruteforce(oracle):
    bits, vals = all_bf16_values()
    fin = np.isfinite(vals) & (vals >= 0) & (bits < 0x8000)
    pos_vals, pos_bits = vals[fin], bits[fin]
    order = np.argsort(pos_vals, kind="stable")
    pos_vals, pos_bits = pos_vals[order], pos_bits[order]
    rng = np.random.default_rng(2)
    v = rng.standard_normal(4000) * np.exp2(rng.integers(-60, 60, 4000))
    # doubles just off the bf16 midpoints (the case a double -> fp32 -> bf16 path gets wrong)
    mids = (pos_vals[100:2100] + pos_vals[101:2101]) / 2
    v = np.concatenate([v, mids, mids * (1 + 2.0 ** -40), mids * (1 - 2.0 ** -40), -mids])
    for x in v:
        assert oracle.double_to_bf16(float(x)) == nearest_bf16_bruteforce(float(x), pos_vals, pos_bits), x


def e4m3_values_from_definition():
    """All 256 E4M3FN codes decoded from the format definition (bias 7, 3 mantissa bits,
    subnormals m/8 * 2^-6, S.1111.111 = NaN), written independently of the oracle."""
    out = {}
    for c in range(256):
        s = -1.0 if c & 0x80 else 1.0
        e = (c >> 3) & 0xF
        m = c & 7
        if e == 15 and m == 7:
            out[c] = float("nan")
        elif e == 0:
            out[c] = s * m / 8.0 * 2.0 ** -6
        else:
            out[c] = s * (1 + m / 8.0) * 2.0 ** (e - 7)
    return out


def test_e4m3_decode_matches_torch_and_definition(oracle):
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    defn = e4m3_values_from_definition()
    for c in range(256):
        got = oracle.e4m3_to_double(c)
        if math.isnan(ref[c]):
            assert math.isnan(got) and math.isnan(defn[c])
        else:
            assert got == ref[c] == defn[c]
            assert math.copysign(1.0, got) == math.copysign(1.0, ref[c])
    assert oracle.e4m3_to_double(0x7E) == 448.0 and oracle.e4m3_to_double(0x01) == 2.0 ** -9


def test_e4m3_roundtrip_every_code(oracle):
    for c in range(256):
        v = oracle.e4m3_to_double(c)
        if math.isnan(v):
            continue
        assert oracle.float_to_e4m3(v) == c


def sorted_e4m3_magnitudes():
    defn = e4m3_values_from_definition()
    mags = sorted((v, c) for c, v in defn.items() if c < 0x80 and not math.isnan(v))
    return [v for v, _ in mags], [c for _, c in mags]


def test_e4m3_midpoints_round_to_even(oracle):
    vals, codes = sorted_e4m3_magnitudes()
    for i in range(len(vals) - 1):
        lo, hi = vals[i], vals[i + 1]
        mid = np.float32((lo + hi) / 2)          # exact in fp32 for every pair
        assert float(mid) == (lo + hi) / 2
        even = codes[i] if codes[i] % 2 == 0 else codes[i + 1]
        for sgn in (1.0, -1.0):
            sbit = 0x80 if sgn < 0 else 0
            assert oracle.float_to_e4m3(np.float32(sgn) * mid) == even | sbit
            above = np.nextafter(mid, np.float32(np.inf))
            below = np.nextafter(mid, np.float32(0))
            assert oracle.float_to_e4m3(np.float32(sgn) * above) == codes[i + 1] | sbit
            assert oracle.float_to_e4m3(np.float32(sgn) * below) == codes[i] | sbit


def test_e4m3_subnormal_and_saturation_edges(oracle):
    f = oracle.float_to_e4m3
    assert f(2.0 ** -10) == 0x00                     # halfway 0 .. 2^-9 -> even (0)
    assert f(np.nextafter(np.float32(2.0 ** -10), np.float32(1))) == 0x01
    assert f(-(2.0 ** -10)) == 0x80                  # sign kept on a zero result
    assert f(1.5 * 2.0 ** -9) == 0x02                # halfway 1 .. 2 -> even (2)
    assert f(2.0 ** -6) == 0x08                      # smallest normal
    assert f(448.0) == 0x7E and f(-448.0) == 0xFE
    assert f(460.0) == 0x7E                          # below the 464 midpoint
    assert f(464.0) == 0x7E and f(1e30) == 0x7E      # saturating (satfinite reading)
    assert f(-1e30) == 0xFE
    assert f(0.0) == 0x00 and f(-0.0) == 0x80


def test_e4m3_encode_bruteforce_and_torch(oracle):
    vals, codes = sorted_e4m3_magnitudes()
    vals = np.array(vals)
    rng = np.random.default_rng(3)
    v = (rng.uniform(-1, 1, 30000) * np.exp2(rng.integers(-14, 10, 30000))).astype(np.float32)
    v = v[np.abs(v) < 464]
    ref_torch = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    for x, rt in zip(v, ref_torch):
        a = abs(float(x))
        d = np.abs(vals - a)
        k = np.flatnonzero(d == d.min())
        best = min(k, key=lambda j: codes[j] % 2)      # ties -> even code
        want = codes[best] | (0x80 if math.copysign(1.0, float(x)) < 0 else 0)
        got = oracle.float_to_e4m3(x)
        assert got == want, (x, got, want)
        assert got == rt, (x, got, rt)
