"""Pins of the oracle's fused residual-add + RMSNorm + FP8 e4m3 1x128 block quant.

Definitions: FlashInfer PR #4480 'Add FusedAddRMSNormFP8BlockQuant' (description:
Kernel and API; review thread: scale = amax/448, e4m3 only, scale layout
(H/128, round_up(T,4)) indexed k*stride + m), and FlashInfer commit #5741
'cake_rmsnorm_train', Summary (h_new = bf16(x + residual) is what gets normalised).

Pinned by: hand-derived codes (tests/golden/hand_examples.json); the residual
sum against exact rational arithmetic and torch's bf16 addition; the scale rule
against numpy's IEEE fp32 division; a brute-force nearest-code search; the
invariant that the block maximum always encodes to +-448; the dequantisation
error bound; a planted layout pattern; and the forward oracle (pinned in
test_oracle_rmsnorm.py) for the normed values."""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from workloads import to_bf16_bits

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_examples.json")


def bits_to_f32(b):
    return (np.asarray(b, np.uint16).astype(np.uint32) << 16).view(np.float32)


def block_from_head(head, rest=0.0):
    v = np.full(128, rest, np.float32)
    v[: len(head)] = head
    return to_bf16_bits(v).reshape(1, 128)


def test_golden_block_quant(oracle):
    for ex in json.load(open(GOLDEN))["fp8"]:
        nb = block_from_head(ex["normed_block_head"], ex["rest"])
        assert np.array_equal(bits_to_f32(nb[0, : len(ex["normed_block_head"])]),
                              np.asarray(ex["normed_block_head"], np.float32))   # exact in bf16
        scale, codes = oracle.block_quant_e4m3(nb)
        assert scale[0, 0] == np.float32(ex["scale"])
        assert list(codes[0, : len(ex["codes_head"])]) == ex["codes_head"]


def test_residual_sum_is_exactly_rounded(oracle):
    """h = bf16(x + r) for bf16 x, r: compare with the exact rational sum rounded to
    nearest-even bf16, and with torch's bf16 addition (fp32 add, then RNE)."""
    rng = np.random.default_rng(20)
    n = 3000
    xa = to_bf16_bits((rng.standard_normal(n) * np.exp2(rng.integers(-20, 20, n))).astype(np.float32))
    ra = to_bf16_bits((rng.standard_normal(n) * np.exp2(rng.integers(-20, 20, n))).astype(np.float32))
    T, H = 3, 1024
    x = np.resize(xa, (T, H)).astype(np.uint16)
    r = np.resize(ra, (T, H)).astype(np.uint16)
    w = to_bf16_bits(np.ones(H, np.float32))
    out = oracle.add_rmsnorm_fp8(x, r, w, 1e-6)
    h = out["h"]
    xt = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16)
    rt = torch.from_numpy(r.view(np.int16)).view(torch.bfloat16)
    ht = (xt + rt).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(h, ht)
    xf, rf = bits_to_f32(x.ravel()), bits_to_f32(r.ravel())
    hf = bits_to_f32(h.ravel())
    for i in range(0, T * H, 7):
        exact = Fraction(float(xf[i])) + Fraction(float(rf[i]))
        # candidates: h and its two bf16 neighbours; h must be nearest (ties: even)
        hb = int(h.ravel()[i])
        best = abs(Fraction(float(hf[i])) - exact)
        for nb in ((hb + 1) & 0xFFFF, (hb - 1) & 0xFFFF):
            v = float(bits_to_f32([nb])[0])
            if math.isfinite(v):
                d = abs(Fraction(v) - exact)
                assert d > best or (d == best and hb % 2 == 0)


def test_normed_matches_forward_oracle_on_h(oracle):
    rng = np.random.default_rng(21)
    T, H = 5, 384
    x = to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    r = to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    w = to_bf16_bits((1 + 0.1 * rng.standard_normal(H)).astype(np.float32))
    out = oracle.add_rmsnorm_fp8(x, r, w, 1e-6)
    y, rstd = oracle.rmsnorm_fwd(out["h"], w, 1e-6)
    np.testing.assert_array_equal(out["normed"], y)
    np.testing.assert_array_equal(out["rstd"], rstd)
    nb = np.array([[oracle.double_to_bf16(v) for v in row] for row in y], np.uint16)
    assert np.array_equal(out["normed_bf16"], nb)
    s2, c2 = oracle.block_quant_e4m3(out["normed_bf16"])
    np.testing.assert_array_equal(out["scale"][:, :T], s2[:, :T])
    np.testing.assert_array_equal(out["codes"], c2)


def _nearest_code(q):
    """Brute force over all finite E4M3FN values from the format definition; ties to even."""
    best, bestd = None, None
    for c in range(0x7F):                      # non-negative finite codes (0x7F is NaN)
        e, m = c >> 3, c & 7
        v = (m / 8.0) * 2.0 ** -6 if e == 0 else (1 + m / 8.0) * 2.0 ** (e - 7)
        d = abs(abs(q) - v)
        if bestd is None or d < bestd or (d == bestd and c % 2 == 0):
            best, bestd = c, d
    return best | (0x80 if math.copysign(1.0, q) < 0 else 0)


def test_block_quant_bruteforce_scale_rule_and_invariants(oracle):
    rng = np.random.default_rng(22)
    T, H = 6, 256
    vals = (rng.standard_normal((T, H)) * np.exp2(rng.integers(-8, 4, (T, H)))).astype(np.float32)
    vals[2, :128] = 0.0                                      # an all-zero block
    vals[3, 5] = -0.0
    nb = to_bf16_bits(vals)
    scale, codes = oracle.block_quant_e4m3(nb)
    nf = bits_to_f32(nb.ravel()).reshape(T, H)
    for m in range(T):
        for k in range(H // 128):
            blk = nf[m, 128 * k: 128 * k + 128]
            a = np.float32(np.max(np.abs(blk)))
            s = np.float32(a) / np.float32(448.0)           # numpy: IEEE fp32 division
            assert scale[k, m] == s
            cb = codes[m, 128 * k: 128 * k + 128]
            if a == 0:
                assert s == 0 and np.all(cb == 0)
                continue
            jmax = int(np.argmax(np.abs(blk)))
            assert cb[jmax] == (0xFE if blk[jmax] < 0 else 0x7E)   # the block max encodes to +-448
            for j in range(0, 128, 5):
                q = np.float32(blk[j]) / s
                assert cb[j] == _nearest_code(float(q)), (m, k, j)
                # dequantisation error bound: half a code spacing at |q|, times s
                dec = oracle.e4m3_to_double(int(cb[j]))
                aq = abs(float(q))
                spacing = 2.0 ** -9 if aq < 2.0 ** -6 else 2.0 ** (math.floor(math.log2(aq)) - 3)
                assert abs(dec - float(q)) <= spacing / 2 * (1 + 1e-12)
    # sign of a zero is kept in its code
    assert codes[3, 5] in (0x80, 0x00) and (codes[3, 5] == 0x80) == (math.copysign(1, nf[3, 5]) < 0)


def test_scale_layout_planted(oracle):
    """Scale of (row m, block k) sits at scale[k, m] (row index fastest); rows
    T .. ld-1 of every block column are left untouched."""
    T, H = 7, 512
    v = np.zeros((T, H), np.float32)
    for m in range(T):
        for k in range(H // 128):
            v[m, 128 * k + (m * 3 + k) % 128] = (m + 1) * 2.0 ** k * 7.0     # planted block max
    nb = to_bf16_bits(v)
    scale, _ = oracle.block_quant_e4m3(nb, scale_ld=12)
    assert scale.shape == (4, 12)
    for m in range(T):
        for k in range(4):
            assert scale[k, m] == np.float32((m + 1) * 2.0 ** k * 7.0) / np.float32(448.0)
    assert np.all(np.isnan(scale[:, T:]))
    # the view a block-scaled GEMM reads: (T, H/128) = scale[:, :T].T
    view = torch.from_numpy(scale)[:, :T].T
    assert view.shape == (T, 4) and view.stride() == (1, 12)
