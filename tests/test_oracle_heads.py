"""Pins of the oracle's per-head RMSNorm (QK-norm): every (token, head) slice
of head_dim values is one row with a shared weight.

* a hand-derived example whose head and token strides leave padding between
  and after the heads (padding values would change every result if read);
* the gathered-rows identity: the result equals the plain forward on the rows
  gathered into a dense [T*heads, head_dim] array by numpy indexing;
* heads = 1 is the plain forward with the token stride as the row stride;
* permuting heads permutes the outputs.

Definition: FlashInfer PR #6332 (QKV projection + QK-RMSNorm + RoPE overlapped
with the Ulysses head exchange), Description, operator math."""
import json
import os

import numpy as np
import pytest

from workloads import to_bf16_bits

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_examples.json")


def test_golden_heads(oracle):
    for ex in json.load(open(GOLDEN))["fwd_heads"]:
        x = np.asarray(ex["x_rows"], np.float32)
        assert x.shape[1] == ex["ld_token"]
        w = np.asarray(ex["w"], np.float32)
        y, rstd = oracle.rmsnorm_fwd_heads(x, ex["heads"], ex["head_dim"], w, ex["eps"], ld_head=ex["ld_head"])
        np.testing.assert_allclose(rstd, ex["rstd"], rtol=1e-15)
        np.testing.assert_allclose(y, ex["y"], rtol=1e-15, atol=1e-300)


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_gathered_rows_identity(oracle, dt):
    rng = np.random.default_rng(51)
    T, nh, D = 9, 4, 64
    qkv = rng.standard_normal((T, 3 * nh * D)).astype(np.float32)
    w = (1 + 0.1 * rng.standard_normal(D)).astype(np.float32)
    if dt == "bf16":
        qkv, w = to_bf16_bits(qkv), to_bf16_bits(w)
    for part in range(2):                                   # the q and the k band of a fused projection
        view = qkv[:, part * nh * D:]
        y, rstd = oracle.rmsnorm_fwd_heads(view, nh, D, w, 1e-6)
        dense = np.ascontiguousarray(qkv[:, part * nh * D:(part + 1) * nh * D].reshape(T * nh, D))
        yr, rr = oracle.rmsnorm_fwd(dense, w, 1e-6)
        np.testing.assert_array_equal(y.reshape(T * nh, D), yr)
        np.testing.assert_array_equal(rstd.reshape(T * nh), rr)


def test_single_head_is_plain_forward(oracle):
    rng = np.random.default_rng(52)
    x = rng.standard_normal((7, 40)).astype(np.float32)
    w = (1 + 0.1 * rng.standard_normal(32)).astype(np.float32)
    y, rstd = oracle.rmsnorm_fwd_heads(x, 1, 32, w, 1e-6)
    yr, rr = oracle.rmsnorm_fwd(x[:, :32], w, 1e-6)
    np.testing.assert_array_equal(y[:, 0, :], yr)
    np.testing.assert_array_equal(rstd[:, 0], rr)


def test_head_permutation(oracle):
    rng = np.random.default_rng(53)
    T, nh, D = 5, 6, 16
    x = rng.standard_normal((T, nh * D)).astype(np.float32)
    w = (1 + 0.1 * rng.standard_normal(D)).astype(np.float32)
    perm = rng.permutation(nh)
    xp = np.ascontiguousarray(x.reshape(T, nh, D)[:, perm, :].reshape(T, nh * D))
    y, rstd = oracle.rmsnorm_fwd_heads(x, nh, D, w, 1e-6)
    yp, rp = oracle.rmsnorm_fwd_heads(xp, nh, D, w, 1e-6)
    np.testing.assert_array_equal(yp, y[:, perm, :])
    np.testing.assert_array_equal(rp, rstd[:, perm])
