"""Tensors beyond 4 GiB: 64-bit addressing of rows, scales and partials.

T = 2^18 + 5 rows of H = 8192 bf16 values is 4.3 GB per tensor.  Inputs are
drawn on the GPU (seeded torch generator) and only sampled rows go to the CPU
oracle: forward y and rstd, backward dx, and the fp8 producer's residual,
normed values, codes and scales are compared on rows spread over the whole
tensor, including the last one."""
import numpy as np
import pytest
import torch

from gpu_common import check_rstd, check_values, to_host

pytestmark = pytest.mark.gpu

T, H = (1 << 18) + 5, 8192


@pytest.fixture(scope="module")
def rn():
    import bwd_fp8_block_amd as m
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return m


def _rows():
    rng = np.random.default_rng(12)
    rows = {0, 1, T // 2, T - 2, T - 1, (1 << 17) + 3}
    rows.update(rng.choice(T, 24, replace=False).tolist())
    return np.array(sorted(rows), dtype=np.int64)


def _randn(g, *shape):
    out = torch.empty(*shape, dtype=torch.bfloat16, device="cuda")
    for i in range(0, shape[0], 1 << 16):           # in slices, to bound the fp32 temporary
        out[i:i + (1 << 16)] = torch.randn(min(1 << 16, shape[0] - i), *shape[1:], generator=g,
                                           device="cuda").to(torch.bfloat16)
    return out


def _bits(t):
    return to_host(t)


def test_forward_and_backward_beyond_4gib(rn, oracle):
    g = torch.Generator(device="cuda")
    g.manual_seed(31)
    x = _randn(g, T, H)
    assert x.numel() * 2 > (1 << 32)
    w = (1 + 0.1 * torch.randn(H, generator=g, device="cuda")).to(torch.bfloat16)
    y = torch.empty_like(x)
    rstd = torch.empty(T, device="cuda")
    rn.rmsnorm_fwd(x, w, y, rstd, 1e-6)
    rows = _rows()
    ri = torch.from_numpy(rows).cuda()
    xs, ws = _bits(x[ri]), _bits(w)
    yref, rref = oracle.rmsnorm_fwd(xs, ws, 1e-6)
    check_rstd(to_host(rstd)[rows], rref)
    check_values("y", _bits(y[ri]), yref, True)
    del y
    dy = _randn(g, T, H)
    dx = torch.empty_like(x)
    dw = torch.empty(H, device="cuda")
    ws_buf = torch.empty(rn.rmsnorm_bwd_workspace_bytes(T, H) // 4, device="cuda")
    rn.rmsnorm_bwd(dy, x, w, rstd, dx, dw, deterministic=True, workspace=ws_buf)
    rs = to_host(rstd)[rows].astype(np.float64)
    dxref, _ = oracle.rmsnorm_bwd(_bits(dy[ri]), xs, ws, rs, want_dw=False)
    check_values("dx", _bits(dx[ri]), dxref, True)
    # dw over all rows: the sum of the backward's dw over the two halves of the rows
    h = T // 2
    dwa = torch.empty(H, device="cuda")
    dwb = torch.empty(H, device="cuda")
    rn.rmsnorm_bwd(dy[:h], x[:h], w, rstd[:h], dx[:h], dwa, deterministic=True, workspace=ws_buf)
    rn.rmsnorm_bwd(dy[h:], x[h:], w, rstd[h:], dx[h:], dwb, deterministic=True, workspace=ws_buf)
    full, a, b = (to_host(t).astype(np.float64) for t in (dw, dwa, dwb))
    np.testing.assert_allclose(full, a + b, rtol=1e-5, atol=1e-3)


def test_fp8_producer_beyond_4gib(rn, oracle):
    g = torch.Generator(device="cuda")
    g.manual_seed(32)
    x = _randn(g, T, H)
    res = _randn(g, T, H)
    w = (1 + 0.1 * torch.randn(H, generator=g, device="cuda")).to(torch.bfloat16)
    rows = _rows()
    ri = torch.from_numpy(rows).cuda()
    xs, rs0, ws = _bits(x[ri]), _bits(res[ri]), _bits(w)
    out = torch.empty(T, H, dtype=torch.uint8, device="cuda")
    sld = (T + 3) // 4 * 4
    scale = torch.empty(H // 128, sld, device="cuda")
    normed = torch.empty_like(x)
    rn.add_rmsnorm_fp8_block_quant(x, res, w, out, scale, normed, 1e-6)
    ref = oracle.add_rmsnorm_fp8(xs, rs0, ws, 1e-6)
    assert np.array_equal(_bits(res[ri]), ref["h"])
    nb = _bits(normed[ri])
    check_values("normed", nb, ref["normed"], True)
    sref, cref = oracle.block_quant_e4m3(nb)
    assert np.array_equal(to_host(scale)[:, rows].view(np.uint32), sref[:, :len(rows)].view(np.uint32))
    assert np.array_equal(to_host(out[ri]), cref)
