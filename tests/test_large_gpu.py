"""Tensors beyond 4 GiB and the dw accuracy at very large T.

T = 2^18 + 5 rows of H = 8192 bf16 values is 4.3 GB per tensor: 64-bit
addressing of rows, scales and partials.  Inputs are drawn on the GPU (seeded
torch generator) and copied to the host, where the FP64 oracle checks every
row of the backward's dx and every dw element (the oracle runs on row chunks
in parallel threads; dw is their FP64 sum in row order).  The forward and the
fp8 producer are compared on rows spread over the whole tensor.

The dw budget (every element within 1e-4 + 1e-4*|ref| of the FP64 sum) is
checked at the row counts miles-ext-kernels PR #15 reports its worst element
for (Summary / Accuracy / Known limitation: H = 4096 at T = 393216 and 524288,
H = 5120 at T = 524288, fp32 weight); each run prints its worst element as a
fraction of the budget."""
import numpy as np
import pytest
import torch

from gpu_common import (check_dw, check_rstd, check_values, compare_all_rows, dw_budget_ratio, oracle_dw_chunked,
                        to_host)

pytestmark = pytest.mark.gpu

T, H = (1 << 18) + 5, 8192


@pytest.fixture(scope="module")
def rn():
    import bwd_fp8_block_amd as m
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return m


def _rows(T):
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


def _backward_all_rows(rn, oracle, x, dy, w, rstd, label):
    """Runs the backward and checks every row of dx and every dw element against the
    oracle; returns dw's worst element as a fraction of its budget."""
    Tn, Hn = x.shape
    dx = torch.empty_like(x)
    dw = torch.empty(Hn, device="cuda")
    ws = torch.full((rn.rmsnorm_bwd_workspace_bytes(Tn, Hn) // 4,), float("nan"), device="cuda")
    rn.rmsnorm_bwd(dy, x, w, rstd, dx, dw, deterministic=True, workspace=ws)
    dwh = to_host(dw)
    dxh = _bits(dx)
    del dx, ws
    xh, dyh, wh = _bits(x), _bits(dy), to_host(w)
    r64 = to_host(rstd).astype(np.float64)
    compare_all_rows("dx", Tn, 4096, lambda lo, hi: dxh[lo:hi],
                     lambda lo, hi: oracle.rmsnorm_bwd(dyh[lo:hi], xh[lo:hi], wh, r64[lo:hi], want_dw=False)[0],
                     True)
    del dxh
    ref = oracle_dw_chunked(oracle, dyh, xh, wh, r64)
    ratio = dw_budget_ratio(dwh, ref)
    print("%s: dw worst element at %.4f of the budget (T=%d, H=%d)" % (label, ratio, Tn, Hn), flush=True)
    check_dw(dwh, ref)
    return ratio


def test_forward_and_backward_beyond_4gib(rn, oracle):
    g = torch.Generator(device="cuda")
    g.manual_seed(31)
    x = _randn(g, T, H)
    assert x.numel() * 2 > (1 << 32)
    w = (1 + 0.1 * torch.randn(H, generator=g, device="cuda")).to(torch.bfloat16)
    y = torch.empty_like(x)
    rstd = torch.empty(T, device="cuda")
    rn.rmsnorm_fwd(x, w, y, rstd, 1e-6)
    rows = _rows(T)
    ri = torch.from_numpy(rows).cuda()
    xs, ws = _bits(x[ri]), _bits(w)
    yref, rref = oracle.rmsnorm_fwd(xs, ws, 1e-6)
    check_rstd(to_host(rstd)[rows], rref)
    check_values("y", _bits(y[ri]), yref, True)
    del y
    dy = _randn(g, T, H)
    _backward_all_rows(rn, oracle, x, dy, w, rstd, "bf16 rows, bf16 weight, beyond 4 GiB")


@pytest.mark.parametrize("Tn,Hn", [(393216, 4096), (524288, 4096), (524288, 5120)])
def test_dw_budget_at_very_large_t(rn, oracle, Tn, Hn):
    """bf16 x and dy ~ N(0,1), fp32 weight 1 + 0.1 N(0,1): every dw element within the budget
    (the pages report deterministic dw over it at these row counts before their fix)."""
    g = torch.Generator(device="cuda")
    g.manual_seed(Tn + Hn)
    x = _randn(g, Tn, Hn)
    w = 1 + 0.1 * torch.randn(Hn, generator=g, device="cuda")
    y = torch.empty_like(x)
    rstd = torch.empty(Tn, device="cuda")
    rn.rmsnorm_fwd(x, w, y, rstd, 1e-6)
    del y
    dy = _randn(g, Tn, Hn)
    _backward_all_rows(rn, oracle, x, dy, w, rstd, "bf16 rows, fp32 weight")


def test_fp8_producer_beyond_4gib(rn, oracle):
    g = torch.Generator(device="cuda")
    g.manual_seed(32)
    x = _randn(g, T, H)
    res = _randn(g, T, H)
    w = (1 + 0.1 * torch.randn(H, generator=g, device="cuda")).to(torch.bfloat16)
    rows = _rows(T)
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
