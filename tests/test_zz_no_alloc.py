"""rmsnorm_bwd_noalloc (the backward without a workspace, for callers that
cannot allocate) through the C ABI: the same dx and dw bits as rmsnorm_bwd
with a caller workspace, on two calls in a row whose second has fewer rows and
columns (the library's scratch keeps the first call's partials), on the
few-row path that needs no scratch, and a clear error with nothing written for
a shape whose partials exceed the scratch."""
import numpy as np
import pytest
import torch

from gpu_common import check_dw, check_values, to_dev, to_host
from workloads import Workload, generate

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def rn():
    import bwd_fp8_block_amd as m
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return m


def _inputs(rn, T, H, xd, wd, seed):
    d = generate(Workload("noalloc", T, H, xd, wd, seed=seed))
    xdev, wdev, dydev = to_dev(d["x"]), to_dev(d["w"]), to_dev(d["dy"])
    rstd = torch.empty(T, dtype=torch.float32, device="cuda")
    rn.rmsnorm_fwd(xdev, wdev, torch.empty_like(xdev), rstd, 1e-6)
    return d, xdev, wdev, dydev, rstd


def _both(rn, xdev, wdev, dydev, rstd, det):
    T, H = xdev.shape
    dx0, dw0 = torch.empty_like(xdev), torch.full((H,), float("nan"), device="cuda")
    nbytes = rn.rmsnorm_bwd_workspace_bytes(T, H)
    ws = torch.full((max(nbytes // 4, 1),), float("nan"), device="cuda")
    rn.rmsnorm_bwd(dydev, xdev, wdev, rstd, dx0, dw0, deterministic=det, workspace=ws)
    dx1, dw1 = torch.empty_like(xdev), torch.full((H,), float("nan"), device="cuda")
    rn.rmsnorm_bwd_noalloc(dydev, xdev, wdev, rstd, dx1, dw1, deterministic=det)
    torch.cuda.synchronize()
    return (to_host(dx0), to_host(dw0)), (to_host(dx1), to_host(dw1))


@pytest.mark.parametrize("first,second", [
    ((8192, 4096, "bf16", "bf16"), (3001, 2048, "bf16", "f32")),
    ((65536, 5120, "bf16", "f32"), (4099, 4096, "bf16", "bf16")),
    ((2999, 8192, "f32", "f32"), (129, 256, "f32", "f32")),
])
def test_noalloc_matches_the_workspace_entry_point(rn, oracle, first, second):
    for k, (T, H, xd, wd) in enumerate((first, second)):
        print("noalloc call %d: T=%d H=%d %s/%s" % (k, T, H, xd, wd), flush=True)
        d, xdev, wdev, dydev, rstd = _inputs(rn, T, H, xd, wd, 8100 + T + H)
        (dx0, dw0), (dx1, dw1) = _both(rn, xdev, wdev, dydev, rstd, det=(k == 0))
        assert np.array_equal(dw1.view(np.uint32), dw0.view(np.uint32)), "dw differs from rmsnorm_bwd's"
        assert np.array_equal(dx1, dx0), "dx differs from rmsnorm_bwd's"
        if T * H <= 1 << 24:
            rs = to_host(rstd).astype(np.float64)
            dxref, dwref = oracle.rmsnorm_bwd(d["dy"], d["x"], d["w"], rs)
            check_values("dx", dx1, dxref, xd == "bf16")
            check_dw(dw1, dwref)


def test_noalloc_few_rows_and_limits(rn):
    # rows that one strip walks need no scratch, at any H the backward takes
    for T, H in ((2, 16384), (3, 64)):
        d, xdev, wdev, dydev, rstd = _inputs(rn, T, H, "bf16", "bf16", 8200 + H)
        (dx0, dw0), (dx1, dw1) = _both(rn, xdev, wdev, dydev, rstd, det=True)
        assert np.array_equal(dw1.view(np.uint32), dw0.view(np.uint32)) and np.array_equal(dx1, dx0)
    # partials of 256 strips x 16384 columns exceed the 8 MiB scratch: an error, nothing written
    T, H = 4096, 16384
    x = torch.zeros(T, H, dtype=torch.bfloat16, device="cuda")
    w = torch.ones(H, dtype=torch.bfloat16, device="cuda")
    rstd = torch.ones(T, device="cuda")
    dx = torch.full((T, H), 3.0, dtype=torch.bfloat16, device="cuda")
    dw = torch.full((H,), 9.0, device="cuda")
    if torch.cuda.get_device_properties(0).multi_processor_count * H * 4 > 8 << 20:
        with pytest.raises(rn.RNError) as e:
            rn.rmsnorm_bwd_noalloc(x, x, w, rstd, dx, dw)
        assert e.value.status == 6
        torch.cuda.synchronize()
        assert torch.all(dw == 9.0) and torch.all(dx == 3.0)
