"""The bench-side streaming probe on the GPU: every destination stream holds the
XOR of the source streams (or the vector index pattern when there are none),
for every read:write mix it takes, every walk order, vectors in flight and
group size, with a ragged vector count and grids both smaller and larger than
the tile count, and nothing is written past the streams."""
import os
import sys

import pytest
import torch

pytestmark = pytest.mark.gpu
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def probe():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    sys.path.insert(0, ROOT)
    import bench_probe
    return bench_probe


def _pattern(n16):
    i = torch.arange(n16, dtype=torch.int64, device="cuda").to(torch.int32)
    return torch.stack([i, ~i, i, ~i], dim=1).reshape(-1).view(torch.uint8)


@pytest.mark.parametrize("r,w", [(1, 1), (2, 1), (3, 1), (2, 2), (4, 5), (0, 3), (4, 0)])
@pytest.mark.parametrize("order,vpt,wgs,grid", [("stride", 1, 256, 97), ("xcd", 4, 512, 300), ("chunk", 8, 256, 41),
                                                ("xcd", 2, 1024, 5000), ("chunk", 1, 64, 1)])
def test_stream_mix(probe, r, w, order, vpt, wgs, grid):
    n16 = 100003
    g = torch.Generator(device="cuda")
    g.manual_seed(r * 10 + w)
    src = [torch.randint(0, 256, (n16 * 16,), generator=g, dtype=torch.uint8, device="cuda") for _ in range(r)]
    full = [torch.full((n16 * 16 + 64,), 0xA5, dtype=torch.uint8, device="cuda") for _ in range(w)]
    dst = [t[:n16 * 16] for t in full]
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    probe.stream_mix(src, dst, grid, wgs=wgs, vpt=vpt, order=order, sink=sink)
    torch.cuda.synchronize()
    if r:
        ref = src[0].clone()
        for t in src[1:]:
            ref ^= t
    else:
        ref = _pattern(n16)
    for t in full:
        assert torch.equal(t[:n16 * 16], ref)
        assert torch.all(t[n16 * 16:] == 0xA5)
