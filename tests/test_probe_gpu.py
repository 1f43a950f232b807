"""The practical-ceiling probe (rn_stream_mix) through the C ABI: every
destination stream holds the XOR of the source streams, for every provided
read:write mix, with a ragged vector count and a grid smaller than the
vector count (grid-stride), and nothing is written past the streams."""
import pytest
import torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def rn():
    import bwd_fp8_block_amd as m
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return m


@pytest.mark.parametrize("r,w", [(1, 1), (2, 1), (3, 1), (2, 2), (4, 5)])
def test_stream_mix(rn, r, w):
    n16 = 100003
    g = torch.Generator(device="cuda")
    g.manual_seed(r * 10 + w)
    src = [torch.randint(0, 256, (n16 * 16,), generator=g, dtype=torch.uint8, device="cuda") for _ in range(r)]
    full = [torch.full((n16 * 16 + 64,), 0xA5, dtype=torch.uint8, device="cuda") for _ in range(w)]
    dst = [t[:n16 * 16] for t in full]
    rn.rn_stream_mix(src, dst, 97)
    torch.cuda.synchronize()
    ref = src[0].clone()
    for t in src[1:]:
        ref ^= t
    for t in full:
        assert torch.equal(t[:n16 * 16], ref)
        assert torch.all(t[n16 * 16:] == 0xA5)
