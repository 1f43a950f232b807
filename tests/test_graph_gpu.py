"""The entry points under HIP graph capture and on a side stream: a captured
step (forward, fused backward, fp8 producer, residual pair, per-head norm) is
replayed several times, with eager work and synchronisations between the
replays, and every replay must reproduce the eager results bit for bit."""
import numpy as np
import pytest
import torch

from gpu_common import to_host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def rn():
    import bwd_fp8_block_amd as m
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return m


def _buffers(T, H, seed):
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    bf = torch.bfloat16

    def rnd(*s):
        return torch.randn(*s, generator=g, device="cuda").to(bf)

    b = {"x": rnd(T, H), "w": (1 + 0.1 * torch.randn(H, generator=g, device="cuda")).to(bf), "dy": rnd(T, H),
         "res0": rnd(T, H), "u": rnd(T, H), "gr": rnd(T, H), "qkv": rnd(T, 3 * H)}
    b["y"] = torch.empty(T, H, dtype=bf, device="cuda")
    b["rstd"] = torch.empty(T, device="cuda")
    b["dx"] = torch.empty(T, H, dtype=bf, device="cuda")
    b["dw"] = torch.empty(H, device="cuda")
    b["res"] = torch.empty(T, H, dtype=bf, device="cuda")
    b["out"] = torch.empty(T, H, dtype=torch.uint8, device="cuda")
    b["sc"] = torch.empty(H // 128, (T + 3) // 4 * 4, device="cuda")
    b["n"] = torch.empty(T, H, dtype=bf, device="cuda")
    b["y2"] = torch.empty(T, H, dtype=bf, device="cuda")
    b["h2"] = torch.empty(T, H, dtype=bf, device="cuda")
    b["r2"] = torch.empty(T, device="cuda")
    b["dx2"] = torch.empty(T, H, dtype=bf, device="cuda")
    b["dw2"] = torch.empty(H, device="cuda")
    b["qo"] = torch.empty(T, H // 128, 128, dtype=bf, device="cuda")
    b["qr"] = torch.empty(T * (H // 128), device="cuda")
    return b


def _step(rn, b, ws):
    rn.rmsnorm_fwd(b["x"], b["w"], b["y"], b["rstd"], 1e-6)
    rn.rmsnorm_bwd(b["dy"], b["x"], b["w"], b["rstd"], b["dx"], b["dw"], deterministic=True, workspace=ws)
    b["res"].copy_(b["res0"])                  # the producer updates the residual in place
    rn.add_rmsnorm_fp8_block_quant(b["x"], b["res"], b["w"], b["out"], b["sc"], b["n"], 1e-6)
    rn.rmsnorm_fwd_residual(b["x"], b["u"], b["w"], b["y2"], b["h2"], b["r2"], 1e-6)
    rn.rmsnorm_bwd_residual(b["dy"], b["h2"], b["w"], b["r2"], b["gr"], b["dx2"], b["dw2"], workspace=ws)
    H = b["x"].shape[1]
    rn.rmsnorm_fwd_heads(b["qkv"][:, :H].view(-1, H // 128, 128), b["w"][:128], b["qo"], b["qr"], 1e-6)


OUTS = ["y", "rstd", "dx", "dw", "res", "out", "sc", "n", "y2", "h2", "r2", "dx2", "dw2", "qo", "qr"]


def _snapshot(b):
    snap = {k: to_host(b[k]).copy() for k in OUTS}
    snap["sc"] = snap["sc"][:, :b["x"].shape[0]]     # rows T .. ld-1 of the scales are never written
    return snap


def _poison(b):
    for k in OUTS:
        if b[k].dtype == torch.uint8:
            b[k].fill_(0xA5)
        else:
            b[k].fill_(float("nan"))


@pytest.mark.parametrize("T,H", [(300, 2048), (37, 4096)])
def test_graph_replays_match_eager(rn, T, H):
    b = _buffers(T, H, 99 + T)
    ws = torch.empty(rn.rmsnorm_bwd_workspace_bytes(T, H) // 4, device="cuda")
    _step(rn, b, ws)
    torch.cuda.synchronize()
    ref = _snapshot(b)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):                 # warm up on the capture stream
        _step(rn, b, ws)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        _step(rn, b, ws)
    torch.cuda.synchronize()
    for rep in range(4):
        _poison(b)
        scratch = torch.randn(1 << 20, device="cuda").sum()     # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = _snapshot(b)
        for k in OUTS:
            a, r = got[k], ref[k]
            if a.dtype == np.float32:
                a, r = a.view(np.uint32), r.view(np.uint32)
            assert np.array_equal(a, r), "replay %d: %s differs from the eager result" % (rep, k)
        del scratch


def test_side_stream_matches_default_stream(rn):
    T, H = 129, 1024
    b = _buffers(T, H, 7)
    ws = torch.empty(rn.rmsnorm_bwd_workspace_bytes(T, H) // 4, device="cuda")
    _step(rn, b, ws)
    torch.cuda.synchronize()
    ref = _snapshot(b)
    _poison(b)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        _step(rn, b, ws)
    s.synchronize()
    got = _snapshot(b)
    for k in OUTS:
        a, r = got[k], ref[k]
        if a.dtype == np.float32:
            a, r = a.view(np.uint32), r.view(np.uint32)
        assert np.array_equal(a, r), k
