"""Concurrent calls through the C ABI: host threads, each with its own stream and
its own buffers, run the forward, the backward (with its own workspace) and the
fp8 producer at the same time, several rounds each.  The library keeps no state
between calls beyond a per-device property cache, and every kernel's result
depends only on its inputs and the device, so every output must carry the bits
of the same calls made one after another on one stream.

The shapes differ per thread so that different launch forms (one-strip and
multi-strip backward, short and wide rows, ragged tails) run side by side.
"""
import threading

import pytest
import torch

import bwd_fp8_block_amd as rn

pytestmark = pytest.mark.gpu

# (T, H): one-strip backward (T = 4), ragged multi-strip runs, short and wide rows.
SHAPES = [(1000, 4096), (2055, 2048), (8192, 1024), (300, 7168), (4, 4096), (4099, 5120)]
ROUNDS = 3
EPS = 1e-6


class Case:
    def __init__(self, T, H, seed):
        g = torch.Generator(device="cuda")
        g.manual_seed(seed)
        bf = torch.bfloat16
        dev = torch.device("cuda:0")
        randn = lambda *s: torch.randn(*s, generator=g, device=dev)
        self.T, self.H = T, H
        self.x = randn(T, H).to(bf)
        self.w = (1 + 0.1 * randn(H)).to(bf)
        self.dy = randn(T, H).to(bf)
        self.res0 = randn(T, H).to(bf)
        self.res = torch.empty_like(self.res0)
        self.y = torch.empty_like(self.x)
        self.rstd = torch.empty(T, device=dev)
        self.dx = torch.empty_like(self.x)
        self.dw = torch.empty(H, device=dev)
        nbytes = rn.rmsnorm_bwd_workspace_bytes(T, H)
        self.ws = torch.empty(max(1, nbytes // 4), device=dev) if nbytes else None
        self.out = torch.empty(T, H, dtype=torch.uint8, device=dev)
        self.scale = torch.empty(H // 128, (T + 3) // 4 * 4, device=dev)
        self.normed = torch.empty_like(self.x)

    def outputs(self):
        return {"y": self.y, "rstd": self.rstd, "dx": self.dx, "dw": self.dw, "res": self.res,
                "codes": self.out, "scale": self.scale[:, :self.T], "normed": self.normed}

    def poison(self):
        """Fill every output with a value no correct call leaves there (on the
        current stream)."""
        for t in self.outputs().values():
            if t.dtype == torch.uint8:
                t.fill_(0x7F)
            else:
                t.fill_(float("nan"))

    def run(self):
        """The three ops in order on torch's current stream."""
        self.res.copy_(self.res0)              # the producer updates the residual in place
        rn.rmsnorm_fwd(self.x, self.w, self.y, self.rstd, EPS)
        rn.rmsnorm_bwd(self.dy, self.x, self.w, self.rstd, self.dx, self.dw, deterministic=True, workspace=self.ws)
        rn.add_rmsnorm_fp8_block_quant(self.x, self.res, self.w, self.out, self.scale, self.normed, EPS)

    def snapshot(self):
        return {k: t.contiguous().view(torch.uint8).cpu() for k, t in self.outputs().items()}


def test_concurrent_threads_and_streams():
    cases = [Case(T, H, 900 + i) for i, (T, H) in enumerate(SHAPES)]
    ref = []
    for c in cases:
        c.poison()
        c.run()
        torch.cuda.synchronize()
        ref.append(c.snapshot())

    streams = [torch.cuda.Stream() for _ in cases]     # default priority
    start = threading.Barrier(len(cases))
    errors = []
    got = [None] * len(cases)

    def worker(i):
        try:
            with torch.cuda.stream(streams[i]):
                start.wait(timeout=60)
                for _ in range(ROUNDS):
                    cases[i].poison()
                    cases[i].run()
            streams[i].synchronize()
            got[i] = cases[i].snapshot()
        except BaseException as e:                     # reported below, in the test's thread
            errors.append((i, repr(e)))

    torch.cuda.synchronize()                           # inputs and references are complete
    threads = [threading.Thread(target=worker, args=(i,)) for i in range(len(cases))]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not any(t.is_alive() for t in threads), "a worker thread did not finish"
    assert not errors, errors
    for (T, H), r, g in zip(SHAPES, ref, got):
        for k in r:
            assert torch.equal(r[k], g[k]), "T=%d H=%d: %s differs under concurrent calls" % (T, H, k)


FIRST_CALLS = r'''
import sys, threading
sys.path.insert(0, sys.argv[1])
import torch
import bwd_fp8_block_amd as rn

N = 8
dev = torch.device("cuda:0")
g = torch.Generator(device=dev)
g.manual_seed(77)
xs = [torch.randn(513 + 97 * i, 2048, generator=g, device=dev).to(torch.bfloat16) for i in range(N)]
w = (1 + 0.1 * torch.randn(2048, generator=g, device=dev)).to(torch.bfloat16)
ys = [torch.empty_like(x) for x in xs]
rs = [torch.empty(x.shape[0], device=dev) for x in xs]
sizes = [None] * N
streams = [torch.cuda.Stream() for _ in range(N)]
torch.cuda.synchronize()
start = threading.Barrier(N)
errors = []

def worker(i):
    try:
        with torch.cuda.stream(streams[i]):
            start.wait(timeout=60)
            # the first calls of this process into the library, all at once
            sizes[i] = rn.rmsnorm_bwd_workspace_bytes(8192, 4096)
            rn.rmsnorm_fwd(xs[i], w, ys[i], rs[i], 1e-6)
        streams[i].synchronize()
    except BaseException as e:
        errors.append((i, repr(e)))

threads = [threading.Thread(target=worker, args=(i,)) for i in range(N)]
for t in threads:
    t.start()
for t in threads:
    t.join(timeout=120)
assert not any(t.is_alive() for t in threads), "a thread did not finish"
assert not errors, errors
assert len(set(sizes)) == 1 and sizes[0] > 0, sizes
for i in range(N):
    y2, r2 = torch.empty_like(ys[i]), torch.empty_like(rs[i])
    rn.rmsnorm_fwd(xs[i], w, y2, r2, 1e-6)
    torch.cuda.synchronize()
    assert torch.equal(y2.view(torch.int16), ys[i].view(torch.int16)), i
    assert torch.equal(r2, rs[i]), i
print("first-calls-ok", flush=True)
'''


def test_first_calls_from_many_threads_in_a_fresh_process():
    """The per-device property cache is filled by whichever thread calls first:
    eight threads make their first calls into a freshly loaded library at the same
    moment, and all of them see one workspace size and produce the bits of serial
    calls."""
    import os
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    print("fresh process: 8 threads, first calls at once", flush=True)
    r = subprocess.run([sys.executable, "-c", FIRST_CALLS, root], capture_output=True, text=True, timeout=100)
    assert r.returncode == 0 and "first-calls-ok" in r.stdout, (r.returncode, r.stdout[-2000:], r.stderr[-2000:])
