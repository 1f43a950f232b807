"""Throughput of the RMSNorm hot path on one MI355X.

One step = one pass of the whole path over one batch of synthetic bf16
activations, T = 8192 rows of H = 4096:
    rmsnorm_fwd                   (x -> y, rstd)
    rmsnorm_bwd, deterministic    (dy, x, rstd -> dx, dw)
    add_rmsnorm_fp8_block_quant   (x, residual -> residual, normed, e4m3, scales)
Each op reads its own buffers, and four buffer sets rotate between steps
(2.6 GB in flight; every op alone cycles through at least 0.5 GB), so no call
finds its inputs or its outputs' lines in the 256 MB Infinity Cache left by an
earlier call; inputs are resident in HBM when timing starts.

After the timed steps, the training pair with a residual stream is timed the
same way at the same shape and reported under "next_ops" (not part of value):
    rmsnorm_fwd_residual   (x, u -> y, h_new, rstd)      4*T*H*2 + 2*H + 4*T
    rmsnorm_bwd_residual   (dy, h_new, rstd, g_residual -> dx, dw)
                                                          4*T*H*2 + 2*H + 4*T + 4*H
and the per-head QK-norm of T = 8192 tokens of a fused [T, 3*32*128] bf16
QKV projection: two rmsnorm_fwd_heads calls (the q band and the k band, each
its own [128] weight) into dense [T, 32, 128] outputs with rstd,
    qk_norm                2 * (2*T*32*128*2 + 4*T*32 + 2*128)
and two producer variants at T x H (add_rmsnorm_fp8_quant, normed written):
    fp8_f16_e5m2_block     fp16 rows, e5m2 codes, block scales
                                                          9*T*H + 2*H + 4*(H/128)*round_up(T,4)
    fp8_bf16_e4m3_tensor   bf16 rows, e4m3 codes, one given scale
                                                          9*T*H + 2*H + 4

value = algorithmic bytes of a step / wall time per step (GB/s), timed over the
K steps alone.  The per-op durations (and the roofline of the dominant kernel)
come from HIP events around K back-to-back launches of each op right after.
Algorithmic bytes count each tensor once (weight once, not per row):
    fwd  2*T*H*2 + 2*H + 4*T
    bwd  3*T*H*2 + 2*H + 4*T + 4*H
    fp8  9*T*H + 2*H + 4*(H/128)*round_up(T,4)

`--ceiling` instead times plain streaming passes (the bench-side probe in
bench_probe/, not part of the RMSNorm library) with each op's read:write mix and
bytes at T x H, and read-only and write-only passes of each op's byte count, each
the best over the probe's launch shapes (walk order, vectors in flight, group
size, grid), and prints one JSON line of them: the practical ceiling the op
figures are compared with.

`--latency` instead times single calls at few rows (the launch-bound regime,
T = 1 .. 64): the fp32 T=64 H=256 workload and bf16 rows of H = 2048 / 4096,
forward and backward, back to back on one stream, and prints one JSON line of
microseconds per call (not the contract line).

`--configs` instead times every workload configuration (fp32 T=64 H=256;
bf16 T=8192 H=4096; bf16 rows with an fp32 weight at H=2048, T=58497 with
outlier rows, both dw modes; the fp8 producer at T=4096 H=7168 and T=8192
H=4096; bf16 rows with an fp32 weight at T=65536 H=5120), each op next to the
plain streaming pass with its read:write mix and bytes, and prints one JSON
line of them; `--only NAME` restricts it to one configuration.

`--sweep` instead times the forward, the backward (fixed-order dw) and the
fp8 producer over the grid H in {256, 512, 2048, 4096, 5120, 6144, 7168, 8192} x
T in {256, 1024, 4096, 16231, 65536} (bf16 rows and weight) and prints one
JSON line of microseconds and GB/s per op and shape.

The default run also samples the GPU's shader and memory clocks (sysfs DPM
tables of the card the device sits on) during an untimed window of steps run
right after the timed ones, and reports them under "clocks".

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--no-next] [--latency] [--ceiling]
                       [--configs [--only NAME]] [--sweep] [--sets N]
"""
import argparse
import glob
import hashlib
import json
import os
import statistics
import sys
import threading
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "RMSNorm fwd+bwd & add-RMSNorm-FP8: achieved HBM GB/s, % of peak"
HBM_PEAK_GBS = 8000.0
T_ROWS, HIDDEN, EPS = 8192, 4096, 1e-6
COUNTERS = os.path.join(ROOT, "profiles", "counters_T8192_H4096.json")
# Sources whose change invalidates a kernel's recorded traffic: the kernel and
# its device helpers, and the host file that holds its launch policy.
KERNEL_SOURCES = {
    "fwd": ["bwd_fp8_block_amd/csrc/rn_fwd.hip", "bwd_fp8_block_amd/csrc/rn_device.h",
            "bwd_fp8_block_amd/csrc/rn_host.hip"],
    "bwd": ["bwd_fp8_block_amd/csrc/rn_bwd.hip", "bwd_fp8_block_amd/csrc/rn_device.h",
            "bwd_fp8_block_amd/csrc/rn_host.hip"],
    "fp8": ["bwd_fp8_block_amd/csrc/rn_fp8.hip", "bwd_fp8_block_amd/csrc/rn_device.h",
            "bwd_fp8_block_amd/csrc/rn_host.hip"],
}
KERNEL_NAMES = {"fwd": "k_rmsnorm_fwd", "bwd": "k_rmsnorm_bwd + k_dw_reduce", "fp8": "k_add_rmsnorm_fp8",
                "fwd_residual": "k_rmsnorm_fwd (residual form)",
                "bwd_residual": "k_rmsnorm_bwd (residual form) + k_dw_reduce",
                "qk_norm": "k_rmsnorm_fwd (per-head form) x 2",
                "fp8_f16_e5m2_block": "k_add_rmsnorm_fp8 (fp16 rows, e5m2, block scales)",
                "fp8_bf16_e4m3_tensor": "k_add_rmsnorm_fp8 (bf16 rows, e4m3, per-tensor scale)"}


def algorithmic_bytes(T, H):
    ru4 = (T + 3) // 4 * 4
    return {
        "fwd": 2 * T * H * 2 + 2 * H + 4 * T,
        "bwd": 3 * T * H * 2 + 2 * H + 4 * T + 4 * H,
        "fp8": 9 * T * H + 2 * H + 4 * (H // 128) * ru4,
    }


QK_HEADS, QK_DIM = 32, 128
# Buffer sets rotated by the step and per-op timings (see the module docstring).
NSETS = 4


def next_bytes(T, H):
    return {
        "fwd_residual": 4 * T * H * 2 + 2 * H + 4 * T,
        "bwd_residual": 4 * T * H * 2 + 2 * H + 4 * T + 4 * H,
        "qk_norm": 2 * (2 * T * QK_HEADS * QK_DIM * 2 + 4 * T * QK_HEADS + 2 * QK_DIM),
        "fp8_f16_e5m2_block": 9 * T * H + 2 * H + 4 * (H // 128) * ((T + 3) // 4 * 4),
        "fp8_bf16_e4m3_tensor": 9 * T * H + 2 * H + 4,
    }


def source_hash(op):
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES[op]:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def make_set(torch, gen, dev, T, H, rn):
    """One set of buffers for the three ops (each op has its own inputs)."""
    bf = torch.bfloat16

    def randn(*shape, scale=1.0):
        return (torch.randn(*shape, generator=gen, device=dev, dtype=torch.float32) * scale).to(bf)

    s = {}
    s["w"] = (1.0 + 0.1 * torch.randn(H, generator=gen, device=dev)).to(bf)
    s["x1"] = randn(T, H)
    s["y1"] = torch.empty(T, H, dtype=bf, device=dev)
    s["r1"] = torch.empty(T, dtype=torch.float32, device=dev)
    s["x2"] = randn(T, H)
    s["dy2"] = randn(T, H)
    s["r2"] = torch.empty(T, dtype=torch.float32, device=dev)
    s["dx2"] = torch.empty(T, H, dtype=bf, device=dev)
    s["dw2"] = torch.empty(H, dtype=torch.float32, device=dev)
    s["ws2"] = torch.empty(rn.rmsnorm_bwd_workspace_bytes(T, H) // 4, dtype=torch.float32, device=dev)
    s["x3"] = randn(T, H)
    s["res3"] = randn(T, H)
    s["out3"] = torch.empty(T, H, dtype=torch.uint8, device=dev)
    s["sc3"] = torch.empty(H // 128, (T + 3) // 4 * 4, dtype=torch.float32, device=dev)
    s["n3"] = torch.empty(T, H, dtype=bf, device=dev)
    # the backward's rstd comes from a forward over its own x
    tmp = torch.empty(T, H, dtype=bf, device=dev)
    rn.rmsnorm_fwd(s["x2"], s["w"], tmp, s["r2"], EPS)
    del tmp
    return s


def plan_step(rn, s):
    """The three calls of a step with their arguments marshalled once."""
    return (rn.plan_rmsnorm_fwd(s["x1"], s["w"], s["y1"], s["r1"], EPS),
            rn.plan_rmsnorm_bwd(s["dy2"], s["x2"], s["w"], s["r2"], s["dx2"], s["dw2"], deterministic=True,
                                workspace=s["ws2"]),
            rn.plan_add_rmsnorm_fp8_block_quant(s["x3"], s["res3"], s["w"], s["out3"], s["sc3"], s["n3"], EPS))


def make_res_set(torch, gen, dev, T, H, rn):
    """Buffers of the training pair with a residual stream."""
    bf = torch.bfloat16

    def randn(*shape):
        return torch.randn(*shape, generator=gen, device=dev, dtype=torch.float32).to(bf)

    s = {"w": (1.0 + 0.1 * torch.randn(H, generator=gen, device=dev)).to(bf)}
    s["x"], s["u"] = randn(T, H), randn(T, H)
    s["y"], s["h"] = torch.empty(T, H, dtype=bf, device=dev), torch.empty(T, H, dtype=bf, device=dev)
    s["r"] = torch.empty(T, dtype=torch.float32, device=dev)
    s["dy"], s["gr"] = randn(T, H), randn(T, H)
    s["hb"] = torch.empty(T, H, dtype=bf, device=dev)
    s["rb"] = torch.empty(T, dtype=torch.float32, device=dev)
    s["dx"] = torch.empty(T, H, dtype=bf, device=dev)
    s["dw"] = torch.empty(H, dtype=torch.float32, device=dev)
    s["ws"] = torch.empty(rn.rmsnorm_bwd_workspace_bytes(T, H) // 4, dtype=torch.float32, device=dev)
    # the backward's h_new and rstd come from a residual forward over its own inputs
    tmp = torch.empty(T, H, dtype=bf, device=dev)
    rn.rmsnorm_fwd_residual(randn(T, H), randn(T, H), s["w"], tmp, s["hb"], s["rb"], EPS)
    del tmp
    # per-head QK-norm: q and k bands of a fused QKV projection output
    nh, D = QK_HEADS, QK_DIM
    s["qkv"] = randn(T, 3 * nh * D)
    s["wq"] = (1.0 + 0.1 * torch.randn(D, generator=gen, device=dev)).to(bf)
    s["wk"] = (1.0 + 0.1 * torch.randn(D, generator=gen, device=dev)).to(bf)
    s["qo"] = torch.empty(T, nh, D, dtype=bf, device=dev)
    s["ko"] = torch.empty(T, nh, D, dtype=bf, device=dev)
    s["qr"] = torch.empty(T * nh, dtype=torch.float32, device=dev)
    s["kr"] = torch.empty(T * nh, dtype=torch.float32, device=dev)
    # producer variants
    f16 = torch.float16
    s["vx16"] = torch.randn(T, H, generator=gen, device=dev).to(f16)
    s["vr16"] = torch.randn(T, H, generator=gen, device=dev).to(f16)
    s["vw16"] = (1.0 + 0.1 * torch.randn(H, generator=gen, device=dev)).to(f16)
    s["vn16"] = torch.empty(T, H, dtype=f16, device=dev)
    s["vo"] = torch.empty(T, H, dtype=torch.uint8, device=dev)
    s["vs"] = torch.empty(H // 128, (T + 3) // 4 * 4, dtype=torch.float32, device=dev)
    s["vx"], s["vr"] = randn(T, H), randn(T, H)
    s["vn"] = torch.empty(T, H, dtype=bf, device=dev)
    s["vo2"] = torch.empty(T, H, dtype=torch.uint8, device=dev)
    s["vts"] = torch.full((1,), 0.0125, dtype=torch.float32, device=dev)
    return s


def time_next(torch, rn, gen, dev, T, H, K, W):
    """Per-launch times of the residual training pair, the QK-norm and the producer variants
    (rotating buffer sets)."""
    sets = [make_res_set(torch, gen, dev, T, H, rn) for _ in range(NSETS)]
    nh, D = QK_HEADS, QK_DIM

    def band(s, k):
        return s["qkv"][:, k * nh * D:(k + 1) * nh * D].view(T, nh, D)

    plans = [(rn.plan_rmsnorm_fwd_residual(s["x"], s["u"], s["w"], s["y"], s["h"], s["r"], EPS),
              rn.plan_rmsnorm_bwd_residual(s["dy"], s["hb"], s["w"], s["rb"], s["gr"], s["dx"], s["dw"],
                                           deterministic=True, workspace=s["ws"]),
              rn.plan_rmsnorm_fwd_heads(band(s, 0), s["wq"], s["qo"], s["qr"], EPS),
              rn.plan_rmsnorm_fwd_heads(band(s, 1), s["wk"], s["ko"], s["kr"], EPS),
              rn.plan_add_rmsnorm_fp8_quant(s["vx16"], s["vr16"], s["vw16"], s["vo"], EPS, out_format="e5m2",
                                            block_scale=s["vs"], normed_out=s["vn16"]),
              rn.plan_add_rmsnorm_fp8_quant(s["vx"], s["vr"], s["w"], s["vo2"], EPS, out_format="e4m3",
                                            tensor_scale=s["vts"], normed_out=s["vn"])) for s in sets]
    keys = ["fwd_residual", "bwd_residual", "qk_norm", "fp8_f16_e5m2_block", "fp8_bf16_e4m3_tensor"]
    groups = {"fwd_residual": [0], "bwd_residual": [1], "qk_norm": [2, 3], "fp8_f16_e5m2_block": [4],
              "fp8_bf16_e4m3_tensor": [5]}
    per = {k: per_launch_ms(torch, [[pl[j] for j in groups[k]] for pl in plans], K) for k in keys}
    b = next_bytes(T, H)
    out = {}
    for k, ms in per.items():
        gbs = b[k] / (ms * 1e-3) / 1e9
        out[k] = {"kernel": KERNEL_NAMES[k], "bytes": b[k], "us": round(ms * 1e3, 3), "GB/s": round(gbs, 1),
                  "pct_of_peak": round(100 * gbs / HBM_PEAK_GBS, 2)}
    del sets, plans
    return out


def latency(torch, rn, dev, K):
    """Microseconds per call of back-to-back calls at few rows."""
    def per_call(fn):
        for _ in range(20):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(K):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return round(e0.elapsed_time(e1) * 1e3 / K, 3)

    out = {}
    empty = torch.zeros(1, device=dev)
    out["empty_fill_kernel"] = per_call(lambda: empty.fill_(1.0))
    for H, dt, Ts in ((256, torch.float32, (64,)), (2048, torch.bfloat16, (1, 8, 64)),
                      (4096, torch.bfloat16, (1, 4, 64))):
        for T in Ts:
            x = torch.randn(T, H, device=dev).to(dt)
            w = (1.0 + 0.1 * torch.randn(H, device=dev)).to(dt)
            y, r = torch.empty_like(x), torch.empty(T, device=dev)
            dy, dx = torch.randn(T, H, device=dev).to(dt), torch.empty_like(x)
            dw = torch.empty(H, device=dev)
            ws = torch.empty(rn.rmsnorm_bwd_workspace_bytes(T, H) // 4 + 1, device=dev)
            f = rn.plan_rmsnorm_fwd(x, w, y, r, EPS)
            f()
            b = rn.plan_rmsnorm_bwd(dy, x, w, r, dx, dw, True, ws)
            key = "%s_T%d_H%d" % ("f32" if dt == torch.float32 else "bf16", T, H)
            out[key] = {"fwd_us": per_call(f), "bwd_us": per_call(b)}
    return out


# Practical ceilings: plain streaming passes with each op's read:write mix and
# bytes at T x H (equal-size streams; the fp8 producer's 2 x T*H*2 read and
# 2 x T*H*2 + T*H written bytes become 4 reads and 5 writes of T*H bytes).
CEILING_MIXES = {
    "fwd_1R1W": (1, 1, 2), "bwd_2R1W": (2, 1, 2), "fp8_4R5W": (4, 5, 1),
    "fwd_residual_2R2W": (2, 2, 2), "bwd_residual_3R1W": (3, 1, 2),
}


# The streaming passes' launch shapes: every walk order of the probe (grid-stride,
# the RMSNorm kernels' XCD-aware window, one contiguous chunk per work-group),
# 1 .. 8 vectors per thread per stream in flight, 256- and 512-thread groups, and
# grids from one to 64 work-groups per CU (those with at least one tile each).
CEILING_ORDERS = ("stride", "xcd", "chunk")
CEILING_VPT = (1, 2, 4, 8)
CEILING_WGS = (256, 512)
CEILING_GRIDS = (256, 512, 1024, 2048, 4096, 8192, 16384)


def mix_ceiling(torch, probe, dev, r, w, nb, K, shapes=None):
    """(best launch shape, us per call) of the streaming probe with r source and w
    destination streams of nb bytes each, best over the launch shapes; four buffer sets
    alternate so that no pass finds its inputs in the Infinity Cache."""
    nb = nb // 16 * 16
    sets = [([torch.empty(nb, dtype=torch.uint8, device=dev) for _ in range(r)],
             [torch.empty(nb, dtype=torch.uint8, device=dev) for _ in range(w)]) for _ in range(4)]
    for src, _ in sets:
        for t in src:
            t.fill_(1)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    if shapes is None:
        shapes = [(o, v, g, grid) for o in CEILING_ORDERS for v in CEILING_VPT for g in CEILING_WGS
                  for grid in CEILING_GRIDS if grid * g * v <= nb // 16]
    best = None
    for order, vpt, wgs, grid in shapes:
        plans = [probe.plan_stream_mix(*st, grid, wgs=wgs, vpt=vpt, order=order, sink=sink) for st in sets]

        def one(k):
            plans[k % 4]()
        for k in range(8):
            one(k)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for k in range(K):
            one(k)
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / K
        if best is None or us < best[1]:
            best = ({"order": order, "vpt": vpt, "wgs": wgs, "grid": grid}, us)
    del sets
    torch.cuda.empty_cache()
    return best


def ceiling(torch, probe, dev, T, H, K):
    """Per-call time of the streaming probe for each op's mix at T x H, and of a
    read-only and a write-only pass of each op's byte count, best over the probe's
    launch shapes."""
    out = {}
    runs = []
    for name, (r, w, bytes_per_elem) in CEILING_MIXES.items():
        runs.append((name, r, w, T * H * bytes_per_elem))
    for op, total in (("fwd", 2 * T * H * 2), ("bwd", 3 * T * H * 2), ("fp8", 9 * T * H)):
        nr, nw = min(4, total // (T * H)), min(5, total // (T * H))
        runs.append(("%s_bytes_read_only_%dR" % (op, nr), nr, 0, total // nr))
        runs.append(("%s_bytes_write_only_%dW" % (op, nw), 0, nw, total // nw))
    for name, r, w, nb in runs:
        shape, us = mix_ceiling(torch, probe, dev, r, w, nb, K)
        total = (r + w) * (nb // 16 * 16)
        out[name] = {"bytes": total, "best": shape, "us": round(us, 2), "GB/s": round(total / us / 1e3, 1),
                     "pct_of_peak": round(100 * total / us / 1e3 / HBM_PEAK_GBS, 2)}
        log(name, out[name])
    return out


# The workload configurations timed by --configs: (name, T, H, x dtype, w dtype,
# x standard deviation, outlier-row fraction, ops).  Inputs are drawn on the GPU
# with the distributions of the parity workloads: x ~ N(0, std^2) with the
# outlier rows scaled by 50, dy and residual ~ N(0, 1), w = 1 + 0.1 N(0, 1),
# rounded to the storage dtype; eps = 1e-6.
CONFIG_RUNS = [
    ("f32_T64_H256", 64, 256, "f32", "f32", 1.0, 0.0, ("fwd", "bwd")),
    ("bf16_T8192_H4096", 8192, 4096, "bf16", "bf16", 1.0, 0.0, ("fwd", "bwd")),
    ("bf16_T58497_H2048_outliers_f32w", 58497, 2048, "bf16", "f32", 2.0, 0.01, ("fwd", "bwd", "bwd_nondet")),
    ("fp8_T4096_H7168", 4096, 7168, "bf16", "bf16", 1.0, 0.0, ("fp8",)),
    ("bf16_T65536_H5120_f32w", 65536, 5120, "bf16", "f32", 1.0, 0.0, ("fwd", "bwd")),
    ("fp8_T8192_H4096", 8192, 4096, "bf16", "bf16", 1.0, 0.0, ("fp8",)),
]
# (reads, writes, bytes per element of one stream) of each op's plain-pass twin
OP_MIX = {"fwd": (1, 1, None), "bwd": (2, 1, None), "bwd_nondet": (2, 1, None), "fp8": (4, 5, 1)}


def config_bytes(op, T, H, sx, sw):
    if op == "fwd":
        return 2 * T * H * sx + H * sw + 4 * T
    if op in ("bwd", "bwd_nondet"):
        return 3 * T * H * sx + H * sw + 4 * T + 4 * H
    return 9 * T * H + 2 * H + 4 * (H // 128) * ((T + 3) // 4 * 4)


def configs(torch, rn, probe, dev, only=None):
    """Per-launch time of each op at every workload configuration, with the
    plain streaming pass of the same read:write mix and bytes beside it.  Four
    buffer sets rotate when a set is below 512 MB, two above."""
    out = {}
    gen = torch.Generator(device=dev)
    gen.manual_seed(20261203)
    for name, T, H, xdt, wdt, std, ofrac, ops in CONFIG_RUNS:
        if only and name != only:
            continue
        xt = torch.float32 if xdt == "f32" else torch.bfloat16
        wt = torch.float32 if wdt == "f32" else torch.bfloat16
        sx, sw = (4 if xdt == "f32" else 2), (4 if wdt == "f32" else 2)

        def randn(*shape, scale=1.0):
            return torch.randn(*shape, generator=gen, device=dev, dtype=torch.float32) * scale

        sets = []
        set_bytes = 4 * T * H * sx                       # x, y, dy, dx or x, residual, normed, codes
        for _ in range(NSETS if set_bytes < (512 << 20) else 2):
            st = {"w": (1.0 + 0.1 * randn(H)).to(wt)}
            x = randn(T, H, scale=std)
            if ofrac > 0:
                rows = torch.randperm(T, generator=gen, device=dev)[:int(round(ofrac * T))]
                x[rows] *= 50.0
            st["x"] = x.to(xt)
            del x
            if "fp8" in ops:
                st["res"] = randn(T, H).to(xt)
                st["out"] = torch.empty(T, H, dtype=torch.uint8, device=dev)
                st["sc"] = torch.empty(H // 128, (T + 3) // 4 * 4, dtype=torch.float32, device=dev)
                st["n"] = torch.empty(T, H, dtype=xt, device=dev)
            else:
                st["y"] = torch.empty(T, H, dtype=xt, device=dev)
                st["rstd"] = torch.empty(T, dtype=torch.float32, device=dev)
                st["dy"] = randn(T, H).to(xt)
                st["dx"] = torch.empty(T, H, dtype=xt, device=dev)
                st["dw"] = torch.empty(H, dtype=torch.float32, device=dev)
                st["ws"] = torch.empty(rn.rmsnorm_bwd_workspace_bytes(T, H) // 4 + 1, dtype=torch.float32,
                                       device=dev)
                rn.rmsnorm_fwd(st["x"], st["w"], st["y"], st["rstd"], EPS)
            sets.append(st)
        res = {"T": T, "H": H, "x_dtype": xdt, "w_dtype": wdt, "ops": {}}
        for op in ops:
            plans = []
            for st in sets:
                if op == "fwd":
                    plans.append(rn.plan_rmsnorm_fwd(st["x"], st["w"], st["y"], st["rstd"], EPS))
                elif op == "fp8":
                    plans.append(rn.plan_add_rmsnorm_fp8_block_quant(st["x"], st["res"], st["w"], st["out"], st["sc"],
                                                                    st["n"], EPS))
                else:
                    plans.append(rn.plan_rmsnorm_bwd(st["dy"], st["x"], st["w"], st["rstd"], st["dx"], st["dw"],
                                                     deterministic=(op == "bwd"), workspace=st["ws"]))
            nbytes = config_bytes(op, T, H, sx, sw)
            K = max(20, min(400, int(20e-3 / (nbytes / 5e12))))
            ms = per_launch_ms(torch, [[pl] for pl in plans], K)
            gbs = nbytes / (ms * 1e-3) / 1e9
            e = {"bytes": nbytes, "us": round(ms * 1e3, 2), "GB/s": round(gbs, 1),
                 "pct_of_peak": round(100 * gbs / HBM_PEAK_GBS, 2)}
            r, w, bpe = OP_MIX[op]
            if T * H >= 1 << 20:                         # the few-row case is launch-bound: no ceiling
                nb = T * H * (bpe if bpe else sx)
                shape, us = mix_ceiling(torch, probe, dev, r, w, nb, max(10, K // 2))
                e.update({"mix": "%dR%dW" % (r, w), "mix_us": round(us, 2), "mix_shape": shape,
                          "op_vs_mix": round(us / (ms * 1e3), 3)})
            res["ops"][op] = e
            log(name, op, e)
        out[name] = res
        del sets
        torch.cuda.empty_cache()
    return out


SWEEP_H = (256, 512, 2048, 4096, 5120, 6144, 7168, 8192)
SWEEP_T = (256, 1024, 4096, 16231, 65536)


def sweep(torch, rn, dev):
    """Per-launch time of fwd, bwd and the fp8 producer over the H x T grid (bf16)."""
    bf = torch.bfloat16
    gen = torch.Generator(device=dev)
    gen.manual_seed(20261204)
    out = []
    for H in SWEEP_H:
        for T in SWEEP_T:
            nsets = NSETS if 6 * T * H * 2 < (512 << 20) else 2
            sets = []
            for _ in range(nsets):
                st = {"w": (1.0 + 0.1 * torch.randn(H, generator=gen, device=dev)).to(bf)}
                for k in ("x", "dy", "res"):
                    st[k] = torch.randn(T, H, generator=gen, device=dev).to(bf)
                st["y"], st["dx"], st["n"] = (torch.empty(T, H, dtype=bf, device=dev) for _ in range(3))
                st["rstd"] = torch.empty(T, dtype=torch.float32, device=dev)
                st["dw"] = torch.empty(H, dtype=torch.float32, device=dev)
                st["ws"] = torch.empty(rn.rmsnorm_bwd_workspace_bytes(T, H) // 4 + 1, dtype=torch.float32, device=dev)
                st["out"] = torch.empty(T, H, dtype=torch.uint8, device=dev)
                st["sc"] = torch.empty(H // 128, (T + 3) // 4 * 4, dtype=torch.float32, device=dev)
                rn.rmsnorm_fwd(st["x"], st["w"], st["y"], st["rstd"], EPS)
                sets.append(st)
            row = {"H": H, "T": T}
            plans = {
                "fwd": [rn.plan_rmsnorm_fwd(st["x"], st["w"], st["y"], st["rstd"], EPS) for st in sets],
                "bwd": [rn.plan_rmsnorm_bwd(st["dy"], st["x"], st["w"], st["rstd"], st["dx"], st["dw"],
                                            deterministic=True, workspace=st["ws"]) for st in sets],
                "fp8": [rn.plan_add_rmsnorm_fp8_block_quant(st["x"], st["res"], st["w"], st["out"], st["sc"], st["n"],
                                                            EPS) for st in sets],
            }
            for op, pl in plans.items():
                nbytes = config_bytes(op, T, H, 2, 2)
                K = max(20, min(400, int(20e-3 / (nbytes / 5e12))))
                ms = per_launch_ms(torch, [[f] for f in pl], K)
                row[op] = {"us": round(ms * 1e3, 2), "GB/s": round(nbytes / (ms * 1e-3) / 1e9, 1)}
            log("sweep", row)
            out.append(row)
            del sets, plans
            torch.cuda.empty_cache()
    return out


def _card_sysfs(torch):
    """sysfs device directory of the card that holds cuda:0 (matched by PCI slot)."""
    p = torch.cuda.get_device_properties(0)
    slot = "%04x:%02x:%02x.0" % (p.pci_domain_id, p.pci_bus_id, p.pci_device_id)
    for d in sorted(glob.glob("/sys/class/drm/card*/device")):
        try:
            with open(os.path.join(d, "uevent")) as f:
                if "PCI_SLOT_NAME=" + slot in f.read():
                    return d
        except OSError:
            continue
    return None


def _dpm(path):
    """(current MHz, highest level MHz) from a pp_dpm_* table ('1: 2400Mhz *')."""
    with open(path) as f:
        lines = f.read().splitlines()
    cur, top = None, None
    for l in lines:
        if ":" not in l or "hz" not in l.lower():
            continue
        mhz = int("".join(ch for ch in l.split(":", 1)[1].lower().split("mhz")[0] if ch.isdigit()))
        top = mhz if top is None else max(top, mhz)
        if "*" in l:
            cur = mhz
    return cur, top


def clock_window(torch, plans, seconds=0.3):
    """Shader and memory clocks sampled every 5 ms while steps run (untimed)."""
    d = _card_sysfs(torch)
    if d is None:
        return None
    sclk, mclk = os.path.join(d, "pp_dpm_sclk"), os.path.join(d, "pp_dpm_mclk")
    try:
        _, sclk_top = _dpm(sclk)
        _dpm(mclk)
    except (OSError, ValueError):
        return None
    samples = {"sclk": [], "mclk": []}
    stop = threading.Event()

    def sample():
        while not stop.is_set():
            try:
                for k, path in (("sclk", sclk), ("mclk", mclk)):
                    c, _ = _dpm(path)
                    if c is not None:
                        samples[k].append(c)
            except (OSError, ValueError):
                pass
            time.sleep(0.005)

    th = threading.Thread(target=sample, daemon=True)
    t0 = time.perf_counter()
    th.start()
    i = 0
    while time.perf_counter() - t0 < seconds:
        for _ in range(50):
            run_step(plans[i % len(plans)])
            i += 1
        torch.cuda.synchronize()
    stop.set()
    th.join()

    def stats(v):
        return {"min": min(v), "median": statistics.median(v), "max": max(v)} if v else None

    return {"source": "pp_dpm_sclk / pp_dpm_mclk of %s" % d, "window_s": round(time.perf_counter() - t0, 3),
            "steps": i, "samples": len(samples["sclk"]), "sclk_mhz": stats(samples["sclk"]),
            "mclk_mhz": stats(samples["mclk"]), "sclk_top_level_mhz": sclk_top}


def per_launch_ms(torch, calls_per_set, K):
    """Average duration of one launch of an op (ms): K launches alternating the buffer
    sets, back to back on torch's current stream (the stream the library launches on),
    between two HIP events.  calls_per_set[i] is a list of callables (one op)."""
    for i in range(4):
        for f in calls_per_set[i % len(calls_per_set)]:
            f()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(K):
        for f in calls_per_set[i % len(calls_per_set)]:
            f()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / K


def run_step(calls):
    fwd, bwd, fp8 = calls
    fwd()
    bwd()
    fp8()


def host_threads():
    """Threads for the CPU baseline: the cores this process may run on."""
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:
        return max(1, os.cpu_count() or 1)


def cpu_step(oracle, d, T, H, nthreads):
    """One step of the path on the CPU oracle: forward, backward (at the forward's rstd
    rounded to fp32, as the GPU path stores it) and the fused fp8 producer, over
    contiguous row chunks run in `nthreads` threads (the oracle is plain sequential C
    and releases the GIL in each call).  Rows are independent, so every row output is
    the sequential oracle's; dw is the FP64 sum of the chunks' dw in chunk order.
    Returns (y, rstd, dx, dw, fp8 dict) with the chunks' rows in place."""
    from concurrent.futures import ThreadPoolExecutor

    import numpy as np
    n = max(1, min(nthreads, T))
    bounds = [(T * k // n, T * (k + 1) // n) for k in range(n)]
    with ThreadPoolExecutor(n) as ex:
        fw = list(ex.map(lambda b: oracle.rmsnorm_fwd(d["x"][b[0]:b[1]], d["w"], EPS), bounds))
        r32 = [f[1].astype(np.float32).astype(np.float64) for f in fw]
        bw = list(ex.map(lambda k: oracle.rmsnorm_bwd(d["dy"][bounds[k][0]:bounds[k][1]],
                                                      d["x"][bounds[k][0]:bounds[k][1]], d["w"], r32[k]),
                         range(n)))
        f8 = list(ex.map(lambda b: oracle.add_rmsnorm_fp8(d["x"][b[0]:b[1]], d["residual"][b[0]:b[1]], d["w"], EPS,
                                                          scale_ld=max(4, (b[1] - b[0] + 3) // 4 * 4)),
                         bounds))
    dw = np.zeros(H, np.float64)
    for _, dwk in bw:
        dw += dwk
    y = np.concatenate([f[0] for f in fw])
    rstd = np.concatenate([f[1] for f in fw])
    dx = np.concatenate([b[0] for b in bw])
    fp8 = {k: np.concatenate([f[k] for f in f8]) for k in ("h", "normed_bf16", "codes")}
    fp8["scale"] = np.concatenate([f["scale"][:, :b[1] - b[0]] for f, b in zip(f8, bounds)], axis=1)
    return y, rstd, dx, dw, fp8


def cpu_baseline(T, H, min_seconds=10.0):
    """The CPU oracle on whole steps of the benchmark's shape (T rows of H, bf16), on
    every core of the process's affinity mask, repeated until at least `min_seconds`
    have passed; GB/s of the same algorithmic bytes as the GPU figure."""
    import oracle
    from workloads import Workload, generate
    d = generate(Workload("cpu_sample", T, H, "bf16", "bf16", residual=True, seed=9090))
    n = host_threads()
    reps = 0
    t0 = time.perf_counter()
    while True:
        cpu_step(oracle, d, T, H, n)
        reps += 1
        el = time.perf_counter() - t0
        if el >= min_seconds:
            break
    total = sum(algorithmic_bytes(T, H).values())
    return {
        "value": round(reps * total / el / 1e9, 4),
        "unit": "GB/s",
        "cores": n,
        "kind": "oracle",
        "sample": "%d whole steps (fwd + bwd + fused fp8 producer) over T=%d rows of H=%d (bf16), FP64 C oracle "
                  "on %d threads over contiguous row chunks (dw combined in chunk order), %.1f s" % (
                      reps, T, H, n, el),
    }


def counters_for(op):
    """HBM traffic per launch from the committed rocprofv3 counter summary, if it
    was taken on the current source of that kernel."""
    if not os.path.exists(COUNTERS):
        return None
    with open(COUNTERS) as f:
        c = json.load(f)
    e = c.get("ops", {}).get(op)
    if not e or e.get("source_hash") != source_hash(op):
        return None
    return e.get("hbm_bytes_per_launch")


def main():
    global NSETS
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-next", action="store_true",
                    help="skip the residual pair, QK-norm and producer-variant timings")
    ap.add_argument("--latency", action="store_true", help="time single calls at few rows instead")
    ap.add_argument("--ceiling", action="store_true",
                    help="time plain streaming passes with each op's read:write mix instead (practical ceiling)")
    ap.add_argument("--configs", action="store_true",
                    help="time every workload configuration next to its streaming-pass twin instead")
    ap.add_argument("--only", default=None, help="with --configs: one configuration by name")
    ap.add_argument("--sweep", action="store_true", help="time fwd, bwd and fp8 over the H x T grid instead")
    ap.add_argument("--no-clocks", action="store_true", help="skip the clock-sampling window")
    ap.add_argument("--sets", type=int, default=NSETS, help="buffer sets rotated by the timings")
    ap.add_argument("--calibration-copy", action="store_true",
                    help="also run a plain 1 GiB device copy and 1 GiB read-only and write-only streaming passes "
                         "(for counter calibration under a profiler)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this build runs the RMSNorm path on a single MI355X and has "
              "no multi-GPU mode (requested --gpus %d)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch
    import bwd_fp8_block_amd as rn
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.latency:
        print(json.dumps({"latency_us_per_call": latency(torch, rn, dev, args.steps)}), flush=True)
        return
    if args.ceiling:
        import bench_probe
        print(json.dumps({"stream_mix_ceiling_T%d_H%d" % (T_ROWS, HIDDEN):
                          ceiling(torch, bench_probe, dev, T_ROWS, HIDDEN, min(args.steps, 40))}), flush=True)
        return
    if args.sweep:
        print(json.dumps({"sweep_bf16": sweep(torch, rn, dev)}), flush=True)
        return
    if args.configs:
        names = [c[0] for c in CONFIG_RUNS]
        if args.only and args.only not in names:
            print("--only: one of %s" % ", ".join(names), file=sys.stderr)
            sys.exit(2)
        import bench_probe
        print(json.dumps({"configs": configs(torch, rn, bench_probe, dev, args.only)}), flush=True)
        return
    NSETS = max(2, args.sets)
    T, H = T_ROWS, HIDDEN
    gen = torch.Generator(device=dev)
    gen.manual_seed(20261202)
    sets = [make_set(torch, gen, dev, T, H, rn) for _ in range(NSETS)]
    plans = [plan_step(rn, s) for s in sets]
    torch.cuda.synchronize()

    if args.calibration_copy:
        # kernels of known HBM traffic for the counter passes of a profiler: a 1 GiB device
        # copy (1 GiB read, 1 GiB written) and the streaming probe's read-only and write-only
        # passes over four 256 MiB streams (1 GiB read; 1 GiB written)
        import bench_probe
        a = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        q = [t.view(-1) for t in a.view(4, -1)]
        sink = torch.zeros(1, dtype=torch.int32, device=dev)
        for _ in range(3):
            bench_probe.stream_mix(q, [], 1024, wgs=256, vpt=4, order="stride", sink=sink)
            bench_probe.stream_mix([], [t.view(-1) for t in b.view(4, -1)], 1024, wgs=256, vpt=4, order="stride")
        torch.cuda.synchronize()
        del a, b, q

    for i in range(args.warmup):
        run_step(plans[i % NSETS])
    torch.cuda.synchronize()

    K = args.steps
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        run_step(plans[i % NSETS])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / K

    # Per-op launch durations (for the breakdown and the roofline), measured right
    # after the timed steps on the same buffers: HIP events would add their own
    # time to every step if recorded between the ops of the timed steps.
    per = {k: per_launch_ms(torch, [[pl[j]] for pl in plans], K) for j, k in enumerate(("fwd", "bwd", "fp8"))}
    b = algorithmic_bytes(T, H)
    total = sum(b.values())
    value = total / (ms_per_step * 1e-3) / 1e9
    ops = {}
    for k in per:
        gbs = b[k] / (per[k] * 1e-3) / 1e9
        ops[k] = {"kernel": KERNEL_NAMES[k], "bytes": b[k], "us": round(per[k] * 1e3, 3),
                  "GB/s": round(gbs, 1), "pct_of_peak": round(100 * gbs / HBM_PEAK_GBS, 2)}
    dom = max(per, key=per.get)
    achieved = b[dom] / (per[dom] * 1e-3) / 1e9
    roofline = {"bound": "hbm", "kernel": KERNEL_NAMES[dom], "achieved": round(achieved, 1),
                "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": counters_for(dom)}

    clocks = None if args.no_clocks else clock_window(torch, plans)

    next_ops = None
    if not args.no_next:
        del sets, plans
        next_ops = time_next(torch, rn, gen, dev, T, H, K, args.warmup)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(T, H)

    out = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "rmsnorm fwd + fused bwd (deterministic dw) + add-rmsnorm-fp8 1x128 block quant, "
                               "bf16 T=8192 H=4096", "T": T, "H": H, "eps": EPS,
                   "bytes_per_step": total, "pct_of_peak": round(100 * value / HBM_PEAK_GBS, 2)},
        "ops": ops,
        "roofline": roofline,
        "cpu_baseline": cpu,
        "next_ops": next_ops,
        "clocks": clocks,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
