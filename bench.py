#!/usr/bin/env python3
"""Benchmark of the Parallax forward hot path on one MI355X.

One step = one pass of the whole hot path over one batch of synthetic input:
  * the causal prefill on the 1.7B-like long workload
    (B=2, H=16, L=8192, d=128, bf16, N(0,1) inputs), then
  * one decode step on the decode workload
    (B=64, H=16, 4096-token bf16 KV cache, d=128, 16 splits),
both launched on one dedicated stream with inputs already resident in HBM.

Printed: ONE JSON line.  `value` is the prefill throughput in TFLOP/s
(algorithmic FLOP: 8d per visible (query, key) pair -- the two score and two
value products -- divided by the prefill kernel time measured with HIP events
on its own stream); the decode throughput in GB/s is reported beside it.
`roofline` describes the dominant kernel (the prefill); `cpu_baseline` times
the fp64 CPU oracle on a bounded sample of the same prefill workload.

After the timed steps, the general decode (parallax_attn_decode_paged) is
timed on the decode workload's size in 64-token pages, with 16 and with 4 kv
heads (GQA), reported under "decode_paged" (bytes: the cache read once); the
fused input projections (parallax_qkvr_project, [Q|K|V|R] = X W^T for the
1.7B-like layer: 2 x 8192 tokens, width 2048, 4 x 16 heads x 128) under
"projection"; the Walsh-Hadamard output projection (parallax_hadamard_out on
the prefill's fp32 output [2, 16, 8192, 128] -> bf16 [16384, 2048], with
alpha and beta; bytes: the output read once and y written once) under
"hadamard", with the time of a dense 2048 x 2048 output projection by the
projection kernel beside it for context; Based linear attention
(parallax_based_fwd on 2 x 16 heads x 8192 tokens, 16 query/key and 128
value features; bytes: q, k, v read once and the fp32 output written once;
and one parallax_based_decode step for 64 x 16 heads, bytes: the fp32 state
read and written) under "based"; then the prefill backward (parallax_attn_bwd: dq, dk, dv,
drho of the same prefill workload, with a seeded N(0,1) output gradient) is
timed separately and reported under "backward" (algorithmic FLOP: 16d per
visible pair); it is not part of a step.  Then the 0.6B-like causal prefill
("prefill_0.6b", matrix-core roofline) and the windowed prefill with a
128-key window and 4 sinks ("local_swa128_sink4", HBM roofline), each timed
call by call with a 512 MB buffer overwritten between calls (median and
min); the precise prefill on the headline workload ("precise"); and the
headline prefill on inputs whose scores rise along the sequence ("rising",
with the fraction of query tiles that took the exact second pass).
`--legs` selects a subset of these secondary legs (profiling runs).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "Parallax attn fwd TFLOP/s & % bf16 MFMA peak (L=8192,d=128); decode HBM GB/s"
PEAK_MFMA_TFLOPS = 2500.0   # MI355X dense bf16/f16 matrix peak
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E peak
COPY_BYTES = 1 << 30        # plain copy used to calibrate the HBM byte counters
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
KERNEL_SOURCES = {
    "prefill": os.path.join(ROOT, "parallax_local_linear_amd", "csrc", "parallax_fwd.hip"),
    "decode": os.path.join(ROOT, "parallax_local_linear_amd", "csrc", "parallax_decode.hip"),
    "decode_paged": os.path.join(ROOT, "parallax_local_linear_amd", "csrc", "parallax_decode.hip"),
    "decode_gqa": os.path.join(ROOT, "parallax_local_linear_amd", "csrc", "parallax_decode.hip"),
    "decode_mqa": os.path.join(ROOT, "parallax_local_linear_amd", "csrc", "parallax_decode.hip"),
    "based_decode": os.path.join(ROOT, "parallax_local_linear_amd", "csrc", "parallax_based.hip"),
    "backward": os.path.join(ROOT, "parallax_local_linear_amd", "csrc", "parallax_bwd.hip"),
    "projection": os.path.join(ROOT, "parallax_local_linear_amd", "csrc", "parallax_proj.hip"),
    "hadamard": os.path.join(ROOT, "parallax_local_linear_amd", "csrc", "parallax_hadamard.hip"),
    "based": os.path.join(ROOT, "parallax_local_linear_amd", "csrc", "parallax_based.hip"),
    "prefill_0.6b": os.path.join(ROOT, "parallax_local_linear_amd", "csrc", "parallax_fwd.hip"),
    "precise": os.path.join(ROOT, "parallax_local_linear_amd", "csrc", "parallax_fwd.hip"),
    "local_swa128_sink4": os.path.join(ROOT, "parallax_local_linear_amd", "csrc",
                                       "parallax_fwd.hip"),
}
# Kernels one prefill call launches, per workload.
PREFILL_KERNELS = {
    "prefill_1.7b_long": "parallax_attn_fwd call = parallax_vprep_kernel<128> + "
                         "parallax_fwd_kernel<128, true, false, false>",
    "prefill_0.6b": "parallax_attn_fwd call = parallax_vprep_kernel<64> + "
                    "parallax_fwd_kernel<64, true, false, false>",
    "local_swa128_sink4": "parallax_attn_fwd call = parallax_fwd_window_kernel<64, false, false>",
}
FLUSH_BYTES = 512 << 20     # flush buffers between timed calls: more than L2 + the 256 MB MALL
# Legs timed after the steps, each reported under its own key.
SECONDARY_LEGS = ("decode_paged", "projection", "hadamard", "based", "backward", "prefill_0.6b",
                  "local_swa128_sink4", "precise", "rising")


def parse():
    p = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--settle", type=int, default=25,
                   help="untimed steps before the warm-up steps: the GPU's clock settles over "
                        "the first 15-20 calls (the prefill runs up to 25%% slower on calls "
                        "3-15 than from call 20 on); reported as settle_steps")
    p.add_argument("--no-cpu-baseline", action="store_true",
                   help="skip timing the CPU oracle (profiling runs)")
    p.add_argument("--cpu-sample-heads", type=int, default=16,
                   help="(b,h) slices of the prefill workload the CPU oracle computes")
    p.add_argument("--cpu-single-heads", type=int, default=8,
                   help="(b,h) slices of the 0.6B-like workload the single-thread oracle run "
                        "computes")
    p.add_argument("--no-backward", action="store_true",
                   help="skip timing the prefill backward")
    p.add_argument("--legs", default=None,
                   help="comma-separated subset of the secondary legs to time after the "
                        "steps (default: all of %s)" % ",".join(SECONDARY_LEGS))
    p.add_argument("--calibrate-copy", action="store_true",
                   help="first run a plain 1 GiB device-to-device copy kernel three times, "
                        "the reference for scaling rocprofv3 FETCH_SIZE / WRITE_SIZE")
    return p.parse_args()


def source_hash(path: str) -> str:
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def measured_traffic(kernel: str):
    """HBM bytes per launch from the committed rocprofv3 counter runs, or None
    when they were taken on a different version of the kernel source."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)[kernel]
    except (OSError, KeyError, ValueError):
        return None
    if rec.get("source_sha256_16") != source_hash(KERNEL_SOURCES[kernel]):
        return None
    return rec.get("bytes_per_launch")


def host_cpu():
    """The host's CPU model, its logical CPU count and the CPUs this process may use."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        usable = None
    return {"cpu_model": model, "nproc": os.cpu_count(), "usable_cpus": usable}


def time_oracle_slices(cfg, n_heads: int, nthreads: int):
    """Seconds and algorithmic FLOP of the fp64 oracle on all rows of the first
    n_heads (b, h) slices of a prefill workload, on nthreads host threads."""
    import numpy as np
    import torch

    import oracle
    from parallax_local_linear_amd import accounting, workloads

    q, k, v, r = workloads.prefill_inputs(cfg, device="cpu")
    orc = oracle.default()
    scale = 1.0 / np.sqrt(cfg.d)
    pos = np.arange(cfg.L)
    f64 = lambda t: t.to(torch.float64).numpy()  # noqa: E731
    slices = [(b, h) for b in range(cfg.B) for h in range(cfg.H)][:n_heads]
    data = [(f64(q[b, h]), f64(r[b, h]), f64(k[b, h]), f64(v[b, h])) for b, h in slices]
    t0 = time.perf_counter()
    for Q, R, K, V in data:
        orc.rows(Q, R, pos, K, V, scale, cfg.window, cfg.n_sink, nthreads=nthreads)
    dt = time.perf_counter() - t0
    flops = 8 * cfg.d * len(slices) * accounting.visible_pairs(cfg.L, cfg.window, cfg.n_sink)
    return dt, flops, len(slices)


def cpu_baseline(cfg, n_heads: int, single_cfg, single_heads: int):
    """The fp64 oracle on the host: all rows of the first n_heads (b, h) slices
    of the headline workload on the default thread count, and one
    single-thread run on single_heads slices of single_cfg."""
    import oracle

    nthreads = oracle.default_threads()
    dt, flops, n = time_oracle_slices(cfg, n_heads, nthreads)
    dt1, flops1, n1 = time_oracle_slices(single_cfg, single_heads, 1)
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": nthreads, "kind": "oracle",
            "sample": "all %d rows of %d of the %d (b,h) slices of %s (%.3g GFLOP, %.1f s)"
                      % (cfg.L, n, cfg.B * cfg.H, cfg.name, flops / 1e9, dt),
            "threads_used": nthreads,
            "host": host_cpu(),
            "single_thread": {
                "value": flops1 / dt1 / 1e12, "unit": "TFLOP/s", "cores": 1,
                "sample": "all %d rows of %d of the %d (b,h) slices of %s (%.3g GFLOP, %.1f s)"
                          % (single_cfg.L, n1, single_cfg.B * single_cfg.H, single_cfg.name,
                             flops1 / 1e9, dt1)}}


class CacheFlush:
    """Evicts a call's inputs from L2 and the MALL between timed calls.

    `clean` (the default) overwrites one 512 MB buffer, which evicts
    everything else, then reads a second one, which displaces the first
    one's dirty lines: the timed call starts with its inputs in HBM and
    caches that hold no dirty data.  `dirty` only overwrites the buffer, so
    the timed call also pays for writing 256 MB of the flush's own lines
    back to HBM as its reads evict them."""

    def __init__(self, dev):
        import torch
        self.a = torch.zeros(FLUSH_BYTES, dtype=torch.uint8, device=dev)
        self.b = torch.zeros(FLUSH_BYTES // 8, dtype=torch.int64, device=dev)
        self.total = None

    def __call__(self, i, dirty=False):
        self.a.fill_(i & 0xff)
        if not dirty:
            self.total = self.b.sum()


def time_each_call(fn, runs, warmup, stream, flush=None, dirty=False):
    """Per-call times (ms) from HIP events recorded on `stream` around each
    call; with `flush` (a CacheFlush), the caches are flushed on the same
    stream before every call, outside the timed region."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    times = []
    for i in range(runs):
        if flush is not None:
            with torch.cuda.stream(stream):
                flush(i, dirty)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        fn()
        e1.record(stream)
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1))
    return times


def time_prefill_leg(cfg, bound, runs, warmup, stream, flush=None, precise=False):
    """One prefill workload timed call by call (median and min over `runs`),
    with its roofline: the matrix-core peak for the compute-bound causal
    workloads, HBM for the windowed one (8d FLOP per visible pair; bytes:
    q, k, v, r read once, the fp32 output and lse written once).  With
    `precise`, the call is parallax_attn_fwd_precise (same FLOP count)."""
    import torch

    from parallax_local_linear_amd import (accounting, parallax_attn_fwd,
                                           parallax_attn_fwd_precise,
                                           parallax_attn_fwd_workspace_size, workloads)
    dev = torch.device("cuda:0")
    fwd = parallax_attn_fwd_precise if precise else parallax_attn_fwd
    q, k, v, r = workloads.prefill_inputs(cfg, device=dev)
    o = torch.empty(q.shape, dtype=torch.float32, device=dev)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
    ws = torch.empty(max(1, parallax_attn_fwd_workspace_size(cfg.B, cfg.H, cfg.L, cfg.d)),
                     dtype=torch.uint8, device=dev)
    call = lambda: fwd(q, k, v, r, window=cfg.window, n_sink=cfg.n_sink, out=o, lse=lse,  # noqa: E731
                       workspace=ws, stream=stream)
    times = time_each_call(call, runs, warmup, stream, flush)
    dirty = time_each_call(call, runs, 0, stream, flush, dirty=True) if flush else None
    med = statistics.median(times)
    flops = accounting.prefill_flops(cfg)
    nbytes = accounting.prefill_bytes(cfg)
    tflops = flops / (med * 1e-3) / 1e12
    gbs = nbytes / (med * 1e-3) / 1e9
    if bound == "hbm":
        roof = {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(gbs / PEAK_HBM_GBS, 4), "algorithmic_bytes_per_launch": nbytes}
    else:
        roof = {"bound": "mfma", "achieved": round(tflops, 2), "peak": PEAK_MFMA_TFLOPS,
                "unit": "TFLOP/s", "frac": round(tflops / PEAK_MFMA_TFLOPS, 4),
                "algorithmic_flop_per_launch": flops}
    roof["traffic"] = measured_traffic("precise" if precise else cfg.name)
    roof["kernel"] = PREFILL_KERNELS[cfg.name]
    if precise:
        roof["kernel"] = (roof["kernel"].replace("parallax_attn_fwd call",
                                                 "parallax_attn_fwd_precise call")
                          .replace("false, false>", "false, true>"))
    out = {"workload": cfg.name, "B": cfg.B, "H": cfg.H, "L": cfg.L, "d": cfg.d,
           "window": cfg.window, "n_sink": cfg.n_sink,
           "ms_median": round(med, 4), "ms_min": round(min(times), 4), "runs": runs,
           "mall_flush": flush is not None,
           "value": roof["achieved"], "unit": roof["unit"],
           "tflops": round(tflops, 2), "gbs": round(gbs, 1), "roofline": roof}
    if flush:
        out["flush"] = ("512 MB written, then another 512 MB read, before each call "
                        "(inputs out of L2 and the MALL, no dirty lines left)")
        out["ms_median_dirty_flush"] = round(statistics.median(dirty), 4)
        out["ms_min_dirty_flush"] = round(min(dirty), 4)
    return out


def recomputed_tiles(ws, cfg):
    """Query tiles the last prefill call on workspace `ws` recomputed: the
    counter the library leaves after the f16 V image."""
    import torch
    image = cfg.B * cfg.H * (-(-cfg.L // 32)) * 32 * cfg.d * 2
    return int(ws[image:image + 4].view(torch.int32).item())


def time_rising(cfg, runs, warmup, stream):
    """The prefill call on inputs whose scores rise along the sequence (most
    query tiles then repeat with the exact row maxima): the cost of that
    second pass at full size.  Same FLOP count as the plain call."""
    import statistics

    import torch

    from parallax_local_linear_amd import (accounting, parallax_attn_fwd,
                                           parallax_attn_fwd_workspace_size, workloads)
    dev = torch.device("cuda:0")
    q, k, v, r = workloads.rising_inputs(cfg.B, cfg.H, cfg.L, cfg.d, seed=1000 + cfg.seed,
                                         device=dev)
    o = torch.empty(q.shape, dtype=torch.float32, device=dev)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
    ws = torch.empty(parallax_attn_fwd_workspace_size(cfg.B, cfg.H, cfg.L, cfg.d),
                     dtype=torch.uint8, device=dev)
    times = time_each_call(lambda: parallax_attn_fwd(q, k, v, r, out=o, lse=lse, workspace=ws,
                                                     stream=stream), runs, warmup, stream)
    med = statistics.median(times)
    n_tiles = cfg.B * cfg.H * (-(-cfg.L // 128))
    count = recomputed_tiles(ws, cfg)
    tflops = accounting.prefill_flops(cfg) / (med * 1e-3) / 1e12
    return {"workload": cfg.name + " with rising scores", "ms_median": round(med, 4),
            "ms_min": round(min(times), 4), "value": round(tflops, 2), "unit": "TFLOP/s",
            "recomputed_tiles": count, "tiles": n_tiles,
            "recompute_fraction": round(count / n_tiles, 4),
            "inputs": "q = 3u + 0.1z, k_j = (46 (d/64)^1/2 j/L) u + 0.1z, v ~ N(0,1), "
                      "r ~ 0.25 N(0,1)"}


def time_backward(cfg, steps, warmup, stream):
    """Mean time (HIP events on `stream`) of parallax_attn_bwd on one prefill workload."""
    import torch

    from parallax_local_linear_amd import (accounting, parallax_attn_bwd,
                                           parallax_attn_bwd_workspace_size,
                                           parallax_attn_fwd_train, workloads)
    dev = torch.device("cuda:0")
    q, k, v, r = workloads.prefill_inputs(cfg, device=dev)
    dout = workloads.prefill_grad(cfg, device=dev)
    o, lse, sbar, pv = parallax_attn_fwd_train(q, k, v, r, window=cfg.window, n_sink=cfg.n_sink,
                                               stream=stream)
    grads = tuple(torch.empty(q.shape, dtype=torch.float32, device=dev) for _ in range(4))
    ws = torch.empty(parallax_attn_bwd_workspace_size(cfg.B, cfg.H, cfg.L, cfg.d),
                     dtype=torch.uint8, device=dev)

    def call():
        parallax_attn_bwd(q, k, v, r, dout, o, lse, sbar, pv, window=cfg.window,
                          n_sink=cfg.n_sink, grads=grads, workspace=ws, stream=stream)
    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        call()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    flops = accounting.prefill_bwd_flops(cfg)
    tflops = flops / (ms * 1e-3) / 1e12
    return {
        "workload": cfg.name,
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "ms": round(ms, 4),
        "steps": steps,
        "roofline": {
            "bound": "mfma",
            "achieved": round(tflops, 2),
            "peak": PEAK_MFMA_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(tflops / PEAK_MFMA_TFLOPS, 4),
            "traffic": measured_traffic("backward"),
            "algorithmic_flop_per_launch": flops,
            "kernel": "parallax_attn_bwd call = parallax_bwd_stats_kernel<128> + "
                      "parallax_bwd_record_kernel<128> + parallax_bwd_kv_kernel<128> + "
                      "parallax_bwd_q_kernel<128>",
        },
    }


def time_decode_paged(dcfg, steps, warmup, stream):
    """General decode on the decode workload's size: 64-token pages in a shuffled
    pool, 16 query heads over 16, 4 or 1 kv heads.  GB/s counts the cache once."""
    import torch

    from parallax_local_linear_amd import (parallax_attn_decode_paged,
                                           parallax_attn_decode_paged_workspace_size)
    dev = torch.device("cuda:0")
    B, Hq, Lmax, d, page = dcfg.B, dcfg.H, dcfg.Lmax, dcfg.d, 64
    # Key-split workspace of the grouped-head calls, allocated once.
    ws = torch.empty(parallax_attn_decode_paged_workspace_size(B, Hq, d), dtype=torch.uint8,
                     device=dev)
    out = []
    for Hkv in (16, 4, 1):
        g = torch.Generator(device=dev).manual_seed(2024 + Hkv)
        q = torch.randn((B, Hq, d), generator=g, device=dev).to(torch.bfloat16)
        r = torch.randn((B, Hq, d), generator=g, device=dev).to(torch.bfloat16)
        n_pages = B * Lmax // page
        kp = torch.randn((n_pages, page, Hkv, d), generator=g, device=dev).to(torch.bfloat16)
        vp = torch.randn((n_pages, page, Hkv, d), generator=g, device=dev).to(torch.bfloat16)
        perm = torch.randperm(n_pages, generator=torch.Generator().manual_seed(Hkv))
        table = perm.view(B, Lmax // page).to(torch.int32).to(dev)
        o = torch.empty((B, Hq, d), dtype=torch.float32, device=dev)
        lse = torch.empty((B, Hq), dtype=torch.float32, device=dev)

        def call():
            parallax_attn_decode_paged(q, r, kp, vp, table, None, num_splits=dcfg.num_splits,
                                       out=o, lse=lse, workspace=ws, stream=stream)
        for _ in range(warmup):
            call()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(steps):
            call()
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / steps
        nbytes = 2 * B * Hkv * Lmax * d * 2 + B * Hq * (2 * d * 2 + d * 4 + 4) + B * Lmax // page * 4
        gbs = nbytes / (ms * 1e-3) / 1e9
        # Four or more query heads per kv head take the matrix-core kernel.
        gqa = Hq // Hkv >= 4
        key = "decode_paged" if not gqa else ("decode_gqa" if Hkv == 4 else "decode_mqa")
        out.append({"Hq": Hq, "Hkv": Hkv, "page": page, "ms": round(ms, 4),
                    "value": round(gbs, 1), "unit": "GB/s",
                    "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS,
                                 "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4),
                                 "traffic": measured_traffic(key),
                                 "algorithmic_bytes_per_launch": nbytes,
                                 "kernel": "parallax_decode_gqa_kernel<128,...>" if gqa
                                           else "parallax_decode_paged_kernel<128,...>"}})
        del kp, vp
    return out


def time_projection(pcfg, steps, warmup, stream):
    """parallax_qkvr_project on the prefill workload's layer: M = B L tokens,
    K = H d, N = 4 H d.  TFLOP/s at 2 M N K FLOP per call."""
    import torch

    from parallax_local_linear_amd import parallax_qkvr_project
    dev = torch.device("cuda:0")
    M, K, N = pcfg.B * pcfg.L, pcfg.H * pcfg.d, 4 * pcfg.H * pcfg.d
    g = torch.Generator(device=dev).manual_seed(99)
    x = torch.randn((M, K), generator=g, device=dev).to(torch.bfloat16)
    w = (torch.randn((N, K), generator=g, device=dev) * K ** -0.5).to(torch.bfloat16)
    y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    for _ in range(warmup):
        parallax_qkvr_project(x, w, out=y, stream=stream)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        parallax_qkvr_project(x, w, out=y, stream=stream)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    flops = 2 * M * N * K
    tf = flops / (ms * 1e-3) / 1e12
    return {"M": M, "N": N, "K": K, "ms": round(ms, 4), "value": round(tf, 2), "unit": "TFLOP/s",
            "roofline": {"bound": "mfma", "achieved": round(tf, 2), "peak": PEAK_MFMA_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(tf / PEAK_MFMA_TFLOPS, 4),
                         "traffic": measured_traffic("projection"),
                         "algorithmic_flop_per_launch": flops,
                         "kernel": "parallax_proj_kernel"}}


def _time_calls(fn, steps, warmup, stream):
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        fn()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def time_hadamard(pcfg, steps, warmup, stream):
    """parallax_hadamard_out on the prefill workload's fp32 output: bytes =
    4 B L H d read + 2 B L H d written + alpha and beta; and, for context, a
    dense n x n output projection of the same tokens (bf16, projection kernel)."""
    import torch

    from parallax_local_linear_amd import parallax_hadamard_out, parallax_qkvr_project
    dev = torch.device("cuda:0")
    B, H, L, d = pcfg.B, pcfg.H, pcfg.L, pcfg.d
    n, M = H * d, B * L
    g = torch.Generator(device=dev).manual_seed(98)
    o = torch.randn((B, H, L, d), generator=g, device=dev)
    alpha = 1.0 + 0.1 * torch.randn((n,), generator=g, device=dev)
    beta = 0.1 * torch.randn((n,), generator=g, device=dev)
    y = torch.empty((B, L, n), dtype=torch.bfloat16, device=dev)
    ms = _time_calls(lambda: parallax_hadamard_out(o, alpha, beta, out=y, stream=stream),
                     steps, warmup, stream)
    nbytes = M * n * 4 + M * n * 2 + 2 * n * 4
    gbs = nbytes / (ms * 1e-3) / 1e9
    x = torch.randn((M, n), generator=g, device=dev).to(torch.bfloat16)
    w = (torch.randn((n, n), generator=g, device=dev) * n ** -0.5).to(torch.bfloat16)
    yd = torch.empty((M, n), dtype=torch.bfloat16, device=dev)
    ms_dense = _time_calls(lambda: parallax_qkvr_project(x, w, out=yd, stream=stream),
                           steps, warmup, stream)
    return {"B": B, "H": H, "L": L, "d": d, "ms": round(ms, 4), "value": round(gbs, 1),
            "unit": "GB/s", "dense_output_projection_ms": round(ms_dense, 4),
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS,
                         "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4),
                         "traffic": measured_traffic("hadamard"),
                         "algorithmic_bytes_per_launch": nbytes,
                         "kernel": "parallax_hadamard_kernel<11>"}}


def time_based(steps, warmup, stream):
    """parallax_based_fwd on the Based workload, and one decode step per
    (batch, head) for 64 sequences x 16 heads on the state a prefill returns."""
    import torch

    from parallax_local_linear_amd import (parallax_based_decode, parallax_based_fwd,
                                           parallax_based_workspace_size, workloads)
    cfg = workloads.BASED
    dev = torch.device("cuda:0")
    q, k, v = workloads.based_inputs(cfg, device=dev)
    o = torch.empty((cfg.B, cfg.H, cfg.L, cfg.dv), dtype=torch.float32, device=dev)
    ws = torch.empty(parallax_based_workspace_size(cfg.B, cfg.H, cfg.L, cfg.dk, cfg.dv),
                     dtype=torch.uint8, device=dev)
    ms = _time_calls(lambda: parallax_based_fwd(q, k, v, scale=cfg.scale, out=o, workspace=ws,
                                                stream=stream), steps, warmup, stream)
    tokens = cfg.B * cfg.H * cfg.L
    nbytes = tokens * (2 * cfg.dk * 2 + cfg.dv * 2 + cfg.dv * 4)
    gbs = nbytes / (ms * 1e-3) / 1e9
    # decode: 64 sequences x 16 heads, state of a 4096-token prefill
    Bd = 64
    g = torch.Generator(device=dev).manual_seed(97)
    qd, kd = (torch.randn((Bd, cfg.H, cfg.dk), generator=g, device=dev).to(torch.bfloat16)
              for _ in range(2))
    vd = torch.randn((Bd, cfg.H, cfg.dv), generator=g, device=dev).to(torch.bfloat16)
    kp = torch.randn((Bd, cfg.H, 512, cfg.dk), generator=g, device=dev).to(torch.bfloat16)
    vp = torch.randn((Bd, cfg.H, 512, cfg.dv), generator=g, device=dev).to(torch.bfloat16)
    _, state = parallax_based_fwd(kp, kp, vp, scale=cfg.scale, return_state=True, stream=stream)
    od = torch.empty((Bd, cfg.H, cfg.dv), dtype=torch.float32, device=dev)
    ms_d = _time_calls(lambda: parallax_based_decode(qd, kd, vd, state, scale=cfg.scale, out=od,
                                                     stream=stream), steps, warmup, stream)
    dbytes = Bd * cfg.H * (2 * state[0, 0].numel() * 4 + 2 * cfg.dk * 2 + cfg.dv * 6)
    dgbs = dbytes / (ms_d * 1e-3) / 1e9
    return {"workload": cfg.name, "B": cfg.B, "H": cfg.H, "L": cfg.L, "dk": cfg.dk,
            "dv": cfg.dv, "ms": round(ms, 4), "value": round(gbs, 1), "unit": "GB/s",
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS,
                         "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4),
                         "traffic": measured_traffic("based"),
                         "algorithmic_bytes_per_launch": nbytes,
                         "kernel": "parallax_based_fwd call = parallax_based_state_kernel<128> + "
                                   "parallax_based_scan_kernel<128> + "
                                   "parallax_based_out_kernel<128>"},
            "decode": {"B": Bd, "H": cfg.H, "ms": round(ms_d, 4), "value": round(dgbs, 1),
                       "unit": "GB/s", "frac": round(dgbs / PEAK_HBM_GBS, 4),
                       "traffic": measured_traffic("based_decode"),
                       "algorithmic_bytes_per_launch": dbytes,
                       "kernel": "parallax_based_decode_kernel<128>"}}


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU only: the library runs on a single MI355X and has no "
              "multi-GPU path (requested --gpus %d)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch

    from parallax_local_linear_amd import (accounting, parallax_attn_decode, parallax_attn_fwd,
                                           parallax_attn_fwd_workspace_size, workloads)
    from parallax_local_linear_amd.binding import LIBRARY

    if not os.path.exists(LIBRARY):
        from parallax_local_linear_amd import build as lib_build
        lib_build.build()
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)

    dev = torch.device("cuda:0")
    pcfg = workloads.PREFILL_17B
    dcfg = workloads.DECODE
    print("[bench] generating inputs", file=sys.stderr, flush=True)
    q, k, v, r = workloads.prefill_inputs(pcfg, device=dev)
    o = torch.empty(q.shape, dtype=torch.float32, device=dev)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
    ws = torch.empty(parallax_attn_fwd_workspace_size(pcfg.B, pcfg.H, pcfg.L, pcfg.d),
                     dtype=torch.uint8, device=dev)
    dq, dk, dv, dr = workloads.decode_inputs(dcfg, device=dev)
    do = torch.empty(dq.shape, dtype=torch.float32, device=dev)
    dlse = torch.empty(dq.shape[:2], dtype=torch.float32, device=dev)
    stream = torch.cuda.Stream(device=dev)
    torch.cuda.synchronize()
    if args.calibrate_copy:
        src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print("[bench] copy calibration: 3 x %d bytes read and written" % COPY_BYTES,
              file=sys.stderr, flush=True)
        del src, dst

    def step(events=None):
        if events is not None:
            events[0].record(stream)
        parallax_attn_fwd(q, k, v, r, window=pcfg.window, n_sink=pcfg.n_sink, out=o, lse=lse,
                          workspace=ws, stream=stream)
        if events is not None:
            events[1].record(stream)
        parallax_attn_decode(dq, dr, dk, dv, None, num_splits=dcfg.num_splits, out=do,
                             lse=dlse, stream=stream)
        if events is not None:
            events[2].record(stream)

    print("[bench] settle %d, warmup %d" % (args.settle, args.warmup), file=sys.stderr,
          flush=True)
    for _ in range(args.settle + args.warmup):
        step()
    torch.cuda.synchronize()

    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record(stream)
    for i in range(args.steps):
        step(ev[i])
    t_end.record(stream)
    torch.cuda.synchronize()
    print("[bench] timed %d steps" % args.steps, file=sys.stderr, flush=True)

    total_ms = t_start.elapsed_time(t_end)
    n_tiles = pcfg.B * pcfg.H * (-(-pcfg.L // 128))
    recomputed = recomputed_tiles(ws, pcfg)
    pre_ms = [e[0].elapsed_time(e[1]) for e in ev]
    dec_ms = [e[1].elapsed_time(e[2]) for e in ev]
    pre_avg = sum(pre_ms) / len(pre_ms)
    dec_avg = sum(dec_ms) / len(dec_ms)

    p_flops = accounting.prefill_flops(pcfg)
    p_tflops = p_flops / (pre_avg * 1e-3) / 1e12
    d_bytes = accounting.decode_bytes(dcfg)
    d_gbs = d_bytes / (dec_avg * 1e-3) / 1e9

    res = {
        "metric": METRIC,
        "value": round(p_tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle_steps": args.settle,
        "ms_per_step": round(total_ms / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "%s + %s" % (pcfg.name, dcfg.name),
            "prefill": {"B": pcfg.B, "H": pcfg.H, "L": pcfg.L, "d": pcfg.d, "mask": "causal",
                        "inputs": "N(0,1) bf16, seed %d" % pcfg.seed},
            "decode": {"B": dcfg.B, "H": dcfg.H, "Lmax": dcfg.Lmax, "d": dcfg.d,
                       "num_splits": dcfg.num_splits, "inputs": "N(0,1) bf16, seed %d" % dcfg.seed},
            "precision": "bf16 inputs; bf16 score MFMA, f16 value MFMA, fp32 accumulate; fp32 O",
        },
        "prefill_ms": round(pre_avg, 4),
        "prefill_recompute": {"recomputed_tiles": recomputed, "tiles": n_tiles,
                              "fraction": round(recomputed / n_tiles, 4)},
        "prefill_ms_median": round(statistics.median(pre_ms), 4),
        "prefill_ms_min": round(min(pre_ms), 4),
        "roofline": {
            "bound": "mfma",
            "achieved": round(p_tflops, 2),
            "peak": PEAK_MFMA_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(p_tflops / PEAK_MFMA_TFLOPS, 4),
            "traffic": measured_traffic("prefill"),
            "algorithmic_flop_per_launch": p_flops,
            "kernel": PREFILL_KERNELS[pcfg.name],
        },
        "decode": {
            "value": round(d_gbs, 1),
            "unit": "GB/s",
            "ms": round(dec_avg, 4),
            "ms_median": round(statistics.median(dec_ms), 4),
            "ms_min": round(min(dec_ms), 4),
            "roofline": {
                "bound": "hbm",
                "achieved": round(d_gbs, 1),
                "peak": PEAK_HBM_GBS,
                "unit": "GB/s",
                "frac": round(d_gbs / PEAK_HBM_GBS, 4),
                "traffic": measured_traffic("decode"),
                "algorithmic_bytes_per_launch": d_bytes,
                "kernel": "parallax_decode_kernel<128,16>",
            },
        },
    }
    legs = set(SECONDARY_LEGS if args.legs is None else args.legs.split(","))
    unknown = legs - set(SECONDARY_LEGS)
    if unknown:
        sys.exit("unknown --legs %s (known: %s)" % (",".join(sorted(unknown)),
                                                    ",".join(SECONDARY_LEGS)))
    if args.no_backward:
        legs.discard("backward")
    few, warm = min(args.steps, 20), max(1, min(args.warmup, 3))
    if "decode_paged" in legs:
        print("[bench] timing the general decode", file=sys.stderr, flush=True)
        res["decode_paged"] = time_decode_paged(dcfg, few, warm, stream)
    if "projection" in legs:
        print("[bench] timing the projections", file=sys.stderr, flush=True)
        res["projection"] = time_projection(pcfg, few, warm, stream)
    if "hadamard" in legs:
        print("[bench] timing the Hadamard output projection", file=sys.stderr, flush=True)
        res["hadamard"] = time_hadamard(pcfg, few, warm, stream)
    if "based" in legs:
        print("[bench] timing Based linear attention", file=sys.stderr, flush=True)
        res["based"] = time_based(few, warm, stream)
    if "backward" in legs:
        print("[bench] timing the backward", file=sys.stderr, flush=True)
        res["backward"] = time_backward(pcfg, few, warm, stream)
    flush = CacheFlush(dev)
    if "prefill_0.6b" in legs:
        print("[bench] timing the 0.6B-like prefill", file=sys.stderr, flush=True)
        res["prefill_0.6b"] = time_prefill_leg(workloads.PREFILL_06B, "mfma", 20, 5, stream,
                                               flush)
    if "local_swa128_sink4" in legs:
        print("[bench] timing the windowed prefill", file=sys.stderr, flush=True)
        res["local_swa128_sink4"] = time_prefill_leg(workloads.LOCAL, "hbm", 20, 5, stream,
                                                     flush)
    del flush
    if "precise" in legs:
        print("[bench] timing the precise prefill", file=sys.stderr, flush=True)
        res["precise"] = time_prefill_leg(pcfg, "mfma", 20, 3, stream, precise=True)
    if "rising" in legs:
        print("[bench] timing the prefill on rising scores", file=sys.stderr, flush=True)
        res["rising"] = time_rising(pcfg, 10, 2, stream)
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle", file=sys.stderr, flush=True)
        res["cpu_baseline"] = cpu_baseline(pcfg, args.cpu_sample_heads, workloads.PREFILL_06B,
                                           args.cpu_single_heads)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
