"""Benchmark: Fibottention sparse attention, forward + backward, on one MI355X.

One step = one forward and one backward pass over one batch of a workload
(default: the ViT-B/16 attention, B=64, H=12, N=197, d_h=64, bf16 inputs,
fp32 accumulation), inputs resident in HBM.  Several buffer sets are rotated
so that each pass reads data that the previous passes did not leave in the
256 MB last-level cache (the backward of a step works on a set whose forward
ran half a rotation earlier, as in a network with other layers in between).

Prints one JSON line:
  * value: Q.K pairs per second over forward + backward, from events around
    K back-to-back steps (launch gaps included), taken after the per-pass
    timings below and W warmup steps, so at the GPU's steady clocks;
  * kernels: each pass timed alone over max(K, 100) launches, every launch
    bracketed by events the GPU records at its kernels' own start and end
    (fibatt_time_next_call): median, p10, p90;
  * roofline: the dominant pass against the 8 TB/s HBM peak, with the
    algorithmic bytes of the scope table (forward: Q, K, V read, O and LSE
    written; backward: Q, K, V, dO, O and LSE read, fp32 dQ, dK, dV written)
    and, as a second denominator, a hand-written HIP stream kernel that moves
    the same bytes with nothing else in it (fibatt_hbm_stream);
  * workloads: the same per-pass figures for all five workloads, their
    algorithmic flops per second over the 157.3 TFLOP/s vector-ALU peak, and, where
    the committed counters match the current sources, the L2-miss read rate
    (FETCH_SIZE / time) over the rate at which the XCDs' L2s can be filled
    from beyond them (fibatt_fabric_read, l2_fill_ref_gbps): the bound of
    the long-sequence kernels, whose rows at large distances miss L2;
  * cpu_baseline: the fp64 CPU oracle on this host's cores (a process pool,
    one BLAS thread per worker), run before the GPU is touched;
  * pages_context: the figures the Fibottention pages state themselves.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 2]
"""

from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import math
import multiprocessing as mp
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E, published
VALU_PEAK_TFLOPS = 157.3  # MI355X vector fp32 (packed or dot2), published
FLOPS_PER_PAIR_ELEM = {"fwd": 4, "bwd": 10}  # scope table: per pair and element of d_h
MAX_POOL = 16           # worker processes for the CPU oracle (the host's share of cores)


# ---------------------------------------------------------------------------
# Counting: pairs and algorithmic bytes per pass
# ---------------------------------------------------------------------------

def _pairs_per_slab(N, F):
    return [int(sum(2 * (N - int(f)) if f > 0 else N for f in fs)) for fs in F]


def _cls_extra_pairs_per_slab(N, F):
    """Pairs the class-token mask adds to each head's support: (0, k) and
    (k, 0) for every k >= 1 that is not a distance, and (0, 0) when 0 is not
    a distance."""
    out = []
    for fs in F:
        pos = len([f for f in fs if f >= 1])
        out.append(2 * (N - 1 - pos) + (0 if 0 in fs else 1))
    return out


def pass_bytes(wl, esize):
    """Algorithmic HBM bytes per pass (whole batch), as the scope table counts
    them, and the backward without O (this backward computes D = sum P dP
    itself and does not read O).

    forward : read Q, K, V (input dtype); write O (input dtype), LSE (fp32).
    backward: read Q, K, V, dO, O (input dtype), LSE (fp32); write dQ, dK, dV (fp32).
    """
    rows = wl.B * wl.H * wl.N
    row = wl.d * esize
    fwd = rows * (4 * row + 4)
    bwd = rows * (5 * row + 4 + 3 * wl.d * 4)
    bwd_moved = rows * (4 * row + 4 + 3 * wl.d * 4)
    return int(fwd), int(bwd), int(bwd_moved)


# Kernels each pass dispatches, per workload (the dispatch rules of
# csrc/fwd.hip and csrc/bwd.hip for these shapes), and the sources whose hash
# identifies the build a counter measurement was taken on.
KERNELS = {
    1: {"fwd": ["fwd_slab_kernel"], "bwd": ["bwd_slab_kernel"]},
    2: {"fwd": ["fwd_slab_bf16_kernel"], "bwd": ["bwd_slab_bf16_kernel"]},
    3: {"fwd": ["fwd_win_bf16_kernel"], "bwd": ["bwd_dq_win_kernel", "bwd_dkdv_tile_kernel"]},
    4: {"fwd": ["fwd_win_bf16_kernel"], "bwd": ["bwd_dq_win_kernel", "bwd_dkdv_tile_kernel"]},
    5: {"fwd": ["fwd_tile_bf16_kernel"], "bwd": ["bwd_dq_tile_kernel", "bwd_dkdv_tile_kernel"]},
}
SOURCES = {
    "fwd_slab_kernel": ["fwd.hip"],
    "bwd_slab_kernel": ["bwd.hip"],
    "fwd_slab_bf16_kernel": ["fwd_slab_bf16.hip", "slab_bf16_common.h"],
    "bwd_slab_bf16_kernel": ["bwd_slab_bf16.hip", "slab_bf16_common.h"],
    "fwd_tile_bf16_kernel": ["fwd_tile_bf16.hip", "tile_bf16_common.h", "slab_bf16_common.h"],
    "fwd_win_bf16_kernel": ["fwd_tile_bf16.hip", "window_bf16_common.h", "tile_bf16_common.h",
                            "slab_bf16_common.h"],
    "bwd_dq_tile_kernel": ["bwd_tile_bf16.hip", "tile_bf16_common.h", "slab_bf16_common.h"],
    "bwd_dkdv_tile_kernel": ["bwd_tile_bf16.hip", "tile_bf16_common.h", "slab_bf16_common.h"],
    "bwd_dq_win_kernel": ["bwd_tile_bf16.hip", "window_bf16_common.h", "tile_bf16_common.h",
                          "slab_bf16_common.h"],
}


def source_hash(kernel):
    """Hash of a kernel's sources and of the compile flags of its own file."""
    from structured_sparse_head_amd.build import FILE_FLAGS
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "structured_sparse_head_amd", "csrc")
    for f in SOURCES[kernel] + ["kernel_common.h", "problem.h", "fib_offsets.h", "launch.h"]:
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(fh.read())
    for f in SOURCES[kernel]:
        h.update(" ".join(FILE_FLAGS.get(f, [])).encode())
    return h.hexdigest()[:16]


def measured_traffic(workload, pass_name):
    """HBM bytes per pass (read + write, summed over the pass's kernels) from
    the committed counter summary profiles/hbm_traffic.txt, or None unless
    every kernel of the pass was measured on this workload with the current
    sources."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic.txt")
    if not os.path.exists(path):
        return None
    table = {}
    with open(path) as fh:
        for line in fh:
            f = line.split()
            if len(f) == 5 and not f[0].startswith("#"):
                table[(f[0], f[1], f[2])] = int(f[3]) + int(f[4])
    total = 0
    for k in KERNELS[workload][pass_name]:
        key = (f"W{workload}", k, source_hash(k))
        if key not in table:
            return None
        total += table[key]
    return total


def measured_fetch(workload, pass_name):
    """L2-miss read bytes per pass (FETCH_SIZE, scaled) from the same summary,
    or None (see measured_traffic)."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic.txt")
    if not os.path.exists(path):
        return None
    table = {}
    with open(path) as fh:
        for line in fh:
            f = line.split()
            if len(f) == 5 and not f[0].startswith("#"):
                table[(f[0], f[1], f[2])] = int(f[3])
    total = 0
    for k in KERNELS[workload][pass_name]:
        key = (f"W{workload}", k, source_hash(k))
        if key not in table:
            return None
        total += table[key]
    return total


FABRIC_MIB = 64     # larger than all eight L2s together (32 MiB)
FABRIC_PASSES = 4


def fabric_ref(hip, torch, fa, dev, n=20):
    """Rate (GB/s) at which the XCDs' L2s fill from beyond them
    (fibatt_fabric_read over a buffer larger than every L2), median of n."""
    buf = torch.zeros(FABRIC_MIB * 1024 * 1024 // 4, dtype=torch.int32, device=dev)
    out = torch.empty(fa.FABRIC_OUT_BYTES // 4, dtype=torch.int32, device=dev)
    for _ in range(2):
        fa.fabric_read(buf, FABRIC_PASSES, out)
    t = kernel_times(hip, lambda i: fa.fabric_read(buf, FABRIC_PASSES, out), n)
    delivered = 8 * buf.numel() * 4 * FABRIC_PASSES
    del buf, out
    return delivered / (t[n // 2] * 1e-3) / 1e9


def pages_context(wl, pairs_per_pass):
    with open(os.path.join(ROOT, "tests", "golden", "pages_figures.json")) as fh:
        g = json.load(fh)
    dense = wl.B * wl.H * wl.N * wl.N
    return {
        "complexity": g["complexity"]["statement"] + " (" + g["complexity"]["source"] + ")",
        "kept_share": f"about {g['kept_interactions']['value_percent']}% of pairwise interactions "
                      f"kept at w_max = {g['kept_interactions']['w_max']} ("
                      + g["kept_interactions"]["source"] + ")",
        "hardware_stated_by_pages": "none (the pages give counts and accuracy, no timings)",
        "kept_share_this_workload": pairs_per_pass / dense,
    }


# ---------------------------------------------------------------------------
# CPU oracle baseline (process pool; runs before the GPU is initialised)
# ---------------------------------------------------------------------------

_POOL_DATA = {}


def _pool_init():
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(1)
    except Exception:  # pragma: no cover
        pass


def _oracle_task(args):
    """Forward + backward of the oracle on batch entries [b0, b1) and heads
    [h0, h1) of the inputs in _POOL_DATA (inherited by fork)."""
    import oracle  # test infrastructure; used only for this baseline leg

    b0, b1, h0, h1 = args
    d = _POOL_DATA
    x = {n: d[n][b0:b1, h0:h1] for n in ("q", "k", "v", "do")}
    F = d["F"][h0:h1]
    oracle.forward(x["q"], x["k"], x["v"], F, cls=d["cls"])
    oracle.backward(x["q"], x["k"], x["v"], x["do"], F, cls=d["cls"])
    return 0


def cpu_baseline(wl, inp, F, budget_s=10.0, cls=False, heads=None, batch=None):
    """The oracle (fp64 numpy), forward + backward, on this host's cores.

    Work items are (batch entry, head) blocks spread over a fork pool of
    min(available cores, MAX_POOL) workers with one BLAS thread each.  With
    `batch`/`heads` set, only that sample of the workload is computed once;
    otherwise the whole batch is repeated until `budget_s` seconds of wall
    time have passed.  Returns the pairs/s record."""
    import numpy as np

    cores = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
    workers = max(1, min(cores, MAX_POOL))
    B = wl.B if batch is None else batch
    H = wl.H if heads is None else heads
    _POOL_DATA.clear()
    for n in ("q", "k", "v", "do"):
        _POOL_DATA[n] = inp[n][:B, :H].double().numpy()
    _POOL_DATA["F"] = F[:H]
    _POOL_DATA["cls"] = cls
    per_slab = _pairs_per_slab(wl.N, F[:H])
    if cls:
        per_slab = [p + e for p, e in zip(per_slab, _cls_extra_pairs_per_slab(wl.N, F[:H]))]
    pairs = B * int(sum(per_slab))
    # items: one per (batch chunk, head) so that every worker has work
    chunk = max(1, (B * H) // (4 * workers))
    items = []
    for h in range(H):
        for b0 in range(0, B, chunk):
            items.append((b0, min(B, b0 + chunk), h, h + 1))
    ctx = mp.get_context("fork")
    with ctx.Pool(workers, initializer=_pool_init) as pool:
        reps = 0
        t0 = time.perf_counter()
        while True:
            pool.map(_oracle_task, items, chunksize=1)
            reps += 1
            el = time.perf_counter() - t0
            if batch is not None or heads is not None or el >= budget_s or reps >= 100000:
                break
    _POOL_DATA.clear()
    whole = batch is None and heads is None
    sample = (f"whole workload (B={wl.B}, H={wl.H}), forward + backward, {reps} repetitions in "
              f"{el:.1f} s" if whole else
              f"{B} of {wl.B} batch entries x {H} of {wl.H} heads, forward + backward once, "
              f"{el:.1f} s")
    return {
        "value": pairs * reps / el,
        "unit": "pairs/s",
        "cores": workers,
        "kind": "oracle",
        "sample": sample + f"; fp64 numpy, {workers} worker processes with one BLAS thread each "
                           f"({cores} cores available to the process)",
    }


# ---------------------------------------------------------------------------
# GPU timing
# ---------------------------------------------------------------------------

class Hip:
    """hipEvent calls through the HIP runtime (events bound to kernels by
    fibatt_time_next_call are read back here)."""

    def __init__(self):
        self.rt = ctypes.CDLL("libamdhip64.so")
        self.rt.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.rt.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                ctypes.c_void_p]
        self.rt.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def events(self, n):
        out = []
        for _ in range(n):
            e = ctypes.c_void_p()
            if self.rt.hipEventCreate(ctypes.byref(e)) != 0:
                raise RuntimeError("hipEventCreate failed")
            out.append(e.value)
        return out

    def elapsed_ms(self, a, b):
        ms = ctypes.c_float()
        rc = self.rt.hipEventElapsedTime(ctypes.byref(ms), a, b)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return ms.value

    def destroy(self, evs):
        for e in evs:
            self.rt.hipEventDestroy(e)


def kernel_times(hip, body, n):
    """Per-call GPU time (ms) of n back-to-back calls of body(i), each with its
    kernels bracketed by fibatt_time_next_call events; returns the sorted
    list.  The stream is synchronised only once, after the loop."""
    import torch

    import structured_sparse_head_amd as fa

    ev = hip.events(2 * n)
    torch.cuda.synchronize()
    for i in range(n):
        fa.time_next_call(ev[2 * i], ev[2 * i + 1])
        body(i)
    torch.cuda.synchronize()
    t = sorted(hip.elapsed_ms(ev[2 * i], ev[2 * i + 1]) for i in range(n))
    hip.destroy(ev)
    return t


def stats_us(t):
    n = len(t)
    return {"median_us": t[n // 2] * 1e3, "p10_us": t[n // 10] * 1e3,
            "p90_us": t[(9 * n) // 10] * 1e3, "launches": n}


def device_inputs(wl, seed, dev, torch):
    """Seeded synthetic tensors on the GPU with the workload's shapes and
    distribution (i.i.d. N(0, 1); for the high-resolution workload the shared
    rank-8 part of workloads.py): the timed sets of the per-workload block."""
    g = torch.Generator(device=dev)
    g.manual_seed(seed)
    shape = (wl.B, wl.H, wl.N, wl.d)
    dt = wl.torch_dtype
    out = {}
    if wl.values == "lowrank":
        r = 8
        U = torch.randn(wl.B, wl.H, wl.N, r, generator=g, device=dev)
        W = torch.randn(wl.B, wl.H, r, wl.d, generator=g, device=dev)
        L = torch.matmul(U, W) / math.sqrt(r)
        out["q"] = (0.5 * torch.randn(shape, generator=g, device=dev) + L).to(dt)
        out["k"] = (0.5 * torch.randn(shape, generator=g, device=dev) + L).to(dt)
        out["v"] = (0.5 * torch.randn(shape, generator=g, device=dev)).to(dt)
        del U, W, L
    else:
        for n in ("q", "k", "v"):
            out[n] = torch.randn(shape, generator=g, device=dev).to(dt)
    out["do"] = torch.randn(shape, generator=g, device=dev).to(dt)
    return out


def make_sets(wl, op, inputs, R, dev, torch):
    """R buffer sets: inputs (a dict of CPU tensors copied to the device, or
    a function of the set index returning device tensors) and outputs."""
    sets = []
    for i in range(R):
        if callable(inputs):
            s = dict(inputs(i))
        else:
            s = {n: inputs[n].to(dev).clone() for n in ("q", "k", "v", "do")}
        s["o"] = torch.empty_like(s["q"])
        s["lse"] = torch.empty(wl.B, wl.H, wl.N, dtype=torch.float32, device=dev)
        for n in ("dq", "dk", "dv"):
            s[n] = torch.empty(wl.B, wl.H, wl.N, wl.d, dtype=torch.float32, device=dev)
        s["ws"] = torch.empty(op.workspace_floats(), dtype=torch.float32, device=dev)
        s["fws"] = torch.empty(max(op.fwd_workspace_floats(), 1), dtype=torch.float32,
                               device=dev)
        sets.append(s)
    return sets


def rotation(wl):
    """Buffer sets: one rotation holds about 2.4 GB, far beyond the 256 MB
    last-level cache, so no pass reads what an earlier pass left there."""
    esize = 2 if wl.dtype == "bf16" else 4
    per_set = wl.B * wl.H * wl.N * (5 * wl.d * esize + 4 + 3 * wl.d * 4)
    return int(min(8, max(2, math.ceil(2.4e9 / per_set))))


def time_workload(wl, op, sets, hip, n, stream, torch, fa, settle_s=0.05):
    """Per-pass kernel times (median over n launches) and the stream
    reference at the same byte mix, after settle_s seconds of the passes."""
    R = len(sets)
    half = R // 2

    def fwd(i):
        s = sets[i % R]
        op.forward(s["q"], s["k"], s["v"], s["o"], s["lse"], s["fws"], stream=stream)

    def bwd(i):
        s = sets[(i + half) % R]
        op.backward(s["q"], s["k"], s["v"], s["lse"], s["do"], s["dq"], s["dk"], s["dv"],
                    s["ws"], stream=stream)

    for i in range(R):
        fwd(i)
    # After the GPU has idled, its first tens of milliseconds of work run at
    # lower clocks (ViT-B/16: 80-83 us per forward + backward step over the
    # first 25 ms, 73.5 us from then on), so the passes run for at least
    # settle_s before anything is timed.
    t0 = time.perf_counter()
    i = 0
    while True:
        for _ in range(8):
            fwd(i)
            bwd(i)
            i += 1
        torch.cuda.synchronize()
        if time.perf_counter() - t0 >= settle_s:
            break
    tf = kernel_times(hip, fwd, n)
    tb = kernel_times(hip, bwd, n)
    esize = 2 if wl.dtype == "bf16" else 4
    nbytes = wl.B * wl.H * wl.N * wl.d * esize

    def sfwd(i):
        s = sets[i % R]
        fa.hbm_stream([s["q"], s["k"], s["v"]], [s["o"]], nbytes, 1, stream=stream)

    def sbwd(i):
        s = sets[(i + half) % R]
        fa.hbm_stream([s["q"], s["k"], s["v"], s["do"]], [s["dq"], s["dk"], s["dv"]], nbytes,
                      2 if esize == 2 else 1, stream=stream)

    ts_f = kernel_times(hip, sfwd, n)
    ts_b = kernel_times(hip, sbwd, n)
    return tf, tb, ts_f, ts_b


def pass_record(t, nbytes, moved, stream_t, stream_bytes, pairs, tokens):
    st = stats_us(t)
    sec = st["median_us"] * 1e-6
    ssec = stats_us(stream_t)["median_us"] * 1e-6
    rec = dict(st)
    rec.update({
        "bytes": nbytes,
        "gbps": nbytes / sec / 1e9,
        "hbm_frac": nbytes / sec / 1e9 / HBM_PEAK_GBPS,
        "pairs_per_s": pairs / sec,
        "tokens_per_s": tokens / sec,
        "stream_ref_us": ssec * 1e6,
        "stream_ref_gbps": stream_bytes / ssec / 1e9,
        # bandwidth of the bytes the kernels move, over the stream kernel's
        # bandwidth at the same read/write mix
        "frac_of_stream_ref": (moved / sec) / (stream_bytes / ssec),
    })
    if moved != nbytes:
        rec["bytes_moved"] = moved
        rec["gbps_moved"] = moved / sec / 1e9
    return rec


# ---------------------------------------------------------------------------
# One attention layer (projections + sparse core)
# ---------------------------------------------------------------------------

def bench_block(args):
    """One ViT-B/16 attention layer with Fibottention heads (README Algorithm 3):
    QKV projection, sparse core, output projection, forward + backward through
    autograd, B=64, N=197, c=768, h=12, bf16."""
    import numpy as np
    import torch

    import structured_sparse_head_amd as fa

    B, N, C, H = 64, 197, 768, 12
    dev = torch.device("cuda:0")
    dt = torch.bfloat16
    layer = fa.FibottentionAttention(C, H, N, modified=args.modified, cls=args.cls, device=dev,
                                     dtype=dt)
    layer.reset_parameters(torch.Generator().manual_seed(0))
    rng = np.random.default_rng(2)
    R = max(2, args.sets or 6)
    xs = [torch.from_numpy(rng.standard_normal((B, N, C), dtype=np.float32)).to(dev, dt)
          .requires_grad_() for _ in range(R)]
    gs = [torch.from_numpy(rng.standard_normal((B, N, C), dtype=np.float32)).to(dev, dt)
          for _ in range(R)]

    def step(i):
        layer(xs[i % R]).backward(gs[i % R])

    def timed(body, n):
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        start.record()
        for i in range(n):
            body(i)
        end.record()
        torch.cuda.synchronize()
        return start.elapsed_time(end) / n

    t0 = time.perf_counter()  # the GPU's clocks settle first (see time_workload)
    i = 0
    while time.perf_counter() - t0 < 0.05:
        for _ in range(4):
            step(i)
            i += 1
        torch.cuda.synchronize()
    for i in range(args.warmup):
        step(i)
    K = args.steps
    ms_step = timed(step, K)
    with torch.no_grad():
        ms_fwd = timed(lambda i: layer(xs[i % R]), K)
        x2 = [x.detach().reshape(B * N, C) for x in xs]
        ms_qkv = timed(lambda i: torch.mm(x2[i % R], layer.w_qkv), K)
        ms_out = timed(lambda i: torch.mm(x2[i % R], layer.w_z), K)
        heads = [[t[:, :, j].permute(0, 2, 1, 3) for j in range(3)]
                 for t in (torch.mm(x, layer.w_qkv).view(B, N, 3, H, C // H) for x in x2[:2])]
        o = torch.empty(B, N, H, C // H, dtype=dt, device=dev).permute(0, 2, 1, 3)
        op = fa.Fibottention(B, H, N, C // H, dt, layer.a, layer.b, layer.w, cls=args.cls)
        ms_core = timed(lambda i: op.forward(*heads[i % 2], o=o), K)
    gemm_fwd_flops = 2 * B * N * C * 3 * C + 2 * B * N * C * C
    gemm_tflops = gemm_fwd_flops / ((ms_qkv + ms_out) * 1e-3) / 1e12
    line = {
        "metric": "tokens/s through one ViT-B/16 Fibottention attention layer (fwd+bwd), 1 GPU",
        "value": B * N / (ms_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "Fibottention ViT-B/16 attention layer (QKV and output projections, "
                        "sparse core), B=64 N=197 c=768 h=12",
            "heads": "modified Wythoff pairs, rows 1..H" if args.modified else "Wythoff rows 1..H",
            "mask": "class-token row and column dense" if args.cls else "Fibonacci support only",
            "buffer_sets": R,
        },
        "forward_us": {"layer": ms_fwd * 1e3, "qkv_projection": ms_qkv * 1e3,
                       "sparse_core": ms_core * 1e3, "output_projection": ms_out * 1e3},
        "roofline": {
            "kernel": "forward projection GEMMs (torch.mm, bf16)",
            "bound": "mfma",
            "achieved": gemm_tflops,
            "peak": 2500.0,
            "unit": "TFLOP/s",
            "frac": gemm_tflops / 2500.0,
            "traffic": None,
        },
    }
    print(json.dumps(line), flush=True)


# ---------------------------------------------------------------------------
# Main
# ---------------------------------------------------------------------------

def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", type=int, default=2)
    ap.add_argument("--sets", type=int, default=0, help="rotated buffer sets (default: enough "
                    "to exceed the last-level cache)")
    ap.add_argument("--workloads", default="1,2,3,4,5",
                    help="workloads of the per-workload block ('' for none)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--modified", action="store_true",
                    help="heads from README Algorithm 2's modified Wythoff pairs")
    ap.add_argument("--cls", action="store_true",
                    help="class-token mask (README Algorithm 2: row and column 0 dense)")
    ap.add_argument("--block", action="store_true",
                    help="time one ViT-B/16 attention layer (projections + sparse core) instead")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="only run a stream copy (fibatt_hbm_stream, one array read, one "
                         "written) of this many MiB, 10 times (scale reference for HBM byte "
                         "counters), then exit")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the op shards over (batch, head) slabs with no communication)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import workloads
    import structured_sparse_head_amd as fa

    if args.copy_mib:
        n = args.copy_mib * (1 << 20)
        src = torch.ones(n // 4, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(10):
            fa.hbm_stream([src], [dst], n, 1)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_each_way": n, "launches": 10}), flush=True)
        return
    if args.block:
        bench_block(args)
        return

    wl = workloads.WORKLOADS[args.workload]
    a, b = fa.wythoff_rows(wl.H, modified=args.modified)
    w = workloads.windows(wl)
    ptr, offs = fa.offsets(wl.N, a, b, w)
    F = [[int(f) for f in offs[ptr[h]:ptr[h + 1]]] for h in range(wl.H)]
    pairs = int(wl.B * sum(_pairs_per_slab(wl.N, F)))
    if args.cls:
        pairs += int(wl.B * sum(_cls_extra_pairs_per_slab(wl.N, F)))
    esize = 2 if wl.dtype == "bf16" else 4
    fwd_bytes, bwd_bytes, bwd_moved = pass_bytes(wl, esize)
    inp = workloads.make_inputs(wl)

    # CPU oracle first: the worker processes fork before the GPU is touched.
    cpu = None
    cpu_samples = {}
    others = [int(x) for x in args.workloads.split(",") if x.strip()]
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(wl, inp, F, cls=args.cls)
        for num in others:
            if num == args.workload or args.cls or args.modified:
                continue
            owl = workloads.WORKLOADS[num]
            sample_b = 1 if num >= 3 else None
            sample_h = 4 if num == 5 else None
            oinp = workloads.make_inputs(owl, B=sample_b or owl.B, H=sample_h or owl.H)
            oa, ob = fa.wythoff_rows(owl.H)
            optr, ooffs = fa.offsets(owl.N, oa, ob, workloads.windows(owl))
            oF = [[int(f) for f in ooffs[optr[h]:optr[h + 1]]] for h in range(owl.H)]
            cpu_samples[num] = cpu_baseline(owl, oinp, oF, batch=sample_b or owl.B,
                                            heads=sample_h or owl.H)
            del oinp

    dev = torch.device("cuda:0")
    hip = Hip()
    op = fa.Fibottention(wl.B, wl.H, wl.N, wl.d, wl.torch_dtype, a, b, w, cls=args.cls)
    R = args.sets or rotation(wl)
    sets = make_sets(wl, op, inp, R, dev, torch)
    stream = torch.cuda.current_stream(dev).cuda_stream
    half = R // 2

    def fwd(i):
        s = sets[i % R]
        op.forward(s["q"], s["k"], s["v"], s["o"], s["lse"], s["fws"], stream=stream)

    def bwd(i):
        s = sets[(i + half) % R]
        op.backward(s["q"], s["k"], s["v"], s["lse"], s["do"], s["dq"], s["dk"], s["dv"],
                    s["ws"], stream=stream)

    for i in range(R):  # every set gets a forward before any backward reads its LSE
        fwd(i)

    # Per pass: kernel-only times over max(K, 100) launches, and the stream
    # reference at the same byte mix.  They run before the headline loop, so
    # that the warmup and timed steps find the GPU at its steady clocks (see
    # time_workload).
    K = args.steps
    n = max(K, 100)
    tf, tb, ts_f, ts_b = time_workload(wl, op, sets, hip, n, stream, torch, fa)

    for i in range(args.warmup):
        fwd(i)
        bwd(i)
    torch.cuda.synchronize()

    # Headline: K whole steps back to back, events around the loop.
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    start.record()
    for i in range(K):
        fwd(i)
        bwd(i)
    end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = start.elapsed_time(end) / K

    tokens = wl.B * wl.N
    nb = wl.B * wl.H * wl.N * wl.d * esize
    stream_fwd_bytes = 4 * nb
    stream_bwd_bytes = 4 * nb + 3 * nb * (2 if esize == 2 else 1)
    kernels = {
        "fwd": pass_record(tf, fwd_bytes, fwd_bytes, ts_f, stream_fwd_bytes, pairs, tokens),
        "bwd": pass_record(tb, bwd_bytes, bwd_moved, ts_b, stream_bwd_bytes, pairs, tokens),
    }
    kernels["fwd"]["kernels"] = KERNELS[wl.number]["fwd"]
    kernels["bwd"]["kernels"] = KERNELS[wl.number]["bwd"]
    dom = "bwd" if kernels["bwd"]["median_us"] >= kernels["fwd"]["median_us"] else "fwd"
    kd = kernels[dom]
    ach = kd["gbps"]
    traffic = None if (args.cls or args.modified) else measured_traffic(wl.number, dom)
    step_s = ms_step * 1e-3
    name = f"{wl.name}"
    line = {
        "metric": f"sparse Q.K pairs/s (fwd+bwd), {name}, 1 GPU",
        "value": pairs / step_s,
        "unit": "pairs/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic",
        "config": {
            "workload": f"Fibottention attention, {name}"
                        + (" (ViT-B/16 224px tokens)" if wl.number == 2 else ""),
            "B": wl.B, "H": wl.H, "N": wl.N, "d_h": wl.d,
            "heads": "modified Wythoff pairs, rows 1..H" if args.modified else "Wythoff rows 1..H",
            "mask": "class-token row and column dense" if args.cls else "Fibonacci support only",
            "pairs_per_pass": pairs,
            "buffer_sets": R,
        },
        "tokens_per_s": tokens / step_s,
        "hbm_gbps_fwd_bwd": (fwd_bytes + bwd_bytes) / step_s / 1e9,
        "wall_s_timed": wall,
        "kernels": kernels,
        "roofline": {
            "kernel": f"{' + '.join(KERNELS[wl.number][dom])} ({dom} pass)"
                      + (" with the class-token kernels" if args.cls else ""),
            "bound": "hbm",
            "achieved": ach,
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": ach / HBM_PEAK_GBPS,
            "traffic": traffic,
            "bytes_per_launch": kd["bytes"],
            "launch_us_median": kd["median_us"],
            "stream_ref_gbps": kd["stream_ref_gbps"],
            "frac_of_stream_ref": kd["frac_of_stream_ref"],
        },
        "pages_context": pages_context(wl, pairs),
    }
    if dom == "bwd":
        line["roofline"]["achieved_moved_bytes"] = kd["gbps_moved"]
        line["roofline"]["note"] = ("achieved counts the scope table's backward bytes (O read); "
                                    "this backward computes D itself and moves bytes_moved")

    # Per-workload block: kernel-only medians for every workload.
    block = {}
    fabric_gbps = fabric_ref(hip, torch, fa, dev) if others else None
    for num in others:
        owl = workloads.WORKLOADS[num]
        if num == wl.number and not (args.cls or args.modified):
            otf, otb, ots_f, ots_b, opairs, oop = tf, tb, ts_f, ts_b, pairs, op
        else:
            oa, ob = fa.wythoff_rows(owl.H)
            ow = workloads.windows(owl)
            optr, ooffs = fa.offsets(owl.N, oa, ob, ow)
            oF = [[int(f) for f in ooffs[optr[h]:optr[h + 1]]] for h in range(owl.H)]
            opairs = int(owl.B * sum(_pairs_per_slab(owl.N, oF)))
            oop = fa.Fibottention(owl.B, owl.H, owl.N, owl.d, owl.torch_dtype, oa, ob, ow)
            OR = rotation(owl)
            osets = make_sets(owl, oop, lambda i, owl=owl: device_inputs(owl, 100 + i, dev, torch),
                              OR, dev, torch)
            otf, otb, ots_f, ots_b = time_workload(owl, oop, osets, hip, 100, stream, torch, fa)
            del osets
            torch.cuda.empty_cache()
        oes = 2 if owl.dtype == "bf16" else 4
        of, obb, obm = pass_bytes(owl, oes)
        onb = owl.B * owl.H * owl.N * owl.d * oes
        rf = pass_record(otf, of, of, ots_f, 4 * onb, opairs, owl.B * owl.N)
        rb = pass_record(otb, obb, obm, ots_b, 4 * onb + 3 * onb * (2 if oes == 2 else 1), opairs,
                         owl.B * owl.N)
        t_sum = (rf["median_us"] + rb["median_us"]) * 1e-6
        entry = {
            "config": owl.name,
            "pairs_per_pass": opairs,
            "fwd_us": {k: rf[k] for k in ("median_us", "p10_us", "p90_us")},
            "bwd_us": {k: rb[k] for k in ("median_us", "p10_us", "p90_us")},
            "pairs_per_s_fwd_bwd": opairs / t_sum,
            "tokens_per_s_fwd_bwd": owl.B * owl.N / t_sum,
            "fwd_hbm_frac": rf["hbm_frac"],
            "bwd_hbm_frac": rb["hbm_frac"],
            "fwd_frac_of_stream_ref": rf["frac_of_stream_ref"],
            "bwd_frac_of_stream_ref": rb["frac_of_stream_ref"],
            "fwd_traffic": measured_traffic(num, "fwd"),
            "bwd_traffic": measured_traffic(num, "bwd"),
        }
        # Algorithmic flops (4 d_h per pair forward, 10 d_h backward) per
        # second, over the vector-ALU peak: the other bound at long sequences.
        for pname, rec in (("fwd", rf), ("bwd", rb)):
            tf_s = FLOPS_PER_PAIR_ELEM[pname] * owl.d * opairs / (rec["median_us"] * 1e-6) / 1e12
            entry[f"{pname}_tflops"] = tf_s
            entry[f"{pname}_valu_frac"] = tf_s / VALU_PEAK_TFLOPS
        # L2-miss reads (FETCH_SIZE from the committed counters, current
        # sources only) per second, over the rate the L2s can be filled.
        for pname, rec in (("fwd", rf), ("bwd", rb)):
            fetch = measured_fetch(num, pname)
            if fetch is not None and fabric_gbps:
                gbps = fetch / (rec["median_us"] * 1e-6) / 1e9
                entry[f"{pname}_l2_fill_gbps"] = gbps
                entry[f"{pname}_frac_of_l2_fill_ref"] = gbps / fabric_gbps
        if num in cpu_samples:
            entry["cpu_oracle"] = cpu_samples[num]
        elif num == wl.number and cpu is not None:
            entry["cpu_oracle"] = cpu
        block[str(num)] = entry
    if block:
        line["workloads"] = block
        line["l2_fill_ref_gbps"] = fabric_gbps
    if cpu is not None:
        line["cpu_baseline"] = cpu
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
