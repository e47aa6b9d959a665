"""Benchmark: Fibottention sparse attention forward + backward on one MI355X.

One step = one forward and one backward pass over one batch of the ViT-B/16
attention workload (B=64, H=12, N=197, d_h=64, bf16 inputs, fp32
accumulation), with inputs resident in HBM.  Several buffer sets are rotated
so that each pass reads data that is not left in the 256 MB last-level
cache by the pass before it (the backward of a step works on a set whose
forward ran half a rotation earlier, as in a network with other layers in
between).

Prints one JSON line.  `value` is Q.K pairs per second over forward +
backward; the line also carries tokens/s, the achieved algorithmic HBM
bandwidth, per-kernel timings, a roofline entry for the dominant kernel and
the CPU oracle timed on this host.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 2]
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time


ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E, published


def _pairs_per_slab(N, F):
    return [int(sum(2 * (N - int(f)) if f > 0 else N for f in fs)) for fs in F]


def _bytes(wl, esize):
    """Algorithmic HBM bytes per pass (whole batch).

    forward : read Q, K, V (input dtype); write O (input dtype), LSE (fp32).
    backward: read Q, K, V, dO (input dtype), LSE (fp32); write dQ, dK, dV (fp32).
    """
    rows = wl.B * wl.H * wl.N
    row = wl.d * esize
    fwd = rows * (4 * row + 4)
    bwd = rows * (4 * row + 4 + 3 * wl.d * 4)
    return int(fwd), int(bwd)


# Dominant kernel on this workload for each pass, and the source files whose
# hash identifies the build its HBM counters were taken on.
KERNELS = {
    "fwd": ("fwd_slab_bf16_kernel", ["fwd_slab_bf16.hip", "slab_bf16_common.h"]),
    "bwd": ("bwd_slab_bf16_kernel", ["bwd_slab_bf16.hip", "slab_bf16_common.h"]),
}


def _source_hash(files):
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "structured_sparse_head_amd", "csrc")
    for f in files + ["kernel_common.h", "fib_offsets.h"]:
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(pass_name):
    """HBM bytes per dispatch (read + write) of the pass's kernel from the
    committed counter summary, or None when the kernel source has changed
    since the counters were taken."""
    name, files = KERNELS[pass_name]
    path = os.path.join(ROOT, "profiles", "hbm_traffic.txt")
    if not os.path.exists(path):
        return None
    want = _source_hash(files)
    with open(path) as fh:
        for line in fh:
            f = line.split()
            if len(f) == 4 and f[0] == name and f[1] == want:
                return int(f[2]) + int(f[3])
    return None


def _cls_extra_pairs_per_slab(N, F):
    """Pairs the class-token mask adds to each head's support: (0, k) and
    (k, 0) for every k >= 1 that is not a distance, and (0, 0) when 0 is not
    a distance."""
    out = []
    for fs in F:
        pos = len([f for f in fs if f >= 1])
        out.append(2 * (N - 1 - pos) + (0 if 0 in fs else 1))
    return out


def cpu_baseline(wl, inp, F, pairs_per_pass, budget_s=10.0, cls=False):
    """The oracle (fp64 numpy), forward + backward over the whole batch,
    repeated until `budget_s` seconds of CPU time have passed."""
    import oracle  # test infrastructure; used only for this baseline leg

    try:
        from threadpoolctl import threadpool_limits
        limiter = threadpool_limits(1)
    except Exception:  # pragma: no cover
        limiter = None
    x = {n: inp[n].double().numpy() for n in ("q", "k", "v", "do")}
    reps = 0
    t0 = time.perf_counter()
    while True:
        oracle.forward(x["q"], x["k"], x["v"], F, cls=cls)
        oracle.backward(x["q"], x["k"], x["v"], x["do"], F, cls=cls)
        reps += 1
        el = time.perf_counter() - t0
        if el >= budget_s or reps >= 50:
            break
    if limiter is not None:
        limiter.unregister()
    return {
        "value": pairs_per_pass * reps / el,
        "unit": "pairs/s",
        "cores": 1,
        "kind": "oracle",
        "sample": f"whole workload (B={wl.B}), forward + backward, {reps} repetitions in "
                  f"{el:.1f} s, fp64 numpy, one thread",
    }


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
    R = max(2, args.sets)
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

    for i in range(args.warmup):
        step(i)
    K = args.steps
    ms_step = timed(step, K)
    with torch.no_grad():
        ms_fwd = timed(lambda i: layer(xs[i % R]), K)
        x2 = [x.detach().reshape(B * N, C) for x in xs]
        ms_qkv = timed(lambda i: torch.mm(x2[i % R], layer.w_qkv), K)
        ms_out = timed(lambda i: torch.mm(x2[i % R], layer.w_z), K)
        # the sparse core as the layer runs it: strided head views of the
        # fused projection in, O written in [B, N, H, d_h] order
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


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", type=int, default=2)
    ap.add_argument("--sets", type=int, default=6, help="rotated buffer sets")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--modified", action="store_true",
                    help="heads from README Algorithm 2's modified Wythoff pairs")
    ap.add_argument("--cls", action="store_true",
                    help="class-token mask (README Algorithm 2: row and column 0 dense)")
    ap.add_argument("--block", action="store_true",
                    help="time one ViT-B/16 attention layer (projections + sparse core) instead")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="only run a device-to-device copy of this many MiB, 10 times "
                         "(scale reference for HBM byte counters), then exit")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the op shards over (batch, head) slabs with no communication)", file=sys.stderr)
        sys.exit(2)

    import torch

    if args.copy_mib:
        n = args.copy_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(10):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_each_way": n * 4, "launches": 10}), flush=True)
        return

    if args.block:
        bench_block(args)
        return

    import workloads
    import structured_sparse_head_amd as fa

    wl = workloads.WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    a, b = fa.wythoff_rows(wl.H, modified=args.modified)
    w = workloads.windows(wl)
    ptr, offs = fa.offsets(wl.N, a, b, w)
    F = [[int(f) for f in offs[ptr[h]:ptr[h + 1]]] for h in range(wl.H)]
    pairs_per_pass = int(wl.B * sum(_pairs_per_slab(wl.N, F)))
    if args.cls:
        pairs_per_pass += int(wl.B * sum(_cls_extra_pairs_per_slab(wl.N, F)))
    esize = 2 if wl.dtype == "bf16" else 4
    fwd_bytes, bwd_bytes = _bytes(wl, esize)

    inp = workloads.make_inputs(wl)
    op = fa.Fibottention(wl.B, wl.H, wl.N, wl.d, wl.torch_dtype, a, b, w, cls=args.cls)
    R = max(2, args.sets)
    sets = []
    for _ in range(R):
        s = {n: inp[n].to(dev).clone() for n in ("q", "k", "v", "do")}
        s["o"] = torch.empty_like(s["q"])
        s["lse"] = torch.empty(wl.B, wl.H, wl.N, dtype=torch.float32, device=dev)
        for n in ("dq", "dk", "dv"):
            s[n] = torch.empty(wl.B, wl.H, wl.N, wl.d, dtype=torch.float32, device=dev)
        s["ws"] = torch.empty(op.workspace_floats(), dtype=torch.float32, device=dev)
        s["fws"] = torch.empty(max(op.fwd_workspace_floats(), 1), dtype=torch.float32,
                               device=dev)
        sets.append(s)
    stream = torch.cuda.current_stream(dev).cuda_stream

    def fwd(s):
        op.forward(s["q"], s["k"], s["v"], s["o"], s["lse"], s["fws"], stream=stream)

    def bwd(s):
        op.backward(s["q"], s["k"], s["v"], s["lse"], s["do"], s["dq"], s["dk"], s["dv"],
                    s["ws"], stream=stream)

    for s in sets:  # every set gets a forward before any backward reads its LSE
        fwd(s)
    half = R // 2
    for i in range(args.warmup):
        fwd(sets[i % R])
        bwd(sets[(i + half) % R])
    torch.cuda.synchronize()

    K = args.steps

    def timed(body, n):
        """Average ms per iteration of `body(i)` over n back-to-back iterations,
        bracketed by events on the launch stream (no events inside the loop)."""
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        start.record()
        for i in range(n):
            body(i)
        end.record()
        torch.cuda.synchronize()
        return start.elapsed_time(end) / n

    # Headline: K whole steps (forward of one set, backward of another).
    t0 = time.perf_counter()
    ms_step = timed(lambda i: (fwd(sets[i % R]), bwd(sets[(i + half) % R])), K)
    wall = time.perf_counter() - t0
    # Per-kernel averages: each pass alone, back to back, over the same rotation.
    fwd_ms = timed(lambda i: fwd(sets[i % R]), K)
    bwd_ms = timed(lambda i: bwd(sets[(i + half) % R]), K)

    kernels = {
        "fwd": {"mean_us": fwd_ms * 1e3, "bytes": fwd_bytes,
                "gbps": fwd_bytes / (fwd_ms * 1e-3) / 1e9},
        "bwd": {"mean_us": bwd_ms * 1e3, "bytes": bwd_bytes,
                "gbps": bwd_bytes / (bwd_ms * 1e-3) / 1e9},
    }
    for kv in kernels.values():  # fraction of the 8 TB/s HBM peak, per pass
        kv["hbm_frac"] = kv["gbps"] / HBM_PEAK_GBPS
    dom = "bwd" if bwd_ms >= fwd_ms else "fwd"
    ach = kernels[dom]["gbps"]
    step_s = ms_step * 1e-3
    line = {
        "metric": "sparse Q.K pairs/s (fwd+bwd), ViT-B/16 N=197 H=12, 1 GPU",
        "value": pairs_per_pass / step_s,
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
            "workload": f"Fibottention attention, {wl.name} (ViT-B/16 224px tokens)"
            if args.workload == 2 else f"Fibottention attention, {wl.name}",
            "B": wl.B, "H": wl.H, "N": wl.N, "d_h": wl.d,
            "heads": "modified Wythoff pairs, rows 1..H" if args.modified else "Wythoff rows 1..H",
            "mask": "class-token row and column dense" if args.cls else "Fibonacci support only",
            "pairs_per_pass": pairs_per_pass,
            "buffer_sets": R,
        },
        "tokens_per_s": wl.B * wl.N / step_s,
        "hbm_gbps_fwd_bwd": (fwd_bytes + bwd_bytes) / step_s / 1e9,
        "wall_s_timed": wall,
        "kernels": kernels,
        "roofline": {
            "kernel": f"all launches of the {dom} pass (class-token mask)" if args.cls
            else f"{KERNELS[dom][0]} ({dom} pass)",
            "bound": "hbm",
            "achieved": ach,
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": ach / HBM_PEAK_GBPS,
            "traffic": None if args.cls else measured_traffic(dom),
        },
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(wl, inp, F, pairs_per_pass, cls=args.cls)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
