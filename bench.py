#!/usr/bin/env python3
"""Attention-forward throughput on one MI355X, as one JSON line on stdout.

A step is one call of the HIP attention forward over the whole workload (one
launch of the fused kernel: Q.K^T, masks, online softmax, P.V, normalisation and
LSE). Inputs and outputs are resident in device memory before timing starts.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]
    python bench.py --backward [--workload NAME] ...   (the backward pass instead: fa_bwd)

FLOPs are algorithmic: 4*D per unmasked (query, key) pair, so the causal
triangle and padded keys are counted once and only where they are computed by
the definition. The roofline figure divides those FLOPs by the kernel's own
average duration, measured with events recorded on the launch stream around
every timed launch.

With --backward a step is one fa_bwd call (its two kernels) on the same workload,
with O and LSE from one forward and a seeded dO. Its algorithmic FLOPs are the
five products of 2*D per unmasked pair (S rebuilt, dP, dV, dK, dQ), 10*D per pair;
the kernels execute seven (S and dP are formed in both), reported beside it.
"""

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "attn fwd TFLOP/s and % bf16 MFMA peak, B2 H32 N8192 D128 bf16"
METRIC_BWD = "attn bwd TFLOP/s (5 products of 2D flops per pair) and % bf16 MFMA peak"
# MI355X published dense matrix peaks, TFLOP/s, and HBM3E bandwidth, GB/s.
PEAK_TFLOPS = {"bf16": 2500.0, "f16": 2500.0, "f32": 157.3}
PEAK_HBM_GBS = 8000.0
# Every source file the library is compiled from (a counter record is current only for them).
KERNEL_SOURCES = sorted(os.path.join("exact_tiled_attention_23_amd", "csrc", f)
                        for f in os.listdir(os.path.join(ROOT, "exact_tiled_attention_23_amd", "csrc"))
                        if f.endswith((".h", ".hip")))
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def pair_count(w, kv_len):
    """Unmasked (query, key) pairs of the whole workload."""
    import numpy as np
    total = 0
    i = np.arange(w.N, dtype=np.int64)
    for b in range(w.B):
        L = w.N if kv_len is None else int(kv_len[b])
        cnt = np.minimum(L, i + 1) if w.causal else np.full(w.N, L, dtype=np.int64)
        total += int(cnt.sum()) * w.H
    return total


def algorithmic_bytes(w, kv_len, elt):
    """Q and O once, K and V rows that some query may see once, LSE once."""
    rows_kv = w.B * w.N if kv_len is None else int(sum(int(x) for x in kv_len))
    return elt * w.D * (2 * w.B * w.N + 2 * rows_kv) * w.H + 4 * w.B * w.H * w.N


def kernel_source_hash():
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(workload):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it is still current."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f).get(workload)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("kernel_source_hash") != kernel_source_hash():
        return None
    return rec.get("hbm_bytes_per_launch")


def blas_info():
    """The NumPy build's BLAS library and the BLAS thread pools, for the CPU baseline record."""
    import numpy as np
    try:
        name = np.__config__.CONFIG["Build Dependencies"]["blas"]["name"]
    except (AttributeError, KeyError, TypeError):
        name = "unknown"
    try:
        from threadpoolctl import threadpool_info
        pools = sorted({f"{p['internal_api']}:{p['num_threads']}" for p in threadpool_info()})
    except ImportError:
        pools = []
    return {"numpy": np.__version__, "blas": name, "blas_pools": pools}


def cpu_baseline(x, w, heads):
    """The float64 oracle on the first `heads` (batch, head) pairs of the same inputs, all rows."""
    import numpy as np
    import oracle
    from exact_tiled_attention_23_amd.workloads import to_f64
    cores = max(1, min(16, len(os.sched_getaffinity(0))))
    heads = min(heads, w.B * w.H)
    sel = [divmod(i, w.H) for i in range(heads)]
    q = np.stack([to_f64(x.q[b, h]) for b, h in sel])[None]
    k = np.stack([to_f64(x.k[b, h]) for b, h in sel])[None]
    v = np.stack([to_f64(x.v[b, h]) for b, h in sel])[None]
    pairs = 0
    i = np.arange(w.N, dtype=np.int64)
    for b, _ in sel:
        L = w.N if x.kv_len is None else int(x.kv_len[b])
        pairs += int((np.minimum(L, i + 1) if w.causal else np.full(w.N, L)).sum())
    t0 = time.perf_counter()
    if x.kv_len is None:
        oracle.attention(q, k, v, x.scale, causal=w.causal, workers=cores)
    else:
        # one (b, h) per call so each keeps its batch's kv_len
        from concurrent.futures import ThreadPoolExecutor
        from threadpoolctl import threadpool_limits
        def one(j):
            b = sel[j][0]
            oracle.attention(q[:, j:j + 1], k[:, j:j + 1], v[:, j:j + 1], x.scale, causal=w.causal,
                             kv_len=x.kv_len[b:b + 1])
        with threadpool_limits(limits=1), ThreadPoolExecutor(max_workers=cores) as ex:
            list(ex.map(one, range(len(sel))))
    dt = time.perf_counter() - t0
    flops = 4.0 * w.D * pairs
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": f"{heads} of {w.B * w.H} (batch, head) pairs, all {w.N} query rows, float64",
            "seconds": round(dt, 3), "workers": cores, "affinity_cpus": len(os.sched_getaffinity(0)),
            "gflops_fp64": round(flops / dt / 1e9, 1), **blas_info()}


def cpu_baseline_backward(x, do, w, heads):
    """The float64 gradient oracle on the first `heads` (batch, head) pairs, all rows."""
    import numpy as np
    import oracle
    from exact_tiled_attention_23_amd.workloads import to_f64
    from threadpoolctl import threadpool_limits
    cores = max(1, min(16, len(os.sched_getaffinity(0))))
    heads = min(heads, w.B * w.H)
    pairs = 0
    i = np.arange(w.N, dtype=np.int64)
    t0 = time.perf_counter()
    with threadpool_limits(limits=cores):
        for j in range(heads):
            b, h = divmod(j, w.H)
            L = w.N if x.kv_len is None else int(x.kv_len[b])
            pairs += int((np.minimum(L, i + 1) if w.causal else np.full(w.N, L)).sum())
            oracle.attention_grad(to_f64(x.q[b:b + 1, h:h + 1]), to_f64(x.k[b:b + 1, h:h + 1]),
                                  to_f64(x.v[b:b + 1, h:h + 1]), to_f64(do[b:b + 1, h:h + 1]), x.scale,
                                  causal=w.causal, kv_len=None if x.kv_len is None else x.kv_len[b:b + 1])
    dt = time.perf_counter() - t0
    return {"value": 10.0 * w.D * pairs / dt / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": f"{heads} of {w.B * w.H} (batch, head) pairs, all {w.N} query rows, float64",
            "seconds": round(dt, 3), "affinity_cpus": len(os.sched_getaffinity(0)), **blas_info()}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-heads", type=int, default=64,
                    help="(batch, head) pairs the CPU oracle baseline runs; all of the headline workload by default")
    ap.add_argument("--backward", action="store_true", help="time the backward (fa_bwd) instead of the forward")
    ap.add_argument("--shape", default=None,
                    help="B,H,N,D,dtype,causal[,padded][,rowscale]: a seeded synthetic workload of this shape "
                         "instead of a named one (the recipe of the named workloads, seed 7); 'padded' draws a "
                         "kv_len per batch element, 'rowscale' scales each query row by a factor in [1, 100]")
    ap.add_argument("--cold-bytes", type=int, default=0,
                    help="write this many bytes of scratch memory between timed launches (e.g. 1 GiB, beyond the "
                         "256 MB MALL) so each launch finds its inputs outside the caches; value is then the "
                         "kernel-timed rate")
    ap.add_argument("--gemm", type=int, default=0,
                    help="instead of attention, time a bf16 N x N x N matrix product through torch (the vendor "
                         "GEMM library): the matrix cores' practical throughput under the same power and clock")
    ap.add_argument("--copy-bytes", type=int, default=0,
                    help="instead of attention, run a plain device copy of this many bytes per step "
                         "(scale reference for the HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(every (batch, head) is independent, so more GPUs would each run this kernel on their share)",
              file=sys.stderr)
        sys.exit(2)
    if int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py runs as a single process on one GPU", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import exact_tiled_attention_23_amd as fa
    from exact_tiled_attention_23_amd.workloads import (HEADLINE, WORKLOADS, Workload, generate_grad_output,
                                                        generate_workload)

    if args.gemm:
        n = args.gemm
        a = torch.randn(n, n, dtype=torch.bfloat16, device="cuda:0")
        bm = torch.randn(n, n, dtype=torch.bfloat16, device="cuda:0")
        c = torch.empty(n, n, dtype=torch.bfloat16, device="cuda:0")
        for _ in range(args.warmup):
            torch.matmul(a, bm, out=c)
        torch.cuda.synchronize()
        ms = []
        for _ in range(args.steps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            torch.matmul(a, bm, out=c)
            e1.record()
            torch.cuda.synchronize()
            ms.append(e0.elapsed_time(e1))
        flops = 2.0 * n ** 3
        print(json.dumps({"calibration": "bf16 GEMM", "n": n, "steps": args.steps,
                          "tflops_median": round(flops / float(np.median(ms)) / 1e9, 1),
                          "tflops_best": round(flops / min(ms) / 1e9, 1),
                          "ms_median": round(float(np.median(ms)), 4)}))
        return

    if args.copy_bytes:
        src = torch.empty(args.copy_bytes // 4, dtype=torch.float32, device="cuda:0").uniform_()
        dst = torch.empty_like(src)
        for _ in range(args.warmup + args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibration": "device copy", "bytes_read_per_step": src.numel() * 4,
                          "bytes_written_per_step": src.numel() * 4, "steps": args.warmup + args.steps}))
        return

    if args.shape:
        fields = [f.strip().lower() for f in args.shape.split(",")]
        B, H, N, D, dt, causal = fields[:6]
        causal = causal in ("1", "true", "causal")
        padded, rowscale = "padded" in fields[6:], "rowscale" in fields[6:]
        name = (f"b{B}h{H}n{N}d{D}-{dt}" + ("-causal" if causal else "") + ("-padded" if padded else "")
                + ("-rowscale" if rowscale else ""))
        w = Workload(name, int(B), int(H), int(N), int(D), dt, causal, padding=padded, q_row_scale=rowscale, seed=7)
    else:
        name = args.workload or HEADLINE
        w = WORKLOADS[name]
    dev = torch.device("cuda:0")
    log(f"bench: generating {name}")
    x = generate_workload(w)
    q, k, v = (t.to(dev) for t in (x.q, x.k, x.v))
    kv = None if x.kv_len is None else torch.as_tensor(x.kv_len, dtype=torch.int32).to(dev)
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    if args.backward:
        if w.dtype == "f32":
            print("the backward is built for bf16 and f16", file=sys.stderr)
            sys.exit(2)
        do_cpu = generate_grad_output(w.B, w.H, w.N, w.D, w.dtype, seed=w.seed + 1000)
        do = do_cpu.to(dev)
        fa.forward(q, k, v, causal=w.causal, scale=x.scale, kv_len=kv, out=o, lse=lse, stream=stream)
        dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
        ws = torch.empty(fa.fa_bwd_workspace_bytes(w.B, w.H, w.N, w.D), dtype=torch.uint8, device=dev)

        def step():
            fa.backward(q, k, v, o, lse, do, causal=w.causal, scale=x.scale, kv_len=kv, dq=dq, dk=dk, dv=dv,
                        workspace=ws, stream=stream)
    else:
        def step():
            fa.forward(q, k, v, causal=w.causal, scale=x.scale, kv_len=kv, out=o, lse=lse, stream=stream)

    log(f"bench: warmup {args.warmup}")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"bench: timing {args.steps} steps")
    scratch = torch.empty(args.cold_bytes // 4, dtype=torch.float32, device=dev) if args.cold_bytes else None
    if scratch is None:
        # The timed steps run back to back; one event pair on the launch stream around all of
        # them gives the kernels' average duration (the attention kernels are the only work
        # on that stream).
        first, last = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        first.record(stream)
        for _ in range(args.steps):
            step()
        last.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        avg_kernel_s = first.elapsed_time(last) / args.steps / 1e3
        # Per-launch spread, from an untimed pass with an event pair around every launch.
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(min(args.steps, 20))]
        for s, e in ev:
            s.record(stream)
            step()
            e.record(stream)
        torch.cuda.synchronize()
        kernel_ms = [s.elapsed_time(e) for s, e in ev]
    else:
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for s, e in ev:
            scratch.fill_(1.0)          # evicts the inputs from L2 and MALL; outside the events
            s.record(stream)
            step()
            e.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        kernel_ms = [s.elapsed_time(e) for s, e in ev]
        avg_kernel_s = float(np.mean(kernel_ms)) / 1e3
    ms_per_step = wall / args.steps * 1e3

    pairs = pair_count(w, x.kv_len)
    flops = (10.0 if args.backward else 4.0) * w.D * pairs
    elt = {"f32": 4, "bf16": 2, "f16": 2}[w.dtype]
    value = flops / (wall / args.steps) / 1e12
    achieved = flops / avg_kernel_s / 1e12
    if args.cold_bytes:
        value = achieved
    peak = PEAK_TFLOPS[w.dtype]
    nbytes = algorithmic_bytes(w, x.kv_len, elt)
    if args.backward:
        # Q, K, V, O, dO read and dQ, dK, dV written once; LSE read once.
        nbytes = 8 * elt * w.B * w.H * w.N * w.D + 4 * w.B * w.H * w.N
    roofline = {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak, "unit": "TFLOP/s",
                "frac": round(achieved / peak, 4),
                "traffic": measured_traffic(("bwd:" if args.backward else "") + name),
                "algorithmic_flops": flops, "algorithmic_bytes": nbytes,
                "hbm_gbs_algorithmic": round(nbytes / avg_kernel_s / 1e9, 1),
                "kernel_ms_avg": round(avg_kernel_s * 1e3, 4), "kernel_ms_min": round(min(kernel_ms), 4),
                "kernel_ms_median": round(float(np.median(kernel_ms)), 4)}
    if args.backward:
        roofline["executed_flops"] = 14.0 * w.D * pairs
        roofline["executed_tflops"] = round(14.0 * w.D * pairs / avg_kernel_s / 1e12, 2)
    cpu = None
    if not args.no_cpu_baseline:
        if args.backward:
            heads = min(args.cpu_heads, 2)
            log(f"bench: CPU gradient oracle baseline on {heads} heads")
            cpu = cpu_baseline_backward(x, do_cpu, w, heads)
        else:
            log(f"bench: CPU oracle baseline on {args.cpu_heads} heads")
            cpu = cpu_baseline(x, w, args.cpu_heads)
    line = {"metric": METRIC_BWD if args.backward else METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4), "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": w.dtype, "data": "synthetic",
            "config": {"workload": name, "B": w.B, "H": w.H, "N": w.N, "D": w.D, "causal": w.causal,
                       "kv_len": None if x.kv_len is None else [int(t) for t in x.kv_len],
                       "parallelism": "single GPU"},
            "pct_of_peak": round(100.0 * value / peak, 2),
            "cold_cache_bytes": args.cold_bytes or None,
            "roofline": roofline, "cpu_baseline": cpu}
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
