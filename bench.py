#!/usr/bin/env python3
"""Benchmark of the exact attention forward on one MI355X.

One step = one full forward pass (``fa_fwd`` through the C ABI: one kernel
launch) over the long-context workload B=1, H=64, N=16384, d=128, bf16,
causal, with Q/K/V already resident in HBM.  Prints ONE JSON line:

  metric / value / unit   attention forward TFLOP/s, counting 4*B*H*N^2*d
                          FLOPs halved for causal, over the timed steps
  roofline                the kernel against the bf16 dense matrix-core peak
                          (achieved = FLOPs per launch / average launch time
                          from HIP events on the launch stream; traffic = HBM
                          bytes per launch from the committed profiler
                          counters, null if the kernel source changed since)
  cpu_baseline            the fp64 CPU oracle timed on a bounded sample of
                          the same workload on this host's cores
  cpu_baseline_native     the oracle's plain-C twin (fp64 tiled recurrence)
                          timed the same way, as a second CPU baseline

With --backward, a step is one ``fa_bwd`` call (dQ, dK, dV recomputed from
the forward's O and LSE) on the same workload instead; FLOPs are counted as
2.5 times the forward's (the five N x N x d products of the backward, the
recomputation of S included).

With --configs, every workload of the five configs is timed in turn (one
JSON line each): HIP-graph replay of the timed calls (GPU time) and eager
calls, TFLOP/s against the bf16 matrix peak (fp32 vector peak for the fp32
config) and algorithmic GB/s against HBM; the small configs also run
through fa_fwd_split.

With --shapes "B,H,N,d,causal;...", each listed shape (bf16, seeded N(0,1)
inputs) is run in turn and one JSON line per shape is printed with its time
and the two byte models of the pages (read-once bytes and tile-stream
bytes); run under rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE this gives the
measured HBM bytes of each shape (one dispatch of the main kernel per step).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--backward]
       python bench.py --shapes "1,64,4096,128,1;1,64,8192,64,0" [--steps K] [--warmup W]
A shape may add ",Hkv,window[,T[,nsplit]]" to run fa_fwd_ex instead: Hkv K/V
heads, a sliding window (0: none) and T query rows at the newest positions
of the N keys (default T = N); FLOPs then count the visible (query, key)
pairs.  nsplit > 1 runs fa_fwd_split (split-KV with that many key chunks,
then the merge) instead; kv_gbs is then the K/V bytes read once per step
over the step time, the bound of decode (T = 1).  With --graph the timed
calls are captured once in a HIP graph and replayed, so that the time is the
GPU's and not the host's launch overhead (which dominates calls of a few
tens of microseconds); the graph's output is checked against the eager one.
"""

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

# MI355X dense bf16 matrix peak: 256 compute units x 4096 bf16 FLOP per clock
# per CU x 2.4 GHz peak engine clock = 2516.6 TFLOP/s (AMD's published
# 2.5 PFLOP/s, unrounded); bf16_peak_tflops() uses the device's own CU count
MI355X_CUS = 256
BF16_FLOP_PER_CLK_PER_CU = 4096
PEAK_SCLK_GHZ = 2.4
PEAK_BF16_TFLOPS = MI355X_CUS * BF16_FLOP_PER_CLK_PER_CU * PEAK_SCLK_GHZ / 1e3
DEFAULT_WORKLOAD = "longctx_n16384_d128_causal"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
# the sources that define the forward kernel (its counters are void once they change)
KERNEL_SOURCES = [os.path.join(ROOT, "io_aware_exact_fa1_amd", "csrc", f) for f in ("fa_fwd.hip", "fa_device.h")]


def kernel_source_sha256():
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=30)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--workload", default=DEFAULT_WORKLOAD)
    p.add_argument("--cpu-seconds", type=float, default=15.0,
                   help="target CPU time of the oracle baseline sample")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--sample-power", action="store_true",
                   help="sample board power and the shader clock (amd-smi, run as a child process) during "
                        "the timed steps; use enough --steps for a few seconds of run time, and not under "
                        "a profiler")
    p.add_argument("--backward", action="store_true",
                   help="time the backward pass (fa_bwd) instead of the forward")
    p.add_argument("--shapes", default=None,
                   help="semicolon-separated B,H,N,d,causal shapes to run one after the other (forward, bf16)")
    p.add_argument("--configs", action="store_true",
                   help="time every workload of the five configs (one JSON line each), graph-replayed and eager")
    p.add_argument("--graph", action="store_true",
                   help="--shapes: capture the timed calls in one HIP graph (no host launch overhead)")
    p.add_argument("--tile", default=None,
                   help="--shapes: 'Br,Bc' of the library under test (FA_MI355X_LIB), for the tile-stream byte "
                        "model (default: the library's own 256 x 64 at d = 128, 256 x 128 at d = 64)")
    p.add_argument("--memory", default=None,
                   help="'B,H,d,causal;N1,N2,...': peak device memory and time of fa_fwd against an unfused "
                        "matmul-softmax-matmul (torch) at each N")
    p.add_argument("--copy-cal", action="store_true",
                   help="run only a plain device copy of 1 GiB (5 times), to calibrate the HBM "
                        "byte counters (FETCH_SIZE / WRITE_SIZE) of a profiler run")
    return p.parse_args()


def bf16_peak_tflops(cus=MI355X_CUS):
    """Dense bf16 matrix peak of a device with ``cus`` compute units at the
    peak engine clock."""
    return cus * BF16_FLOP_PER_CLK_PER_CU * PEAK_SCLK_GHZ / 1e3


def cpu_model():
    """The host CPU's model name (from /proc/cpuinfo), or None."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def copy_calibration():
    """A plain device-to-device copy of known size: its FETCH_SIZE and
    WRITE_SIZE per dispatch, against 1 GiB each way, give the scale of the
    byte counters."""
    import torch
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    # the same bytes through an element-wise kernel (plain vector loads and
    # stores, as the forward's own loads are), as a cross-check of the scale
    srcf, dstf = src.view(torch.float32), dst.view(torch.float32)
    for _ in range(5):
        torch.add(srcf, 0.0, out=dstf)
    torch.cuda.synchronize()
    log(f"[copy-cal] copied {n} bytes x5 (device copy), then x5 (element-wise add of 0)")


class PowerSampler:
    """Board power and shader clock from ``amd-smi metric -p -c`` every
    ~0.25 s on a background thread; samples at an idle clock (the GPU not
    yet or no longer busy) are dropped."""

    def __init__(self):
        import threading
        self.samples = []
        self._stop = threading.Event()
        self._t = threading.Thread(target=self._run, daemon=True)

    def _one(self):
        import re
        import subprocess
        try:
            out = subprocess.run(["amd-smi", "metric", "-p", "-c"], capture_output=True, text=True,
                                 timeout=5).stdout
        except (OSError, subprocess.SubprocessError):
            return None
        pw = re.search(r"SOCKET_POWER:\s*([\d.]+)\s*W", out)
        ck = re.search(r"^\s*CLK:\s*([\d.]+)\s*MHz", out, re.M)
        return (float(pw.group(1)), float(ck.group(1))) if pw and ck else None

    def _run(self):
        while not self._stop.is_set():
            x = self._one()
            if x and x[1] >= 500:
                self.samples.append(x)
            self._stop.wait(0.25)

    def __enter__(self):
        self._t.start()
        return self

    def __exit__(self, *exc):
        self._stop.set()
        self._t.join()

    def summary(self):
        if not self.samples:
            return None
        w = sorted(x[0] for x in self.samples)
        c = sorted(x[1] for x in self.samples)
        return {"samples": len(w), "socket_w_median": w[len(w) // 2], "socket_w_max": w[-1],
                "sclk_mhz_median": c[len(c) // 2], "sclk_mhz_min": c[0],
                "source": "amd-smi metric -p -c, every ~0.25 s during the timed steps"}


def max_sclk_mhz():
    """The device's highest shader-clock DPM level in MHz, read from sysfs
    (pp_dpm_sclk; no child process), or None where it is not readable."""
    import glob
    import re
    best = None
    for f in glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk"):
        try:
            with open(f) as fh:
                for m in re.finditer(r"(\d+)\s*Mhz", fh.read(), re.I):
                    best = max(best or 0.0, float(m.group(1)))
        except OSError:
            continue
    return best


def measured_traffic(workload):
    """HBM bytes per launch from the committed profiler counters
    (FETCH_SIZE + WRITE_SIZE, each scaled by a plain copy's reading), or
    None when they were taken on another workload or on a kernel source
    other than the one built here."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
        sha = kernel_source_sha256()
    except (OSError, ValueError):
        return None
    if t.get("workload") != workload or t.get("kernel_source_sha256") != sha:
        return None
    return t.get("bytes_per_launch")


def cpu_baseline(w, q, k, v, target_s):
    """Time the fp64 oracle (as it stands) on a bounded sample of the same
    workload: whole heads, every query row computed on its own, until about
    ``target_s`` seconds of CPU work have been done."""
    import numpy as np
    import torch
    from oracle import attention_rows_ref  # CPU baseline leg only

    rows = np.arange(w.N)
    flops = 0.0
    heads = 0
    nrows = 0
    t0 = time.perf_counter()
    el = 0.0
    for b in range(w.B):
        for h in range(w.H):
            qh, kh, vh = (x[b, h].to(torch.float64).numpy() for x in (q, k, v))
            for i in range(0, w.N, 256):
                sel = rows[i:i + 256]
                attention_rows_ref(qh, kh, vh, w.scale, w.causal, sel)
                keys = (sel + 1) if w.causal else np.full(sel.size, w.N)
                flops += 4.0 * float(keys.sum()) * w.d
                nrows += sel.size
            heads += 1
            el = time.perf_counter() - t0
            if el >= target_s:
                break
        if el >= target_s:
            break
    cores = len(os.sched_getaffinity(0))
    blas_threads = None
    try:
        import threadpoolctl
        info = threadpoolctl.threadpool_info()
        blas_threads = max([x.get("num_threads", 1) for x in info if x.get("user_api") == "blas"] or [1])
    except Exception:
        pass
    threads = blas_threads if blas_threads else 1
    return {
        "value": flops / el / 1e12,
        "unit": "TFLOP/s",
        # the whole workload at the sampled rate: an extrapolation, not a measurement
        "full_workload_estimate_s": round(w.flops / (flops / el), 1),
        "cores": int(min(threads, cores)),
        "kind": "oracle",
        "cpu": cpu_model(),
        "sample": (f"{heads} whole head(s) ({nrows} query rows) of {w.name}, each row computed on its own "
                   f"by the fp64 numpy oracle (attention_rows_ref), {el:.1f} s wall; "
                   f"{cores} host cores visible, BLAS threads {blas_threads}"),
    }


def cpu_baseline_native(w, q, k, v, target_s):
    """Time the oracle's plain-C twin (as it stands: fp64 tiled recurrence,
    B_r = B_c = 64, one head per thread) on a bounded sample of the same
    workload: a block of 256 consecutive query rows per head, at a position
    that moves from head to head, heads in rounds of one per host core until
    about ``target_s`` seconds have passed."""
    import concurrent.futures

    import numpy as np
    import torch
    from oracle import native  # CPU baseline leg only

    lib = native.load()
    cores = len(os.sched_getaffinity(0))
    workers = max(1, min(cores, 16))
    R = min(256, w.N)
    flops = 0.0
    blocks = 0
    heads = [(b, h) for b in range(w.B) for h in range(w.H)]

    def one(idx):
        b, h = heads[idx % len(heads)]
        r0 = (idx * 7919 * R) % max(1, w.N - R + 1)
        qh, kh, vh = (x[b, h].to(torch.float64).numpy() for x in (q, k, v))
        native.tiled_rows_c(qh, kh, vh, w.scale, w.causal, 64, 64, r0, r0 + R, lib=lib)
        rows = np.arange(r0, r0 + R)
        keys = (rows + 1) if w.causal else np.full(R, w.N)
        return 4.0 * float(keys.sum()) * w.d

    t0 = time.perf_counter()
    el = 0.0
    with concurrent.futures.ThreadPoolExecutor(max_workers=workers) as ex:
        idx = 0
        while el < target_s:
            for f in list(ex.map(one, range(idx, idx + workers))):
                flops += f
            idx += workers
            blocks += workers
            el = time.perf_counter() - t0
    return {
        "value": flops / el / 1e12,
        "unit": "TFLOP/s",
        "cores": int(workers),
        "kind": "oracle (plain C twin, tiled fp64)",
        "cpu": cpu_model(),
        "sample": (f"{blocks} blocks of {R} consecutive query rows (one per head, position varying by head) of "
                   f"{w.name}, the fp64 tiled recurrence in C (oracle/tiled_ref.c, B_r = B_c = 64, gcc -O2), "
                   f"{workers} threads, {el:.1f} s wall"),
    }


def cpu_baseline_bwd(w, q, k, v, do, target_s):
    """Time the fp64 backward oracle (as it stands) on a bounded sample of the
    same workload: whole heads, dQ of every query row computed on its own
    (S, dP and dQ of the row: 6 * keys * d FLOPs), until about ``target_s``
    seconds of CPU work have been done."""
    import numpy as np
    import torch
    from oracle import attention_bwd_rows_ref  # CPU baseline leg only

    rows = np.arange(w.N)
    flops, heads, nrows, el = 0.0, 0, 0, 0.0
    t0 = time.perf_counter()
    for b in range(w.B):
        for h in range(w.H):
            qh, kh, vh, dh = (x[b, h].to(torch.float64).numpy() for x in (q, k, v, do))
            for i in range(0, w.N, 256):
                sel = rows[i:i + 256]
                attention_bwd_rows_ref(qh, kh, vh, dh, w.scale, w.causal, sel)
                keys = (sel + 1) if w.causal else np.full(sel.size, w.N)
                flops += 6.0 * float(keys.sum()) * w.d
                nrows += sel.size
                el = time.perf_counter() - t0
                if el >= target_s:
                    break
            heads += 1
            if el >= target_s:
                break
        if el >= target_s:
            break
    cores = len(os.sched_getaffinity(0))
    return {
        "value": flops / el / 1e12,
        "unit": "TFLOP/s",
        "cores": int(cores),
        "kind": "oracle",
        "cpu": cpu_model(),
        "sample": (f"{nrows} query rows of {heads} head(s) of {w.name}: dQ of each row computed on its own by "
                   f"the fp64 numpy backward oracle (attention_bwd_rows_ref), {el:.1f} s wall; "
                   f"{cores} host cores visible"),
    }


def shape_sweep(args):
    """One JSON line per shape: forward time and the byte models."""
    import torch
    import io_aware_exact_fa1_amd as fa
    import workloads

    fa.load_library()
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    for spec in args.shapes.split(";"):
        f = [int(x) for x in spec.split(",")]
        B, H, N, d, causal = f[:5]
        ext = len(f) > 5
        hkv, window = (f[5], f[6]) if ext else (H, 0)
        T = f[7] if len(f) > 7 else N
        nsplit = f[8] if len(f) > 8 else 1
        q, k, v = workloads.make_qkv(B, H, N, d, torch.bfloat16, 1000 + N + d)
        qd = q[:, :, N - T:].contiguous().to(dev)
        kd, vd = (x[:, :hkv].contiguous().to(dev) for x in (k, v))
        o = torch.empty_like(qd)
        lse = torch.empty((B, H, T), dtype=torch.float32, device=dev)
        scale = 1.0 / math.sqrt(d)
        G = fa.fa_split_chunks(N, nsplit)
        ws_o = torch.empty((G, B, H, T, d), dtype=torch.float32, device=dev) if nsplit > 1 else None
        ws_l = torch.empty((G, B, H, T), dtype=torch.float32, device=dev) if nsplit > 1 else None
        entry = "fa_fwd_split" if nsplit > 1 else ("fa_fwd_ex" if ext else "fa_fwd")

        def step():
            cs = torch.cuda.current_stream().cuda_stream  # (the capture stream under --graph)
            if nsplit > 1:
                st = fa.fa_fwd_split(qd, kd, vd, o, lse, B, H, hkv, T, N, d, scale, causal, N - T, window, nsplit,
                                     ws_o, ws_l, cs)
            elif ext:
                st = fa.fa_fwd_ex(qd, kd, vd, o, lse, B, H, hkv, T, N, d, scale, causal, N - T, window, cs)
            else:
                st = fa.fa_fwd(qd, kd, vd, o, lse, B, H, N, d, scale, causal, cs)
            if st != fa.FA_OK:
                raise fa.FaError(st, entry)

        for _ in range(args.warmup):
            step()
        torch.cuda.synchronize()
        graph_ok = None
        if args.graph:
            ref_o, ref_l = o.clone(), lse.clone()
            o.zero_()
            lse.zero_()
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph):
                for _ in range(args.steps):
                    step()
            graph.replay()  # warm replay
            torch.cuda.synchronize()
            graph_ok = bool(torch.equal(o, ref_o) and torch.equal(lse, ref_l))
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        if args.graph:
            graph.replay()
        else:
            for _ in range(args.steps):
                step()
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / args.steps
        if ext:
            # visible (query, key) pairs: row i (position N - T + i) sees
            # min(position + 1, window or position + 1) keys when causal
            pos = [N - T + i for i in range(T)]
            pairs = sum(min(p + 1, window) if window else p + 1 for p in pos) if causal else T * N
            flops = 4.0 * B * H * pairs * d
        else:
            flops = 4.0 * B * H * N * N * d / (2 if causal else 1)
        br, bc = (256, (64 if d == 128 else 128)) if not args.tile else (int(x) for x in args.tile.split(","))
        print(json.dumps({"shape": {"B": B, "H": H, "N": N, "d": d, "causal": bool(causal), "Hkv": hkv,
                                    "window": window, "T": T, "entry": entry, "nsplit": nsplit, "chunks": G},
                          "ms": round(ms, 4), "tflops": round(flops / ms / 1e9, 1),
                          "kv_gbs": round(2.0 * B * hkv * N * d * 2 / ms / 1e6, 1),
                          "once_bytes": workloads.hbm_once_bytes(B, H, N, d),
                          "stream_bytes": workloads.tile_stream_bytes(B, H, N, d, br, bc, bool(causal)),
                          "tile": {"Br": br, "Bc": bc}, "library": os.path.basename(fa.load_library()._name),
                          "graph": args.graph, "graph_equals_eager": graph_ok}),
              flush=True)
        if args.graph:
            del graph
        del qd, kd, vd, o, lse, ws_o, ws_l


PEAK_FP32_TFLOPS = 157.3   # MI355X published fp32 vector peak (the fp32 config computes on the vector ALUs)
PEAK_HBM_GBS = 8000.0      # MI355X published HBM3E bandwidth


def cpu_oracle_full(w, q, k, v, workers):
    """Time the fp64 oracle (``attention_ref`` as it stands) on the whole
    workload: one (batch, head) per task on a pool of ``workers`` host
    threads, BLAS held to one thread per task (numpy releases the GIL in
    its matrix products and element-wise loops)."""
    import concurrent.futures
    import threadpoolctl
    from oracle import attention_ref  # CPU baseline leg only

    heads = [(b, h) for b in range(w.B) for h in range(w.H)]

    def one(bh):
        b, h = bh
        attention_ref(q[b, h].double().numpy(), k[b, h].double().numpy(), v[b, h].double().numpy(),
                      w.scale, w.causal)

    with threadpoolctl.threadpool_limits(1, user_api="blas"):
        t0 = time.perf_counter()
        with concurrent.futures.ThreadPoolExecutor(max_workers=workers) as ex:
            list(ex.map(one, heads))
        el = time.perf_counter() - t0
    return {"value": w.flops / el / 1e12, "unit": "TFLOP/s", "cores": workers, "kind": "oracle",
            "cpu": cpu_model(),
            "sample": (f"the whole workload: {len(heads)} (batch, head) pairs of {w.name}, attention_ref "
                       f"(fp64 numpy, S materialised) per pair on {workers} threads, {el:.1f} s wall")}


def launch_floor(steps):
    """Time per call of a graph-replayed one-element kernel: the floor under
    any single-kernel call of a few microseconds."""
    import torch
    x = torch.zeros(1, device="cuda")
    x.add_(1.0)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(steps):
            x.add_(1.0)
    graph.replay()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    graph.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def config_sweep(args):
    """One JSON line per workload: fa_fwd (fa_fwd_f32 for fp32) time from a
    HIP graph of `steps` calls and from eager calls, TFLOP/s against the
    matrix (or, for fp32, vector) peak and algorithmic GB/s (Q, K, V read
    once, O and LSE written once) against HBM; for the small configs also
    fa_fwd_split, whose key chunks multiply the work units."""
    import torch
    import io_aware_exact_fa1_amd as fa
    import workloads

    fa.load_library()
    dev = torch.device("cuda:0")
    floor = launch_floor(args.steps)
    print(json.dumps({"workload": "launch_floor", "note": "graph-replayed one-element torch kernel (x.add_)",
                      "ms": round(floor, 5)}), flush=True)
    peak_bf16 = round(bf16_peak_tflops(torch.cuda.get_device_properties(dev).multi_processor_count), 1)
    workers = min(16, len(os.sched_getaffinity(0)))
    for name, w in workloads.WORKLOADS.items():
        qc, kc, vc = workloads.make_qkv(w.B, w.H, w.N, w.d, w.torch_dtype, w.seed, w.k_mult)
        q, k, v = (x.to(dev) for x in (qc, kc, vc))
        o = torch.empty_like(q)
        lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=dev)
        variants = [("fa_fwd_f32" if w.dtype == "f32" else "fa_fwd", 1)]
        if w.dtype == "bf16" and w.B * w.H * -(-w.N // 256) < 512:
            variants += [("fa_fwd_split", n) for n in (2, 4)]
        for entry, nsplit in variants:
            G = fa.fa_split_chunks(w.N, nsplit)
            ws = (torch.empty((G, w.B, w.H, w.N, w.d), dtype=torch.float32, device=dev),
                  torch.empty((G, w.B, w.H, w.N), dtype=torch.float32, device=dev)) if nsplit > 1 else (None, None)

            def step():
                cs = torch.cuda.current_stream().cuda_stream
                if entry == "fa_fwd_f32":
                    st = fa.fa_fwd_f32(q, k, v, o, lse, w.B, w.H, w.N, w.d, w.scale, w.causal, cs)
                elif entry == "fa_fwd":
                    st = fa.fa_fwd(q, k, v, o, lse, w.B, w.H, w.N, w.d, w.scale, w.causal, cs)
                else:
                    st = fa.fa_fwd_split(q, k, v, o, lse, w.B, w.H, w.H, w.N, w.N, w.d, w.scale, w.causal, 0, 0,
                                         nsplit, ws[0], ws[1], cs)
                if st != fa.FA_OK:
                    raise fa.FaError(st, entry)

            for _ in range(args.warmup):
                step()
            torch.cuda.synchronize()
            ref_o, ref_l = o.clone(), lse.clone()
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph):
                for _ in range(args.steps):
                    step()
            graph.replay()
            torch.cuda.synchronize()
            same = bool(torch.equal(o, ref_o) and torch.equal(lse, ref_l))
            stream = torch.cuda.current_stream()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            graph.replay()
            e1.record(stream)
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / args.steps
            e0.record(stream)
            for _ in range(args.steps):
                step()
            e1.record(stream)
            torch.cuda.synchronize()
            ms_eager = e0.elapsed_time(e1) / args.steps
            peak = PEAK_FP32_TFLOPS if w.dtype == "f32" else peak_bf16
            tf = w.flops / ms / 1e9
            gbs = w.algorithmic_bytes / ms / 1e6
            line = {"workload": name, "note": w.note, "entry": entry, "nsplit": nsplit, "chunks": G,
                    "ms": round(ms, 5), "ms_eager": round(ms_eager, 5),
                    "tflops": round(tf, 2), "peak_tflops": peak, "frac_peak": round(tf / peak, 4),
                    "algorithmic_bytes": w.algorithmic_bytes, "gbs": round(gbs, 1),
                    "frac_hbm": round(gbs / PEAK_HBM_GBS, 4), "graph_equals_eager": same}
            del graph, ws
            if nsplit == 1 and not args.no_cpu_baseline and name != DEFAULT_WORKLOAD:
                # (the long-context workload's oracle time is the main bench's cpu_baseline leg)
                log(f"[configs] timing the CPU oracle on the whole of {name}")
                line["cpu_baseline"] = cpu_oracle_full(w, qc, kc, vc, workers)
            print(json.dumps(line), flush=True)
        del q, k, v, o, lse


def memory_compare(args):
    """Peak device memory (beyond the inputs) and time of one fa_fwd call and
    of the unfused computation it replaces -- S = Q K^T materialised, the
    softmax in fp32, then P V -- at each listed N (one JSON line per N).
    The unfused form is torch matrix products and softmax: a reference
    point for the memory argument of the pages, not part of the library."""
    import torch
    import io_aware_exact_fa1_amd as fa
    import workloads

    fa.load_library()
    head, ns = args.memory.split(";")
    B, H, d, causal = (int(x) for x in head.split(","))
    scale = 1.0 / math.sqrt(d)
    dev = torch.device("cuda:0")

    def timed(fn, reps=3):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    for N in (int(x) for x in ns.split(",")):
        q, k, v = (x.to(dev) for x in workloads.make_qkv(B, H, N, d, torch.bfloat16, 2000 + N))
        torch.cuda.synchronize()
        res = {"B": B, "H": H, "N": N, "d": d, "causal": bool(causal)}
        for name in ("fa_fwd", "unfused"):
            def run():
                if name == "fa_fwd":
                    return fa.forward(q, k, v, causal=bool(causal), scale=scale)
                kt = k.transpose(-2, -1).contiguous()      # (a contiguous right operand for the bf16 product)
                s = torch.matmul(q, kt).float() * scale    # [B, H, N, N]
                if causal:
                    s.masked_fill_(torch.ones(N, N, dtype=torch.bool, device=dev).triu_(1), float("-inf"))
                lse = torch.logsumexp(s, dim=-1)
                p = torch.softmax(s, dim=-1).to(torch.bfloat16)
                del s
                return torch.matmul(p, v), lse
            torch.cuda.synchronize()
            torch.cuda.empty_cache()
            base = torch.cuda.memory_allocated()
            torch.cuda.reset_peak_memory_stats()
            out = run()
            torch.cuda.synchronize()
            peak = torch.cuda.max_memory_allocated() - base
            del out
            ms = timed(lambda: run())
            res[name] = {"peak_bytes_beyond_inputs": int(peak), "ms": round(ms, 4)}
            log(f"[memory] N={N} {name}: peak {peak / 2**20:.1f} MiB beyond the inputs, {ms:.3f} ms")
        res["output_bytes"] = B * H * N * (d * 2 + 4)
        print(json.dumps(res), flush=True)
        del q, k, v
        torch.cuda.empty_cache()


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); the forward pass shards over "
              "(batch, head) and query tiles with no exchange, so there is no multi-GPU run to time.",
              file=sys.stderr)
        sys.exit(2)

    if args.copy_cal:
        copy_calibration()
        return
    if args.configs:
        config_sweep(args)
        return
    if args.shapes:
        shape_sweep(args)
        return
    if args.memory:
        memory_compare(args)
        return

    import torch
    import io_aware_exact_fa1_amd as fa
    import workloads

    if not torch.cuda.is_available():
        log("bench.py needs a GPU")
        sys.exit(1)
    fa.load_library()
    w = workloads.get(args.workload)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    props = torch.cuda.get_device_properties(dev)

    log(f"[bench] generating inputs {w.name} B={w.B} H={w.H} N={w.N} d={w.d} {w.dtype} causal={w.causal}")
    q, k, v = workloads.make_qkv(w.B, w.H, w.N, w.d, w.torch_dtype, w.seed, w.k_mult)
    qd, kd, vd = (x.to(dev) for x in (q, k, v))
    o = torch.empty_like(qd)
    lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=dev)
    entry = fa.fa_fwd if w.dtype == "bf16" else fa.fa_fwd_f32
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream

    def step():
        st = entry(qd, kd, vd, o, lse, w.B, w.H, w.N, w.d, w.scale, int(w.causal), sh)
        if st != fa.FA_OK:
            raise fa.FaError(st, "fa_fwd")

    flops = w.flops
    do = None
    if args.backward:
        if w.dtype != "bf16":
            log("--backward needs a bf16 workload")
            sys.exit(2)
        g = torch.Generator(device="cpu")
        g.manual_seed(w.seed + 7919)
        do = torch.randn(q.shape, generator=g, dtype=torch.float32).to(torch.bfloat16)
        dod = do.to(dev)
        dq, dk, dv = (torch.empty_like(qd) for _ in range(3))
        delta = torch.empty_like(lse)
        step()  # O and LSE of the forward
        flops = 2.5 * w.flops

        def step():
            st = fa.fa_bwd(qd, kd, vd, o, lse, dod, dq, dk, dv, delta, w.B, w.H, w.N, w.d, w.scale,
                           int(w.causal), sh)
            if st != fa.FA_OK:
                raise fa.FaError(st, "fa_bwd")

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"[bench] warmup {args.warmup} done")

    # timed region: K steps between synchronisations; HIP events on the
    # launch stream bracket every launch
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    torch.cuda.synchronize()
    sampler = PowerSampler() if args.sample_power else None
    if sampler:
        sampler.__enter__()
    t0 = time.perf_counter()
    for i in range(args.steps):
        evs[i][0].record(stream)
        step()
        evs[i][1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    if sampler:
        sampler.__exit__()
    launch_ms = sorted(a.elapsed_time(b) for a, b in evs)
    avg_ms = sum(launch_ms) / len(launch_ms)
    med_ms = launch_ms[len(launch_ms) // 2]
    ms_per_step = wall * 1e3 / args.steps
    tflop = flops / 1e12
    value = tflop / (ms_per_step / 1e3)
    achieved = tflop / (avg_ms / 1e3)
    peak = round(bf16_peak_tflops(props.multi_processor_count), 1)
    log(f"[bench] {w.name}: wall {ms_per_step:.3f} ms/step, kernel avg {avg_ms:.3f} ms "
        f"(median {med_ms:.3f}, min {launch_ms[0]:.3f}) -> {achieved:.1f} TFLOP/s "
        f"= {100 * achieved / peak:.1f}% of the {peak} TFLOP/s bf16 dense peak")

    traffic = None if args.backward else measured_traffic(w.name)

    cpu = None
    cpu_native = None
    if not args.no_cpu_baseline:
        log(f"[bench] timing the CPU oracle on a sample (~{args.cpu_seconds:.0f} s)")
        if args.backward:
            cpu = cpu_baseline_bwd(w, q, k, v, do, args.cpu_seconds)
        else:
            cpu = cpu_baseline(w, q, k, v, args.cpu_seconds)
        log(f"[bench] cpu baseline {cpu['value'] * 1e3:.3f} GFLOP/s ({cpu['sample']})")
        if not args.backward:
            cpu_native = cpu_baseline_native(w, q, k, v, args.cpu_seconds / 2)
            log(f"[bench] cpu baseline (C twin) {cpu_native['value'] * 1e3:.3f} GFLOP/s ({cpu_native['sample']})")

    metric = "attn fwd TFLOP/s + % bf16 MFMA peak, N=16K d=128 causal (1 MI355X)"
    if args.backward:
        metric = "attn bwd TFLOP/s (2.5x fwd FLOPs) + % bf16 MFMA peak (1 MI355X)"
    out = {
        "metric": metric,
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "N": w.N, "d": w.d, "causal": w.causal,
                   "scale": w.scale, "pass": "backward" if args.backward else "forward",
                   "flops_per_step": flops, "pct_of_bf16_peak": round(100 * value / peak, 2)},
        # peak = CUs x 4096 bf16 FLOP/clk/CU x 2.4 GHz (the published 2.5 PFLOP/s, unrounded)
        "roofline": {"bound": "mfma", "achieved": round(achieved, 3), "peak": peak,
                     "unit": "TFLOP/s", "frac": round(achieved / peak, 4), "traffic": traffic},
        "cpu_baseline": cpu,
        # the oracle's plain-C twin timed the same way (a second CPU baseline)
        "cpu_baseline_native": cpu_native,
        # per-launch kernel times (HIP events on the launch stream) and the device they ran on
        "kernel_ms": {"avg": round(avg_ms, 4), "median": round(med_ms, 4), "min": round(launch_ms[0], 4)},
        "device": {"arch": props.gcnArchName, "cus": props.multi_processor_count, "max_sclk_mhz": max_sclk_mhz()},
    }
    if sampler:
        out["power"] = sampler.summary()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
