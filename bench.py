"""Bench: Q4_K_M-mix GEMV effective weight bandwidth at batch 1 on one MI355X.

A step is one pass of the decode-layer GEMVs of a Llama-7B-shaped layer in the
Q4_K_M mix at batch 1 (q/k/v/o and ffn gate/up as Q4_K, ffn down as Q6_K,
fp32 activations), i.e. every weight of the layer read once.  value = blob
bytes of the layer / time per step, with the blobs resident in HBM.

Method:
  * weights: synthetic N(0, 0.02^2) fp32 (synth.py), quantized on the GPU by
    the library's own quantizer; x ~ N(0, 1) fp32;
  * each step is replayed as a HIP graph of the 7 launches; steps rotate over
    5 distinct copies of the layer (627 MB) so no step finds its weights in the
    256 MB Infinity Cache;
  * timed region: synchronize, K graph replays, synchronize (HIP events on the
    replay stream);
  * roofline: the dominant kernel (largest time per step) is timed live with
    HIP events over graphs of back-to-back launches of that kernel alone,
    rotating over >= 512 MB of copies; achieved = blob bytes per launch /
    average launch duration against the 8 TB/s HBM peak;
  * secondary: the Q4_K 11008x4096 dequant-GEMM at 512 fp16 tokens, GFLOP/s
    against the 2.5 PFLOP/s dense fp16 matrix peak;
  * cpu_baseline: the CPU oracle (fp64 dequant-then-dot, OpenMP over rows) on
    the same layer, the oracle quantizing its own blobs from the same draws.

Prints one JSON line.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "Q4_K_M GEMV effective weight GB/s (% HBM peak) at batch 1; GFLOP/s at 512"
HBM_PEAK_GBS = 8000.0
FP16_PEAK_TFLOPS = 2500.0
CACHE_BYTES = 256 << 20


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--no-cpu", action="store_true", help="skip the CPU-oracle baseline")
    p.add_argument("--no-gemm", action="store_true", help="skip the 512-token GEMM line")
    return p.parse_args()


class Mat:
    def __init__(self, name, t, rows, cols, seed, ncopies):
        import torch
        import gguf_quant_matmul_amd as gq
        import synth
        self.name, self.t, self.rows, self.cols = name, t, rows, cols
        self.tid = gq.TYPES[t]
        self.w = synth.weights(rows, cols, seed=seed)          # host fp32, kept for the oracle
        wd = torch.from_numpy(self.w).cuda()
        blob = gq.quantize(wd, t)
        del wd
        self.bytes = blob.numel()
        self.copies = [blob] + [blob.clone() for _ in range(ncopies - 1)]
        self.x = torch.from_numpy(synth.activations(1, cols, seed=seed + 1)).cuda()
        self.y = torch.empty((1, rows), dtype=torch.float32, device="cuda")

    def launch(self, copy, stream_ptr, n=1, x=None, y=None):
        import gguf_quant_matmul_amd as gq
        x = self.x if x is None else x
        y = self.y if y is None else y
        xt = gq.F16 if x.dtype.itemsize == 2 else gq.F32
        rc = gq.lib().gq_matmul_ex(self.copies[copy % len(self.copies)].data_ptr(), self.tid,
                                   self.rows, self.cols, x.data_ptr(), xt, y.data_ptr(), n,
                                   stream_ptr)
        if rc:
            raise RuntimeError(f"gq_matmul_ex({self.name}) failed: {gq.strerror(rc)}")


def capture(fn):
    """Capture fn(stream_ptr) into a torch CUDA (HIP) graph."""
    import torch
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn(ctypes.c_void_p(s.cuda_stream))          # warm (outside capture)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        fn(ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    torch.cuda.synchronize()
    return g


def time_graphs(graphs, steps, warmup):
    """Average ms per replay over `steps` replays cycling through graphs."""
    import torch
    for i in range(warmup):
        graphs[i % len(graphs)].replay()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(steps):
        graphs[i % len(graphs)].replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def kernel_time_ms(mat, steps, launches_per_graph=16, n=1, x=None, y=None):
    """Live HIP-event timing of back-to-back launches of one kernel, rotating
    over copies of its blob totalling >= 2x the Infinity Cache."""
    need = max(2, -(-2 * CACHE_BYTES // mat.bytes))
    while len(mat.copies) < need:
        mat.copies.append(mat.copies[0].clone())
    ng = -(-len(mat.copies) // launches_per_graph)
    graphs = []
    for gi in range(ng):
        def fn(sp, gi=gi):
            for j in range(launches_per_graph):
                mat.launch(gi * launches_per_graph + j, sp, n=n, x=x, y=y)
        graphs.append(capture(fn))
    reps = max(4, steps // launches_per_graph)
    ms = time_graphs(graphs, reps, warmup=2)
    return ms / launches_per_graph


def cpu_baseline(mats, xs):
    import numpy as np
    import oracle
    threads = max(1, min(16, len(os.sched_getaffinity(0))))
    blobs = [oracle.quantize(m.w, m.t) for m in mats]       # the oracle's own blobs
    total = sum(b.size for b in blobs)
    res = {}
    for th in (1, threads):
        ts = []
        for _ in range(3 if th > 1 else 1):
            t0 = time.perf_counter()
            for m, b, x in zip(mats, blobs, xs):
                oracle.matmul_f64(b, m.t, m.rows, m.cols, x, threads=th)
            ts.append(time.perf_counter() - t0)
        res[th] = float(np.median(ts))
    cpu = "unknown"
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    cpu = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {
        "value": round(total / res[threads] / 1e9, 3), "unit": "GB/s", "cores": threads,
        "kind": "oracle",
        "sample": f"the full layer once per repetition (7 matrices, {total} blob bytes), "
                  f"fp64 dequant-then-dot, median of 3; 1-thread: "
                  f"{round(total / res[1] / 1e9, 3)} GB/s ({res[1]:.2f} s); CPU: {cpu}",
    }


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (this build has no multi-GPU path); got --gpus {args.gpus}",
              file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch
    import gguf_quant_matmul_amd as gq
    import synth

    gq.lib()
    torch.cuda.init()
    layer = synth.LLAMA7B_LAYER_Q4KM
    layer_bytes = sum(gq.row_bytes(t, c) * r for _, t, r, c in layer)
    ncopy = max(2, -(-(2 * CACHE_BYTES + CACHE_BYTES // 2) // layer_bytes))
    log(f"setup: {len(layer)} matrices, {layer_bytes} blob bytes, {ncopy} rotating copies")
    mats = [Mat(n, t, r, c, seed=7000 + 17 * i, ncopies=ncopy) for i, (n, t, r, c) in enumerate(layer)]
    torch.cuda.synchronize()

    step_graphs = []
    for ci in range(ncopy):
        def fn(sp, ci=ci):
            for m in mats:
                m.launch(ci, sp)
        step_graphs.append(capture(fn))
    log("timing the layer step")
    ms = time_graphs(step_graphs, args.steps, args.warmup)
    value = layer_bytes / (ms * 1e-3) / 1e9

    # per-kernel live timing; kernels are distinct per (type, launch shape)
    per = []
    for m in mats:
        kms = kernel_time_ms(m, args.steps)
        per.append({"matrix": m.name, "type": m.t, "rows": m.rows, "cols": m.cols,
                    "blob_bytes": m.bytes, "us_per_launch": round(kms * 1e3, 3),
                    "GBps": round(m.bytes / (kms * 1e-3) / 1e9, 1)})
        log(f"  {m.name:9s} {m.t} {m.rows}x{m.cols}: {kms*1e3:.2f} us  {per[-1]['GBps']} GB/s")
    # group identical launch shapes (same kernel instantiation)
    groups = {}
    for p in per:
        k = (p["type"], p["rows"], p["cols"])
        g = groups.setdefault(k, {"launches": 0, "us": p["us_per_launch"], "bytes": p["blob_bytes"]})
        g["launches"] += 1
    dom_key = max(groups, key=lambda k: groups[k]["launches"] * groups[k]["us"])
    dom = groups[dom_key]
    achieved = dom["bytes"] / (dom["us"] * 1e-6) / 1e9
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                "kernel": f"gemv {dom_key[0]} {dom_key[1]}x{dom_key[2]} batch 1 fp32 x",
                "per_launch_bytes": dom["bytes"], "us_per_launch": dom["us"]}

    secondary = None
    if not args.no_gemm:
        name, t, r, c = synth.GEMM_Q4K_11008[0]
        gm = Mat(name, t, r, c, seed=9000, ncopies=1)
        n = 512
        xg = torch.from_numpy(synth.activations(n, c, seed=9001, dtype="f16")).cuda()
        yg = torch.empty((n, r), dtype=torch.float32, device="cuda")
        gms = kernel_time_ms(gm, max(64, args.steps // 2), launches_per_graph=8, n=n, x=xg, y=yg)
        flops = 2.0 * r * c * n
        tf = flops / (gms * 1e-3) / 1e12
        secondary = {"metric": "Q4_K 11008x4096 dequant-GEMM GFLOP/s at 512 fp16 tokens",
                     "value": round(tf * 1e3, 1), "unit": "GFLOP/s", "us_per_launch": round(gms * 1e3, 2),
                     "roofline": {"bound": "mfma", "achieved": round(tf, 2), "peak": FP16_PEAK_TFLOPS,
                                  "unit": "TFLOP/s", "frac": round(tf / FP16_PEAK_TFLOPS, 4),
                                  "traffic": None}}
        log(f"  gemm n=512: {gms*1e3:.1f} us  {tf:.1f} TFLOP/s")
        del gm

    cpu = None
    if not args.no_cpu:
        log("cpu baseline (oracle)")
        xs = [m.x.cpu().numpy() for m in mats]
        cpu = cpu_baseline(mats, xs)

    out = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic (seeded N(0,0.02) weights quantized on the GPU, N(0,1) activations)",
        "config": {"workload": "Llama-7B-shaped decode layer, Q4_K_M mix, batch 1",
                   "matrices": [f"{n} {t} {r}x{c}" for n, t, r, c in layer],
                   "layer_blob_bytes": layer_bytes, "n_tok": 1, "x_dtype": "f32",
                   "rotating_copies": ncopy, "pct_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2)},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "secondary": secondary,
        "per_matrix": per,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
