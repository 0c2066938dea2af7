"""Bench: Q4_K_M-mix GEMV effective weight bandwidth at batch 1 on one MI355X.

Workload: a Llama-7B-shaped decode layer in the Q4_K_M mix at batch 1 —
q/k/v/o 4096x4096 and ffn gate/up 11008x4096 as Q4_K, ffn down 4096x11008 as
Q6_K, fp32 activations.  As in decode engines, the projections that share an
input are stored as one matrix (q|k|v: 12288x4096, gate|up: 22016x4096), so a
step is four dependent GEMV launches (qkv, o, gate_up, down) that read every
weight of the layer once.  value = layer blob bytes / time per step, with the
blobs resident in HBM.

Method:
  * weights: synthetic N(0, 0.02^2) fp32, one seeded draw per original matrix,
    quantized on the GPU by the library's quantizer; x ~ N(0, 1) fp32;
  * steps rotate over distinct copies of the layer (>= 640 MB) so no step
    finds its weights in the 256 MB Infinity Cache; the K timed steps run as
    replays of HIP graphs holding 32 consecutive steps each, the way a decode
    engine captures one token's pass over a 32-layer model as one graph (a
    graph per single step adds ~5 us of replay boundary to every step);
    timed region: synchronize, the replays, synchronize, HIP events on the
    replay stream;
  * roofline: the dominant kernel (largest time per step) timed live with HIP
    events over graphs of 16 back-to-back launches of that kernel alone,
    rotating over >= 512 MB of copies; achieved = blob bytes per launch /
    average launch duration, against the 8 TB/s HBM peak; traffic from the
    committed counter summary when it was taken on the current kernel source;
  * fused_layer: the same step with the RMSNorm and SwiGLU fusions of the
    decode entry point on (same weight bytes; norm and gate work added);
  * secondary: the Q4_K 11008x4096 dequant-GEMM at 512 fp16 tokens (GFLOP/s
    against the 2.5 PFLOP/s dense fp16 matrix peak) and a sweep of the other
    workload shapes;
  * attn_decode: one decode step of grouped-query attention over q8_0 and
    q4_0 K/V caches (32k positions, 8 KV heads, head_dim 128, 40 query
    heads), cache bytes per call / time, rotating over >= 512 MB of caches;
  * stream_read_reference (inside roofline): the library's plain
    streaming-read kernel at the dominant launch's size and at 1 GiB;
  * cpu_baseline: the CPU oracle (fp64 dequant-then-dot, OpenMP over rows) on
    the same layer, the oracle quantizing its own blobs from the same draws.

Prints one JSON line.  `--profile-launches N` instead runs N plain (ungraphed)
launches of each layer matrix plus a device copy of known size, and
`--profile-gemm N` N plain launches of the 512-token GEMM, `--profile-attn N` N
plain calls of the q8_0 KV-cache attention decode, and `--profile-shape
TYPE,ROWS,COLS,NTOK,XDT[,N]` N plain launches of any one shape, for rocprofv3
kernel traces and counters.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "Q4_K_M GEMV effective weight GB/s (% HBM peak) at batch 1; GFLOP/s at 512"
HBM_PEAK_GBS = 8000.0
FP16_PEAK_TFLOPS = 2500.0
CACHE_BYTES = 256 << 20
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemv_q4k_decode_layer_counters.md")
GEMV_SRC = os.path.join(ROOT, "gguf_quant_matmul_amd", "csrc", "k_gemv.hip")
GEMM_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemm_q4k_11008x4096_n512.md")
GEMM_SRC = os.path.join(ROOT, "gguf_quant_matmul_amd", "csrc", "k_gemm.hip")

# (name, type, [(part, rows)], cols): parts are the original matrices, stored
# one after another (row-major blobs concatenate row-wise).
LAYER = [
    ("qkv", "q4_k", [("attn_q", 4096), ("attn_k", 4096), ("attn_v", 4096)], 4096),
    ("attn_o", "q4_k", [("attn_o", 4096)], 4096),
    ("ffn_gate_up", "q4_k", [("ffn_gate", 11008), ("ffn_up", 11008)], 4096),
    ("ffn_down", "q6_k", [("ffn_down", 4096)], 11008),
]


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--no-cpu", action="store_true", help="skip the CPU-oracle baseline")
    p.add_argument("--no-sweep", action="store_true", help="skip the secondary shapes")
    p.add_argument("--profile-gemm", type=int, default=0, metavar="N",
                   help="only run N plain launches of the 512-token GEMM (for rocprofv3)")
    p.add_argument("--profile-launches", type=int, default=0)
    p.add_argument("--profile-attn", type=int, default=0, metavar="N",
                   help="only run N plain calls of the q8_0 KV-cache attention decode")
    p.add_argument("--profile-shape", default="", metavar="TYPE,ROWS,COLS,NTOK,XDT[,N]",
                   help="only run N (default 50) plain gq_matmul launches of one shape, e.g. "
                        "q4_k,11008,4096,64,f16 (for rocprofv3 traces and counters)")
    return p.parse_args()


class Mat:
    """A (possibly fused) weight matrix on the GPU with rotating copies."""

    def __init__(self, name, t, parts, cols, seed, ncopies, n_tok=1, x_dtype="f32", keep_w=False):
        import torch
        import gguf_quant_matmul_amd as gq
        import synth
        self.name, self.t, self.cols = name, t, cols
        self.rows = sum(r for _, r in parts)
        self.tid = gq.TYPES[t]
        self.n_tok = n_tok
        self.w = []
        blobs = []
        for i, (_, r) in enumerate(parts):
            w = synth.weights(r, cols, seed=seed + i)
            if keep_w:
                self.w.append(w)
            wd = torch.from_numpy(w).cuda()
            blobs.append(gq.quantize(wd, t))
            del wd
        blob = torch.cat(blobs) if len(blobs) > 1 else blobs[0]
        self.bytes = blob.numel()
        self.copies = [blob] + [blob.clone() for _ in range(ncopies - 1)]
        x = synth.activations(n_tok, cols, seed=seed + 100, dtype=x_dtype)
        self.x_host = x
        self.x = torch.from_numpy(x).cuda()
        self.xt = gq.F16 if x_dtype == "f16" else gq.F32
        self.y = torch.empty((n_tok, self.rows), dtype=torch.float32, device="cuda")

    def ensure_copies(self, total_bytes):
        need = max(2, -(-total_bytes // self.bytes))
        while len(self.copies) < need:
            self.copies.append(self.copies[0].clone())

    def launch(self, copy, stream_ptr):
        import gguf_quant_matmul_amd as gq
        rc = gq.lib().gq_matmul_ex(self.copies[copy % len(self.copies)].data_ptr(), self.tid,
                                   self.rows, self.cols, self.x.data_ptr(), self.xt,
                                   self.y.data_ptr(), self.n_tok, stream_ptr)
        if rc:
            raise RuntimeError(f"gq_matmul_ex({self.name}) failed: {gq.strerror(rc)}")


def capture(fn):
    """Capture fn(stream_ptr) into a HIP graph (torch.cuda.CUDAGraph)."""
    import torch
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn(ctypes.c_void_p(s.cuda_stream))          # warm, outside capture
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


STEPS_PER_GRAPH = 32       # one decoded token of a 32-layer model


def time_steps(step, ncopy, steps, warmup, per_graph=STEPS_PER_GRAPH):
    """Average ms per step over `steps` steps, step i running step(sp, i %
    ncopy), replayed as graphs of per_graph consecutive steps (the last graph
    holds the remainder)."""
    import torch
    if steps < 1:
        raise ValueError("steps must be >= 1")
    g = min(per_graph, steps)
    full, rem = divmod(steps, g)

    def graph_of(first, count):
        def fn(sp):
            for k in range(count):
                step(sp, (first + k) % ncopy)
        return capture(fn)

    # replay j covers steps j*g .. j*g+g-1: one graph per distinct first copy
    by_off = {}
    for j in range(full):
        off = (j * g) % ncopy
        if off not in by_off:
            by_off[off] = graph_of(off, g)
    tail = graph_of((full * g) % ncopy, rem) if rem else None
    order = [by_off[(j * g) % ncopy] for j in range(full)]
    sp = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    for i in range(warmup):                      # exactly `warmup` steps, plain launches
        step(sp, i % ncopy)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for gr in order:
        gr.replay()
    if tail is not None:
        tail.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def replay_spread(graphs, n, per_graph):
    """p10 / p50 / p90 of the per-launch time (ms) over n individually timed
    replays of graphs holding per_graph launches each."""
    import torch
    import numpy as np
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(n)]
    for i in range(n):
        ev[i][0].record()
        graphs[i % len(graphs)].replay()
        ev[i][1].record()
    torch.cuda.synchronize()
    t = np.array([a.elapsed_time(b) for a, b in ev]) / per_graph
    return [float(np.percentile(t, q)) for q in (10, 50, 90)]


def stream_read_reference(steps):
    """Achieved bandwidth of the library's plain streaming-read kernel
    (gq_probe_stream_read: non-temporal 128-bit loads, every byte once) at the dominant
    launch's size and at 1 GiB, rotating over copies totalling >= 2x the
    Infinity Cache: the practical ceiling the GEMV's fraction of the nominal
    peak is read against."""
    import torch
    import gguf_quant_matmul_amd as gq
    out = {}
    for label, nbytes in (("29.5 MB", 29491200), ("1 GiB", 1 << 30)):
        k = max(2, -(-2 * CACHE_BYTES // nbytes))
        bufs = [torch.full((nbytes // 4,), i + 1, dtype=torch.int32, device="cuda") for i in range(k)]
        res = torch.empty(gq.PROBE_OUT_WORDS, dtype=torch.int32, device="cuda")
        per = 16 if nbytes < (64 << 20) else 2
        graphs = []
        for gi in range(-(-k // per)):
            def fn(sp, gi=gi):
                for j in range(per):
                    rc = gq.lib().gq_probe_stream_read(bufs[(gi * per + j) % k].data_ptr(), nbytes,
                                                       res.data_ptr(), sp)
                    if rc:
                        raise RuntimeError(f"gq_probe_stream_read: {gq.strerror(rc)}")
            graphs.append(capture(fn))
        ms = time_graphs(graphs, max(16, steps // per), warmup=2) / per
        out[label] = round(nbytes / (ms * 1e-3) / 1e9, 1)
        del bufs, graphs
        torch.cuda.empty_cache()
    return {"kernel": "gq_probe_stream_read (non-temporal 128-bit loads, each byte once)",
            "GBps": out}


def kernel_time_ms(mat, steps, per_graph=16, spread=False):
    """Live HIP-event timing of back-to-back launches of one matrix, rotating
    over copies totalling >= 2x the Infinity Cache."""
    mat.ensure_copies(2 * CACHE_BYTES)
    graphs = []
    for gi in range(-(-len(mat.copies) // per_graph)):
        def fn(sp, gi=gi):
            for j in range(per_graph):
                mat.launch(gi * per_graph + j, sp)
        graphs.append(capture(fn))
    # eight warmup replays: the compute-bound shapes run a few percent slower
    # in the first milliseconds after lighter work (the 512-token GEMM: 72.6
    # us with two, 68.9 with eight)
    ms = time_graphs(graphs, max(4, steps // per_graph), warmup=8)
    if spread:
        return ms / per_graph, replay_spread(graphs, 32, per_graph)
    return ms / per_graph


def traffic_from_profile(kernel_bytes):
    """HBM bytes per launch of the dominant kernel from the committed counter
    summary, or None when absent or taken on a different kernel source."""
    try:
        text = open(TRAFFIC_FILE).read()
    except OSError:
        return None
    m_sha = re.search(r"k_gemv\.hip sha256:\s*([0-9a-f]{64})", text)
    m_b = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    m_k = re.search(r"for_blob_bytes:\s*(\d+)", text)
    if not (m_sha and m_b and m_k) or int(m_k.group(1)) != kernel_bytes:
        return None
    if hashlib.sha256(open(GEMV_SRC, "rb").read()).hexdigest() != m_sha.group(1):
        return None
    return float(m_b.group(1))


def gemm_fetch_from_profile():
    """HBM bytes fetched per launch of the 512-token GEMM, from the committed
    counter summary, or None when that summary was taken on other source."""
    try:
        text = open(GEMM_TRAFFIC_FILE).read()
    except OSError:
        return None
    m_sha = re.search(r"k_gemm\.hip sha256:\s*([0-9a-f]{64})", text)
    m_b = re.search(r"fetch_bytes_per_launch:\s*(\d+)", text)
    if not (m_sha and m_b):
        return None
    if hashlib.sha256(open(GEMM_SRC, "rb").read()).hexdigest() != m_sha.group(1):
        return None
    return float(m_b.group(1))


def cpu_threads():
    """Threads for the CPU oracle: every core of the affinity mask, within the
    host's CPU share for this GPU when the environment states one
    (OMP_NUM_THREADS); returns (threads, affinity cores)."""
    aff = len(os.sched_getaffinity(0))
    share = os.environ.get("OMP_NUM_THREADS", "")
    th = min(aff, int(share)) if share.isdigit() and int(share) > 0 else aff
    return max(1, th), aff


def cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(layer_mats):
    import numpy as np
    import oracle
    threads, aff = cpu_threads()
    work = []
    for m in layer_mats:
        blob = np.concatenate([oracle.quantize(w, m.t) for w in m.w])   # the oracle's own blobs
        work.append((m, blob, m.x_host))
    total = sum(b.size for _, b, _ in work)
    # repetitions of the whole layer until ~3 s (one thread) and ~8 s (all
    # threads) have passed, at least 3 each: about 10 s of wall time
    res, reps = {}, {}
    for th, budget in ((1, 3.0), (threads, 8.0)):
        ts = []
        t_start = time.perf_counter()
        while len(ts) < 3 or time.perf_counter() - t_start < budget:
            t0 = time.perf_counter()
            for m, b, x in work:
                oracle.matmul_f64(b, m.t, m.rows, m.cols, x, threads=th)
            ts.append(time.perf_counter() - t0)
        res[th] = float(np.median(ts))
        reps[th] = len(ts)
    return {
        "value": round(total / res[threads] / 1e9, 3), "unit": "GB/s", "cores": threads,
        "kind": "oracle",
        "sample": f"the whole layer (4 matrices, {total} blob bytes) per repetition, fp64 "
                  f"dequant-then-dot, median of {reps[threads]} repetitions on {threads} threads "
                  f"({aff} cores in the affinity mask, {threads} the host's share for this GPU); "
                  f"1 thread: {round(total / res[1] / 1e9, 3)} GB/s (median of {reps[1]}, "
                  f"{res[1]:.2f} s each); CPU: {cpu_model()}",
    }


def cpu_baselines():
    """The CPU oracle on every workload configuration (bounded samples of
    rows, all tokens, about one second each on all threads): the single
    2048x2048 Q4_K GEMV, the per-type 4096x4096 sweep and the 32000x4096 Q6_K
    head, Q4_K 11008x4096 at 1, 8 and 64 fp16 tokens, and the Llama-3-8B layer
    set at 1, 8 and 64 tokens.  GB/s = blob bytes of the sampled rows / time;
    GFLOP/s = 2 * sampled rows * cols * tokens / time."""
    import numpy as np
    import oracle
    import synth
    threads, _ = cpu_threads()
    cases = [("single q4_k 2048x2048 n=1", "q4_k", 2048, 2048, 1, "f32")]
    cases += [(f"per-type {t} {r}x{c} n=1", t, r, c, 1, "f32") for _, t, r, c in synth.PER_TYPE_SWEEP_4096]
    cases += [(f"q4_k 11008x4096 n={n} f16", "q4_k", 11008, 4096, n, "f16") for n in (1, 8, 64)]
    for n in synth.LLAMA3_8B_TOKENS:
        for name, t, r, c in synth.LLAMA3_8B_LAYER_Q4KM:
            cases.append((f"llama3-8b {name} {t} {r}x{c} n={n}", t, r, c, n, "f32" if n == 1 else "f16"))
    out = []
    for i, (label, t, rows, cols, n, xdt) in enumerate(cases):
        # rows sampled so one repetition is ~30 M fp64 multiply-adds
        sr = int(min(rows, max(64, 30e6 // (cols * max(n, 4)))))
        w = synth.weights(sr, cols, seed=9500 + i)
        blob = oracle.quantize(w, t)
        x = synth.activations(n, cols, seed=9600 + i, dtype=xdt)
        ts = []
        t_start = time.perf_counter()
        while len(ts) < 3 or time.perf_counter() - t_start < 0.8:
            t0 = time.perf_counter()
            oracle.matmul_f64(blob, t, sr, cols, x, threads=threads)
            ts.append(time.perf_counter() - t0)
        tm = float(np.median(ts))
        out.append({"case": label, "rows_sampled": sr, "GBps": round(blob.size / tm / 1e9, 3),
                    "GFLOPs": round(2.0 * sr * cols * n / tm / 1e9, 2), "threads": threads})
        log(f"  cpu {label}: {sr} rows, {out[-1]['GBps']} GB/s, {out[-1]['GFLOPs']} GFLOP/s")
    return out


def cpu_baseline_gemm(threads=None):
    """The CPU oracle on the 512-token GEMM workload: Q4_K weights drawn as
    the bench draws them (N(0, 0.02^2), quantized by the oracle) times 512
    fp16 N(0, 1) tokens, on a sample of 688 rows (1/16 of the 11008-row
    matrix, all 512 tokens), repeated for about 8 s on all threads;
    GFLOP/s = 2 * rows * cols * 512 / time."""
    import numpy as np
    import oracle
    import synth
    threads = threads or cpu_threads()[0]
    rows, cols, n = 688, 4096, 512
    w = synth.weights(rows, cols, seed=9000)
    blob = oracle.quantize(w, "q4_k")
    x = synth.activations(n, cols, seed=9100, dtype="f16")
    ts = []
    t_start = time.perf_counter()
    while len(ts) < 3 or time.perf_counter() - t_start < 8.0:
        t0 = time.perf_counter()
        oracle.matmul_f64(blob, "q4_k", rows, cols, x, threads=threads)
        ts.append(time.perf_counter() - t0)
    t = float(np.median(ts))
    return {"value": round(2.0 * rows * cols * n / t / 1e9, 2), "unit": "GFLOP/s", "cores": threads,
            "kind": "oracle",
            "sample": f"{rows} of the 11008 rows x 4096 columns, all {n} fp16 tokens, fp64 "
                      f"dequant-then-dot, median of {len(ts)} repetitions ({t:.2f} s each)"}


def sweep(steps):
    """Secondary shapes: one line each, graph-timed with rotating copies."""
    import synth
    out = []
    cases = [("single q4_k 2048x2048", "q4_k", [("w", 2048)], 2048, 1, "f32")]
    cases += [(f"per-type {t} {r}x{c}", t, [(n, r)], c, 1, "f32") for n, t, r, c in synth.PER_TYPE_SWEEP_4096]
    cases += [(f"q4_k 11008x4096 n={n} f16", "q4_k", [("w", 11008)], 4096, n, "f16") for n in synth.GEMM_TOKENS]
    for t in ("q4_1", "q5_k", "q2_k", "q3_k"):
        cases += [(f"{t} 4096x4096 n=1", t, [("w", 4096)], 4096, 1, "f32"),
                  (f"{t} 4096x4096 n=64 f16", t, [("w", 4096)], 4096, 64, "f16"),
                  (f"{t} 4096x4096 n=512 f16", t, [("w", 4096)], 4096, 512, "f16")]
    for n in synth.LLAMA3_8B_TOKENS:
        for name, t, r, c in synth.LLAMA3_8B_LAYER_Q4KM:
            cases.append((f"llama3-8b {name} {t} {r}x{c} n={n}", t, [(name, r)], c, n, "f32" if n == 1 else "f16"))
    for i, (label, t, parts, cols, n, xdt) in enumerate(cases):
        m = Mat(label, t, parts, cols, seed=9000 + 31 * i, ncopies=1, n_tok=n, x_dtype=xdt)
        ms = kernel_time_ms(m, max(64, steps // 2), per_graph=8 if m.bytes > (64 << 20) else 16)
        flops = 2.0 * m.rows * cols * n
        gbps = m.bytes / (ms * 1e-3) / 1e9
        tfl = flops / (ms * 1e-3) / 1e12
        # the roofline this shape sits under: fp16 matrix peak once the
        # flops per weight byte pass the ridge (peak flops / peak bandwidth)
        mfma = flops / m.bytes > FP16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)
        out.append({"case": label, "blob_bytes": m.bytes, "us": round(ms * 1e3, 2),
                    "GBps": round(gbps, 1), "TFLOPs": round(tfl, 2),
                    "bound": "mfma" if mfma else "hbm",
                    "frac": round(tfl / FP16_PEAK_TFLOPS if mfma else gbps / HBM_PEAK_GBS, 4)})
        log(f"  {label}: {ms*1e3:.2f} us  {out[-1]['GBps']} GB/s  {out[-1]['TFLOPs']} TFLOP/s "
            f"({out[-1]['bound']} {out[-1]['frac']})")
        del m
    return out


def fused_layer(mats, steps, warmup):
    """The same layer with the decode fusions on, as an engine would run it:
    RMSNorm fused ahead of qkv, attn_o plain, RMSNorm fused ahead of the
    gate and up halves with the SwiGLU product written by that launch, and
    ffn_down reading that product.  Same weight bytes as the plain step,
    three fewer launches than an engine that normalises and gates apart."""
    import torch
    import gguf_quant_matmul_amd as gq
    import synth
    by = {m.name: m for m in mats}
    qkv, o, gu, down = by["qkv"], by["attn_o"], by["ffn_gate_up"], by["ffn_down"]
    lib = gq.lib()
    half = gu.bytes // 2
    nw1 = torch.from_numpy(synth.norm_weights(qkv.cols, seed=7900)).cuda()
    nw2 = torch.from_numpy(synth.norm_weights(gu.cols, seed=7901)).cuda()
    h = torch.empty(gu.rows // 2, dtype=torch.float32, device="cuda")
    ncopy = len(qkv.copies)

    def call(blob, up, m, rows, x, xt, nw, y, sp):
        rc = lib.gq_matmul_decode(blob, up, m.tid, rows, m.cols, x, xt, nw, ctypes.c_float(1e-5), y, sp)
        if rc:
            raise RuntimeError(f"gq_matmul_decode({m.name}) failed: {gq.strerror(rc)}")

    def step(sp, ci):
        call(qkv.copies[ci].data_ptr(), None, qkv, qkv.rows, qkv.x.data_ptr(), qkv.xt,
             nw1.data_ptr(), qkv.y.data_ptr(), sp)
        o.launch(ci, sp)
        g = gu.copies[ci].data_ptr()
        call(g, g + half, gu, gu.rows // 2, gu.x.data_ptr(), gu.xt, nw2.data_ptr(), h.data_ptr(), sp)
        call(down.copies[ci].data_ptr(), None, down, down.rows, h.data_ptr(), gq.F32,
             None, down.y.data_ptr(), sp)
    return time_steps(step, ncopy, steps, warmup)


# Decode attention over a quantized KV cache: the 30B-class cache of the
# Hitchhiker's Guide §13.2 (8 KV heads, head_dim 128, 32k positions) with 40
# query heads, one layer's K and V.
ATTN = {"kv_len": 32768, "n_kv": 8, "n_heads": 40, "head_dim": 128}


class AttnCase:
    def __init__(self, t, ncopies=None, seed=9500):
        import torch
        import gguf_quant_matmul_amd as gq
        a = ATTN
        self.t = t
        rows = a["kv_len"] * a["n_kv"]
        gen = torch.Generator(device="cuda").manual_seed(seed)
        k = torch.randn(rows, a["head_dim"], device="cuda", generator=gen)
        v = torch.randn(rows, a["head_dim"], device="cuda", generator=gen)
        kb, vb = gq.quantize(k, t), gq.quantize(v, t)
        del k, v
        self.cache_bytes = kb.numel() + vb.numel()
        n = ncopies or max(2, -(-2 * CACHE_BYTES // self.cache_bytes) + 1)
        self.copies = [(kb, vb)] + [(kb.clone(), vb.clone()) for _ in range(n - 1)]
        self.q = torch.randn(a["n_heads"], a["head_dim"], device="cuda", generator=gen)
        self.out = torch.empty_like(self.q)
        need = gq.attn_decode_workspace_bytes(a["kv_len"], a["n_kv"], a["n_heads"], a["head_dim"])
        self.ws = torch.empty(need, dtype=torch.uint8, device="cuda")
        self.tid = gq.TYPES[t]

    def launch(self, i, sp):
        import gguf_quant_matmul_amd as gq
        a = ATTN
        kb, vb = self.copies[i % len(self.copies)]
        rc = gq.lib().gq_attn_decode(kb.data_ptr(), vb.data_ptr(), self.tid, a["kv_len"], a["n_kv"],
                                     a["head_dim"], self.q.data_ptr(), a["n_heads"],
                                     self.out.data_ptr(), self.ws.data_ptr(), self.ws.numel(), sp)
        if rc:
            raise RuntimeError(f"gq_attn_decode: {gq.strerror(rc)}")


def attn_bench(steps):
    """Per-call time of the attention decode (both of its kernels), graph-
    timed over rotating caches totalling >= 2x the Infinity Cache."""
    out = []
    for t in ("q8_0", "q4_0"):
        c = AttnCase(t)
        per = 8
        graphs = []
        for gi in range(-(-len(c.copies) // per)):
            def fn(sp, gi=gi):
                for j in range(per):
                    c.launch(gi * per + j, sp)
            graphs.append(capture(fn))
        ms = time_graphs(graphs, max(32, steps // 2), warmup=2) / per
        gbs = c.cache_bytes / (ms * 1e-3) / 1e9
        out.append({"case": f"decode attention, {t} K and V caches, {ATTN['kv_len']} positions x "
                            f"{ATTN['n_kv']} KV heads x {ATTN['head_dim']}, {ATTN['n_heads']} query heads",
                    "cache_bytes": c.cache_bytes, "us": round(ms * 1e3, 2), "GBps": round(gbs, 1),
                    "frac_of_hbm_peak": round(gbs / HBM_PEAK_GBS, 4)})
        log(f"  attention {t}: {ms*1e3:.2f} us  {gbs:.1f} GB/s")
        del c, graphs
    return out


def profile_launches(mats, n):
    """Plain launches for rocprofv3, in dispatch order: each layer matrix n
    times in turn (rotating copies), then n single-dispatch elementwise
    copies that read 256 MiB and write 256 MiB (counter calibration)."""
    import torch
    sp = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    for m in mats:
        m.ensure_copies(2 * CACHE_BYTES)
    torch.cuda.synchronize()
    for m in mats:
        for i in range(n):
            m.launch(i, sp)
        torch.cuda.synchronize()
    src = torch.ones(64 << 20, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(n):
        torch.mul(src, 1.0, out=dst)
    torch.cuda.synchronize()
    log(f"profile: {n} launches each of {[m.name for m in mats]}, then {n} elementwise copies "
        f"of {src.numel() * 4} bytes")


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU (the library has no multi-GPU path); got --gpus {args.gpus}",
              file=sys.stderr)
        sys.exit(2)
    import torch
    import gguf_quant_matmul_amd as gq

    gq.lib()
    torch.cuda.init()
    if args.profile_attn:
        c = AttnCase("q8_0")
        sp = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        torch.cuda.synchronize()
        for i in range(args.profile_attn):
            c.launch(i, sp)
        torch.cuda.synchronize()
        log(f"profile: {args.profile_attn} calls of the q8_0 attention decode")
        return
    if args.profile_shape:
        f = args.profile_shape.split(",")
        t, rows, cols, n, xdt = f[0], int(f[1]), int(f[2]), int(f[3]), f[4]
        reps = int(f[5]) if len(f) > 5 else 50
        m = Mat(f"{t} {rows}x{cols} n={n} {xdt}", t, [("w", rows)], cols, seed=9000, ncopies=1,
                n_tok=n, x_dtype=xdt)
        m.ensure_copies(2 * CACHE_BYTES)
        sp = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        torch.cuda.synchronize()
        for i in range(reps):
            m.launch(i, sp)
        torch.cuda.synchronize()
        log(f"profile: {reps} launches of {m.name}")
        return
    if args.profile_gemm:
        m = Mat("gemm q4_k 11008x4096 n=512", "q4_k", [("w", 11008)], 4096, seed=9000, ncopies=1,
                n_tok=512, x_dtype="f16")
        m.ensure_copies(2 * CACHE_BYTES)
        sp = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        torch.cuda.synchronize()
        for i in range(args.profile_gemm):
            m.launch(i, sp)
        torch.cuda.synchronize()
        log(f"profile: {args.profile_gemm} launches of {m.name}")
        return
    layer_bytes = sum(gq.row_bytes(t, c) * sum(r for _, r in parts) for _, t, parts, c in LAYER)
    ncopy = max(2, -(-(2 * CACHE_BYTES + CACHE_BYTES // 2) // layer_bytes))
    log(f"setup: {len(LAYER)} launches per step, {layer_bytes} blob bytes, {ncopy} rotating copies")
    mats = [Mat(n, t, parts, c, seed=7000 + 17 * i, ncopies=ncopy, keep_w=not args.no_cpu)
            for i, (n, t, parts, c) in enumerate(LAYER)]
    torch.cuda.synchronize()

    if args.profile_launches:
        profile_launches(mats, args.profile_launches)
        return

    def step(sp, ci):
        for m in mats:
            m.launch(ci, sp)
    log("timing the layer step")
    ms = time_steps(step, ncopy, args.steps, args.warmup)
    value = layer_bytes / (ms * 1e-3) / 1e9
    ms1 = time_steps(step, ncopy, args.steps, args.warmup, per_graph=1)
    log(f"  {ms*1e3:.2f} us/step in {STEPS_PER_GRAPH}-step graphs, {ms1*1e3:.2f} us in one-step graphs")

    log("timing the fused layer step")
    fms = fused_layer(mats, args.steps, args.warmup)
    fused = {"what": "same layer, RMSNorm fused ahead of qkv and gate/up, SwiGLU product "
                     "written by the gate/up launch, ffn_down reading it (4 launches)",
             "ms_per_step": round(fms, 5), "GBps": round(layer_bytes / (fms * 1e-3) / 1e9, 1),
             "vs_plain_step": round(ms / fms, 4)}
    log(f"  fused layer: {fms*1e3:.2f} us/step ({fused['GBps']} GB/s); plain {ms*1e3:.2f} us")

    # per-kernel live timing; a kernel is a (type, launch shape) instantiation
    per, kernels = [], {}
    for m in mats:
        kms, (p10, p50, p90) = kernel_time_ms(m, args.steps, spread=True)
        per.append({"launch": m.name, "type": m.t, "rows": m.rows, "cols": m.cols,
                    "blob_bytes": m.bytes, "us_per_launch": round(kms * 1e3, 3),
                    "us_p10_p50_p90": [round(p10 * 1e3, 3), round(p50 * 1e3, 3), round(p90 * 1e3, 3)],
                    "GBps": round(m.bytes / (kms * 1e-3) / 1e9, 1)})
        log(f"  {m.name:12s} {m.t} {m.rows}x{m.cols}: {kms*1e3:.2f} us  {per[-1]['GBps']} GB/s")
        key = f"gemv {m.t}, {m.cols} cols, fp32 x, batch 1"
        k = kernels.setdefault(key, {"launches": 0, "us": 0.0, "bytes": 0})
        k["launches"] += 1
        k["us"] += kms * 1e3
        k["bytes"] += m.bytes
    dom_key = max(kernels, key=lambda k: kernels[k]["us"])
    dom = kernels[dom_key]
    avg_us = dom["us"] / dom["launches"]
    avg_bytes = dom["bytes"] / dom["launches"]
    achieved = avg_bytes / (avg_us * 1e-6) / 1e9
    traffic = traffic_from_profile(int(avg_bytes))
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                "kernel": dom_key, "launches_per_step": dom["launches"],
                "bytes_per_launch": avg_bytes, "us_per_launch": round(avg_us, 3)}

    log("streaming-read reference")
    roofline["stream_read_reference"] = stream_read_reference(args.steps)
    log(f"  {roofline['stream_read_reference']}")

    secondary, shapes = None, None
    if not args.no_sweep:
        shapes = sweep(args.steps)
        g = [s for s in shapes if s["case"] == "q4_k 11008x4096 n=512 f16"][0]
        tf = g["TFLOPs"]
        secondary = {"metric": "Q4_K 11008x4096 dequant-GEMM GFLOP/s at 512 fp16 tokens",
                     "value": round(tf * 1e3, 1), "unit": "GFLOP/s", "us_per_launch": g["us"],
                     "roofline": {"bound": "mfma", "achieved": tf, "peak": FP16_PEAK_TFLOPS,
                                  "unit": "TFLOP/s", "frac": round(tf / FP16_PEAK_TFLOPS, 4),
                                  "traffic": gemm_fetch_from_profile(),
                                  "traffic_note": "HBM bytes fetched per launch (FETCH_SIZE, "
                                                  "calibrated); writes not included"}}
        if not args.no_cpu:
            log("cpu baseline of the 512-token GEMM (oracle)")
            secondary["cpu_baseline"] = cpu_baseline_gemm()

    attn = None
    if not args.no_sweep:
        log("attention decode over quantized KV caches")
        attn = attn_bench(args.steps)

    cpu, cpus = None, None
    if not args.no_cpu:
        log("cpu baseline (oracle)")
        cpu = cpu_baseline(mats)
        if not args.no_sweep:
            log("cpu baselines of the other workload configurations (oracle, row samples)")
            cpus = cpu_baselines()

    out = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic (seeded N(0,0.02) weights quantized on the GPU, N(0,1) activations)",
        "config": {"workload": "Llama-7B-shaped decode layer, Q4_K_M mix, batch 1",
                   "launches": [f"{n} {t} {sum(r for _, r in p)}x{c}" for n, t, p, c in LAYER],
                   "layer_blob_bytes": layer_bytes, "n_tok": 1, "x_dtype": "f32",
                   "rotating_copies": ncopy, "steps_per_graph": STEPS_PER_GRAPH,
                   "pct_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2)},
        "one_step_graphs": {"ms_per_step": round(ms1, 5),
                            "GBps": round(layer_bytes / (ms1 * 1e-3) / 1e9, 1),
                            "what": "the same steps replayed as one graph per step"},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "secondary": secondary,
        "attn_decode": attn,
        "fused_layer": fused,
        "per_launch": per,
        "sweep": shapes,
        "cpu_baselines": cpus,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
