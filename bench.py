#!/usr/bin/env python3
"""mpgemm benchmark: TFLOPS/TOPS per precision and fraction of the MI355X
MFMA / HBM roofline, with the CPU oracle timed beside it.

One step is one FP16 GEMM C = A * B^T at M = N = K = 8192 (the FP16 square
workload at its largest size) with inputs resident in HBM; `value` is its
throughput. The same run also measures every precision at every size of the
workloads (FP16/INT8/INT4 square N = 512 ... 8192, W4A16 4096 x 4096 at
M = 1, 16, 128), the INT4 x INT4 GEMM with scale epilogue (W4A4) at N = 4096
and 8192, the same with its rank-32 low-rank branch (w4a4lr), the INT4 weight
quantiser at N = K = 4096 and 8192 (G = 128),
and one pass of the whole GEMM hot path (all of those GEMMs at their largest
size), reported under `per_precision` and `hot_path`.

Timing: HIP events recorded on the stream the kernels are launched on (torch's
current stream), W warm-up launches, then K timed launches between two
synchronisations. Small problems rotate through enough distinct input copies
that the 256 MB Infinity Cache cannot serve repeats ("cold"); their sweep
entries also carry `us_warm`, the same launches on a single input set that
stays cached (context only: every throughput and roofline figure is cold).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-sweep]
                       [--no-cpu-baseline] [--only f16|i8|i4|w4a16|w4a4|w4a4lr|quantize] [--eager]
"""
import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

# MI355X published dense peaks (no sparsity) and HBM bandwidth.
PEAK = {"f16": 2500.0, "i8": 5000.0, "i4": 5000.0, "w4a4": 5000.0,   # TFLOP/s or TOP/s; INT4 runs on i8 MFMA
        "w4a4lr": 5000.0}   # W4A4 with the low-rank branch: priced as its INT4 product
HBM_GBS = 8000.0
MALL_BYTES = 256 << 20

SQUARE_SIZES = [512, 1024, 2048, 4096, 8192]
W4A16_M = [1, 16, 128]
W4A16_NK = 4096
W4A16_G = 128
CONFIG_INDEX = {"i8_512": 0, "f16": 1, "i8": 2, "i4": 3, "w4a16": 4, "quantize": 5, "w4a4": 6, "w4a4lr": 7}
W4A4_SIZES = [4096, 8192]
LOWRANK_R = 32   # rank of the W4A4 low-rank branch in the sweep
QUANT_NK = [4096, 8192]   # N = K of the weight matrices quantised (G = 128)


def log(*a):
    print(*a, file=sys.stderr, flush=True)


TILE_SOURCE = os.path.join(ROOT, "precision_dense_gemm_tiled_amd", "csrc", "gemm_tile.hip")
TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "traffic_gemm_tile_f16_8192.md")
W4A16_SOURCE = os.path.join(ROOT, "precision_dense_gemm_tiled_amd", "csrc", "w4a16.hip")
W4A16_TRACE_PROFILE = os.path.join(ROOT, "profiles", "w4a16_4096_kernel_trace.md")


def source_sha256(path):
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def measured_traffic():
    """HBM-side bytes per launch of the headline kernel from the committed
    rocprofv3 FETCH_SIZE / WRITE_SIZE summary, or None if there is none or the
    kernel source changed since the counters were taken."""
    try:
        text = open(TRAFFIC_PROFILE).read()
    except OSError:
        return None
    sha = re.search(r"kernel_source_sha256:\s*([0-9a-f]{64})", text)
    val = re.search(r"traffic_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not sha or not val or sha.group(1) != source_sha256(TILE_SOURCE):
        return None
    return float(val.group(1))


def w4a16_kernel_trace():
    """Per-call kernel durations (ns, summed over the kernels of a call) of
    the W4A16 workloads from the committed rocprofv3 kernel-trace summary, as
    {M: ns}, or None if there is none or the kernel source changed since."""
    try:
        text = open(W4A16_TRACE_PROFILE).read()
    except OSError:
        return None
    sha = re.search(r"w4a16_source_sha256:\s*([0-9a-f]{64})", text)
    val = re.search(r"kernel_trace_ns_per_call:\s*(\{.*\})", text)
    if not sha or not val or sha.group(1) != source_sha256(W4A16_SOURCE):
        return None
    return {int(k): float(v) for k, v in json.loads(val.group(1)).items()}


def algorithmic_bytes(prec, M, N, K, G=W4A16_G):
    """Compulsory HBM bytes of one call: read A and B (and scales) once, write C."""
    if prec == "f16":
        return 2 * M * K + 2 * N * K + 4 * M * N
    if prec == "i8":
        return M * K + N * K + 4 * M * N
    if prec == "i4":
        return (M * K + N * K) // 2 + 4 * M * N
    if prec == "w4a16":
        return 2 * M * K + N * K // 2 + 2 * N * (K // G) + 2 * M * N
    if prec == "w4a4":       # packed A and B, fp16 scales and bias, fp16 Y
        return (M * K + N * K) // 2 + 2 * M * N + 2 * M + 4 * N
    if prec == "w4a4lr":     # the same plus fp16 X, LD (R x K) and LU (N x R)
        return algorithmic_bytes("w4a4", M, N, K) + 2 * M * K + 2 * LOWRANK_R * (K + N)
    if prec == "quantize":   # read fp16 W, write packed codes and scales
        return 2 * N * K + N * K // 2 + 2 * N * (K // G)
    raise ValueError(prec)


def roofline(prec, M, N, K, seconds):
    ops = 2.0 * M * N * K if prec != "quantize" else 0.0
    nbytes = algorithmic_bytes(prec, M, N, K)
    if prec in ("w4a16", "quantize"):
        peak_ops = PEAK["f16"] * 1e12
    else:
        peak_ops = PEAK[prec] * 1e12
    t_compute = ops / peak_ops
    t_mem = nbytes / (HBM_GBS * 1e9)
    bound = "mfma" if t_compute >= t_mem else "hbm"
    if bound == "mfma":
        achieved = ops / seconds / 1e12
        peak = peak_ops / 1e12
        unit = "TFLOP/s" if prec in ("f16", "w4a16") else "TOP/s"
    else:
        achieved = nbytes / seconds / 1e9
        peak = HBM_GBS
        unit = "GB/s"
    return {"bound": bound, "achieved": round(achieved, 3), "peak": peak, "unit": unit,
            "frac": round(achieved / peak, 4), "algorithmic_bytes": nbytes, "ops": ops}


# ------------------------------------------------------------------ problems

class Problem:
    """Device-resident inputs of one (precision, shape), with `copies` distinct
    input sets when the working set would otherwise stay in the MALL."""

    def __init__(self, prec, M, N, K, seed, copies=1, b_layout="nk"):
        import torch
        from precision_dense_gemm_tiled_amd import inputs
        self.prec, self.M, self.N, self.K = prec, M, N, K
        self.b_layout = b_layout
        if prec in ("w4a4", "w4a4lr"):
            if prec == "w4a4":
                vals = inputs.w4a4_problem(M, N, K, seed)
            else:
                vals = inputs.w4a4_lowrank_problem(M, N, K, LOWRANK_R, seed)
            t = [torch.from_numpy(v).cuda() for v in vals]
            self.ins = [tuple(t)] + [tuple(v.clone() for v in t) for _ in range(copies - 1)]
            self.out = torch.empty((M, N), dtype=torch.float16, device="cuda")
        elif prec == "quantize":
            W = torch.from_numpy(inputs.f16_weights(seed, 0, N, K)).cuda()
            self.ins = [W] + [W.clone() for _ in range(copies - 1)]
            self.out = (torch.empty((N, K // 2), dtype=torch.uint8, device="cuda"),
                        torch.empty((N, K // W4A16_G), dtype=torch.float16, device="cuda"))
        elif prec == "w4a16":
            X, W, S = inputs.w4a16_problem(M, N, K, W4A16_G, seed)
            x, w, s = (torch.from_numpy(v).cuda() for v in (X, W, S))
            # rotate weights+scales (the streamed operand); activations stay put
            self.ins = [(x, w.clone(), s.clone()) for _ in range(copies)]
            self.out = torch.empty((M, N), dtype=torch.float16, device="cuda")
        else:
            A, B = inputs.gemm_problem(prec, M, N, K, seed)
            if b_layout == "kn":
                B = transpose_b(prec, B, N, K)
            a, b = torch.from_numpy(A).cuda(), torch.from_numpy(B).cuda()
            self.ins = [(a, b)] + [(a.clone(), b.clone()) for _ in range(copies - 1)]
            odt = torch.float32 if prec == "f16" else torch.int32
            self.out = torch.empty((M, N), dtype=odt, device="cuda")
        self.i = 0

    def launch(self):
        import precision_dense_gemm_tiled_amd as mp
        ins = self.ins[self.i % len(self.ins)]
        self.i += 1
        if self.b_layout == "kn":
            if self.prec == "i4":
                mp.gemm_i4_kn(ins[0], ins[1], self.N, out=self.out)
            else:
                (mp.gemm_f16_kn if self.prec == "f16" else mp.gemm_i8_kn)(ins[0], ins[1], out=self.out)
        elif self.prec == "f16":
            mp.gemm_f16(ins[0], ins[1], out=self.out)
        elif self.prec == "i8":
            mp.gemm_i8(ins[0], ins[1], out=self.out)
        elif self.prec == "i4":
            mp.gemm_i4(ins[0], ins[1], self.K, out=self.out)
        elif self.prec == "quantize":
            mp.quantize_w4(ins, W4A16_G, out_q=self.out[0], out_s=self.out[1])
        elif self.prec == "w4a4":
            mp.gemm_w4a4(ins[0], ins[1], self.K, ins[2], ins[3], ins[4], out=self.out)
        elif self.prec == "w4a4lr":
            mp.gemm_w4a4_lowrank(ins[0], ins[1], self.K, ins[2], ins[3], ins[5], ins[6], ins[7], bias=ins[4],
                                 out=self.out)
        else:
            mp.gemm_w4a16(ins[0], ins[1], ins[2], W4A16_G, out=self.out)


def transpose_b(prec, B, N, K):
    """B (N x K, packed along K for INT4) -> the same values stored K x N
    (INT4: packed two n per byte, low nibble = even n), for the transposed-B
    control. Host-side layout change only."""
    import numpy as np
    if prec != "i4":
        return np.ascontiguousarray(B.T)
    lo = (B & 0x0F).astype(np.uint8)
    hi = (B >> 4).astype(np.uint8)
    q = np.empty((N, 2 * B.shape[1]), dtype=np.uint8)   # nibbles, N x K
    q[:, 0::2], q[:, 1::2] = lo, hi
    qt = np.ascontiguousarray(q[:, :K].T)               # K x N
    if N % 2:
        qt = np.concatenate([qt, np.zeros((K, 1), dtype=np.uint8)], axis=1)
    return (qt[:, 0::2] | (qt[:, 1::2] << 4)).astype(np.uint8)


class ReadProblem:
    """A plain streaming read of `nbytes` (mpgemm_stream_read), rotating over
    enough distinct copies that the Infinity Cache cannot serve repeats: the
    cold-read ceiling of a call that must move those bytes once."""

    def __init__(self, nbytes, loads_per_lane, copies):
        import torch
        self.nbytes = nbytes
        self.lpl = loads_per_lane
        base = torch.randint(0, 256, (nbytes,), dtype=torch.uint8, device="cuda")
        self.ins = [base] + [base.clone() for _ in range(copies - 1)]
        self.words = -(-nbytes // (4096 * loads_per_lane))
        self.out = torch.empty(self.words, dtype=torch.int32, device="cuda")
        self.i = 0

    def launch(self):
        import torch
        import precision_dense_gemm_tiled_amd as mp
        src = self.ins[self.i % len(self.ins)]
        self.i += 1
        st = mp.mpgemm_stream_read(src.data_ptr(), self.nbytes, self.lpl, self.out.data_ptr(), self.words,
                                   torch.cuda.current_stream().cuda_stream)
        if st != 0:
            raise mp.MpgemmError(st, "mpgemm_stream_read")


def read_floor(nbytes, steps):
    """Fastest cold streaming read of nbytes over 1, 2, 4 and 8 loads per
    lane: (seconds per read, loads per lane)."""
    import torch
    copies = int(math.ceil(2 * MALL_BYTES / nbytes))
    best = None
    for lpl in (1, 2, 4, 8):
        p = ReadProblem(nbytes, lpl, copies)
        t = time_graph(p, max(copies, 2048 // 4), max(steps, 3))
        del p
        torch.cuda.empty_cache()
        if best is None or t < best[0]:
            best = (t, lpl)
    return best


def copies_for_cold(prec, M, N, K):
    b = algorithmic_bytes(prec, M, N, K)
    return 1 if b >= 2 * MALL_BYTES else int(math.ceil(2 * MALL_BYTES / b))


def time_launches(launch, steps, warmup):
    """Average seconds per launch over `steps` launches, HIP events on the
    current stream, synchronised on both sides of the timed region."""
    import torch
    for _ in range(warmup):
        launch()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(steps):
        launch()
    stop.record()
    torch.cuda.synchronize()
    return start.elapsed_time(stop) / 1e3 / steps


def time_graph(prob, launches, replays):
    """Average seconds per launch with `launches` consecutive launches (cycling
    through the problem's input copies) captured in one HIP graph and the graph
    replayed `replays` times between events. Removes the host launch overhead
    that dominates microsecond kernels. The replayed output is checked against
    an eager launch on the same inputs."""
    import torch
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):      # warm-up outside capture
        for _ in range(3):
            prob.launch()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    prob.i = 0
    with torch.cuda.graph(g):
        for _ in range(launches):
            prob.launch()
    g.replay()
    torch.cuda.synchronize()
    outs = prob.out if isinstance(prob.out, tuple) else (prob.out,)
    replayed = [o.clone() for o in outs]
    prob.i = launches - 1
    prob.launch()
    torch.cuda.synchronize()
    if not all(torch.equal(r, o) for r, o in zip(replayed, outs)):
        raise RuntimeError("graph replay output differs from the eager launch")
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(replays):
        g.replay()
    stop.record()
    torch.cuda.synchronize()
    del g
    return start.elapsed_time(stop) / 1e3 / (replays * launches)


def sweep_entry(prec, M, N, K, seed, steps, warmup, eager=False, b_layout="nk", launches=None):
    copies = copies_for_cold(prec, M, N, K)
    p = Problem(prec, M, N, K, seed, copies, b_layout)
    if launches is None:
        # expected kernel time at ~30% of the roofline sets the launches per graph
        est_s = max(roofline(prec, M, N, K, 1.0)["ops"] / (PEAK.get(prec, 2500.0) * 1e12 * 0.3),
                    algorithmic_bytes(prec, M, N, K) / (HBM_GBS * 1e9 * 0.3))
        launches = int(min(max(len(p.ins), 0.02 / max(est_s, 1e-7)), 2048))
    launches = max(launches, 2)
    if eager:
        # one launch at a time (for counter collection, which does not follow
        # graph replays); launch overhead is included
        reps = launches * max(steps, 3)
        t = time_launches(p.launch, reps, max(warmup, 1))
    else:
        t = time_graph(p, launches, max(steps, 3))
        reps = launches * max(steps, 3)
    rf = roofline(prec, M, N, K, t)
    del p
    import torch
    torch.cuda.empty_cache()
    # warm: the same launches on one input set, which then stays in the
    # Infinity Cache (reported beside the cold figure, never instead of it)
    t_warm = None
    if copies > 1 and not eager:
        pw = Problem(prec, M, N, K, seed, 1, b_layout)
        t_warm = time_graph(pw, launches, max(steps, 3))
        del pw
        torch.cuda.empty_cache()
    unit = "TFLOP/s" if prec in ("f16", "w4a16") else "TOP/s"
    thr = 2.0 * M * N * K / t / 1e12
    if prec == "quantize":
        unit, thr = "GB/s", algorithmic_bytes(prec, M, N, K) / t / 1e9
    e = {"M": M, "N": N, "K": K, "us": round(t * 1e6, 3),
         "throughput": round(thr, 3), "unit": unit,
         "roofline_bound": rf["bound"], "roofline_frac": rf["frac"],
         "hbm_GBps_algorithmic": round(algorithmic_bytes(prec, M, N, K) / t / 1e9, 1),
         "input_copies": copies, "launches": reps,
         "timing": "eager launches" if eager else "hip graph replay"}
    if b_layout != "nk":
        e["b_layout"] = b_layout
    if t_warm is not None:
        e["us_warm"] = round(t_warm * 1e6, 3)
    return e


def annotate_w4a16(entries, steps):
    """W4A16 entries gain the cold-read floor of their bytes (the fastest
    plain streaming read, measured in the same run) and, when the committed
    kernel-trace summary matches the kernel source, the kernels' own
    durations per call beside the event-timed figure (which includes the
    dispatch gaps of the replayed graph)."""
    trace = w4a16_kernel_trace()
    for e in entries:
        nbytes = algorithmic_bytes("w4a16", e["M"], e["N"], e["K"])
        t_floor, lpl = read_floor(nbytes, steps)
        e["cold_read_floor_us"] = round(t_floor * 1e6, 3)
        e["cold_read_floor_GBps"] = round(nbytes / t_floor / 1e9, 1)
        e["cold_read_floor_loads_per_lane"] = lpl
        e["us_over_floor"] = round(e["us"] / (t_floor * 1e6), 3)
        e["roofline_from"] = "hip events around graph replays (dispatch gaps included)"
        if trace and e["M"] in trace:
            t_k = trace[e["M"]] * 1e-9
            e["kernel_trace_us"] = round(t_k * 1e6, 3)
            e["kernel_trace_roofline_frac"] = roofline("w4a16", e["M"], e["N"], e["K"], t_k)["frac"]
            e["kernel_trace_over_floor"] = round(t_k / t_floor, 3)
            e["kernel_trace_source"] = "profiles/w4a16_4096_kernel_trace.md"
        else:
            e["kernel_trace_us"] = None
    return entries


# ------------------------------------------------------------------ CPU baseline

def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def _oracle_rows(prec, n, seed, budget_s):
    """The oracle on the first r rows of an n^3 problem against all of B, r
    calibrated so the timed call takes about budget_s: (rows, seconds)."""
    import oracle
    from precision_dense_gemm_tiled_amd import inputs

    def gen_a(rows):
        return inputs.gemm_problem(prec, rows, 1, n, seed)[0] if prec != "f16" else \
            inputs.f16_uniform(seed, 0, rows, n, -1.0, 1.0)

    if prec == "f16":
        B = inputs.f16_uniform(seed, n * n, n, n, -1.0, 1.0)
    else:
        B = inputs.gemm_problem(prec, n, n, n, seed)[1]
    run = {"f16": lambda a: oracle.gemm_f16(a, B), "i8": lambda a: oracle.gemm_i8(a, B),
           "i4": lambda a: oracle.gemm_i4(a, B, n)}[prec]
    run(gen_a(8))                                  # thread pool, page faults
    t_cal = []
    for r in (8, 24):
        a = gen_a(r)
        t0 = time.perf_counter()
        run(a)
        t_cal.append(time.perf_counter() - t0)
    per_row = max((t_cal[1] - t_cal[0]) / 16, 1e-7)
    fixed = max(t_cal[0] - 8 * per_row, 0.0)
    rows = int(max(8, min(n, (budget_s - fixed) / per_row)))
    a = gen_a(rows)
    t0 = time.perf_counter()
    run(a)
    return rows, time.perf_counter() - t0


def cpu_baseline(budget_s=6.0):
    """The CPU oracle (test infrastructure, untuned) timed on the host cores
    beside the GPU figures, in the same run. value: the FP16 8192^3 problem on
    a row sample (all of B against the first r rows of A, r calibrated to
    about budget_s). per_config: every workload on a bounded sample (INT8 and
    INT4 8192^3 row samples, W4A16 4096 x 4096 at M = 1, 16, 128 in full),
    plus single-thread timings at N = 512 (whole problems) and 2048 (row
    samples) as a per-core figure. GOPS = 2 M N K / t over the part timed."""
    import oracle
    from precision_dense_gemm_tiled_amd import inputs
    if not os.path.exists(oracle._LIB_PATH):
        from oracle import build
        build.build()
    threads = oracle.threads()
    per = []

    def entry(name, prec, M, N, K, dt, nthreads, sampled):
        per.append({"config": name, "prec": prec, "M": M, "N": N, "K": K, "seconds": round(dt, 4),
                    "GOPS": round(2.0 * M * N * K / dt / 1e9, 3), "threads": nthreads, "sampled": sampled})

    n = 8192
    rows, dt = _oracle_rows("f16", n, inputs.config_seed(CONFIG_INDEX["f16"], n), budget_s)
    entry(f"fp16 {n}^3", "f16", rows, n, n, dt, threads, f"first {rows} of {n} rows")
    head = {"value": round(2.0 * rows * n * n / dt / 1e12, 6), "unit": "TFLOP/s", "cores": threads,
            "kind": "oracle",
            "sample": f"FP16 8192^3 problem: first {rows} rows of A against all of B "
                      f"({rows}x8192x8192, fp64 oracle including the binary16 decode of A and B), "
                      f"{dt:.1f} s"}
    for prec, budget in (("i8", 2.0), ("i4", 3.0)):
        rows, dt = _oracle_rows(prec, n, inputs.config_seed(CONFIG_INDEX[prec], n), budget)
        entry(f"{prec} {n}^3", prec, rows, n, n, dt, threads, f"first {rows} of {n} rows")
    for m in W4A16_M:
        X, W, S = inputs.w4a16_problem(m, W4A16_NK, W4A16_NK, W4A16_G, inputs.config_seed(CONFIG_INDEX["w4a16"], m))
        t0 = time.perf_counter()
        oracle.gemm_w4a16(X, W, S, W4A16_NK, W4A16_G)
        entry(f"w4a16 M={m}", "w4a16", m, W4A16_NK, W4A16_NK, time.perf_counter() - t0, threads, "whole problem")
    # per core: one thread
    oracle.set_threads(1)
    try:
        for prec in ("i8", "f16", "i4"):
            idx = CONFIG_INDEX["i8_512"] if prec == "i8" else CONFIG_INDEX[prec]
            A, B = inputs.gemm_problem(prec, 512, 512, 512, inputs.config_seed(idx, 512))
            t0 = time.perf_counter()
            {"i8": lambda: oracle.gemm_i8(A, B), "f16": lambda: oracle.gemm_f16(A, B),
             "i4": lambda: oracle.gemm_i4(A, B, 512)}[prec]()
            entry(f"{prec} 512^3, one thread", prec, 512, 512, 512, time.perf_counter() - t0, 1, "whole problem")
        for prec in ("i8", "f16"):
            rows, dt = _oracle_rows(prec, 2048, inputs.config_seed(CONFIG_INDEX[prec], 2048), 1.0)
            entry(f"{prec} 2048^3, one thread", prec, rows, 2048, 2048, dt, 1, f"first {rows} of 2048 rows")
    finally:
        oracle.set_threads(threads)
    head["per_config"] = per
    head["cpu_model"] = cpu_model()
    head["hardware_concurrency"] = os.cpu_count()
    head["omp_threads"] = threads
    return head


# ------------------------------------------------------------------ main

def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    # ~50 ms of sustained MFMA load before the timed steps: with 5 ms the clock
    # has not settled and FP16 8192 reads about 8 % low
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--settle-ms", type=float, default=150.0,
                    help="untimed launches of the headline GEMM for about this long before its warm-up steps, "
                         "so that the timed steps run at the clock the GPU sustains under this load (the clock "
                         "ramps up over ~0.1 s of MFMA work); 0 disables")
    ap.add_argument("--no-sweep", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only", choices=["f16", "i8", "i4", "w4a16", "w4a4", "w4a4lr", "quantize"], default=None,
                    help="time only this precision's sweep (no headline line)")
    ap.add_argument("--sizes", type=str, default=None,
                    help="with --only: comma-separated sizes (N, or M for w4a16)")
    ap.add_argument("--b-layout", choices=["nk", "kn"], default="nk",
                    help="with --only f16/i8/i4: B stored N x K (default) or K x N (the "
                         "transposed-B control, mpgemm_run_*_kn)")
    ap.add_argument("--eager", action="store_true",
                    help="time the sweep with eager launches instead of HIP graph replay")
    ap.add_argument("--launches", type=int, default=None,
                    help="with --only: launches per timed batch (default: enough for ~20 ms); "
                         "counter collection uses a few eager launches")
    ap.add_argument("--no-floor", action="store_true",
                    help="with --only w4a16: skip the cold-read floor measurement")
    ap.add_argument("--calib-copy", action="store_true",
                    help="first run one plain 256 MiB device copy (reference dispatch for "
                         "scaling the FETCH_SIZE / WRITE_SIZE counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: --gpus {args.gpus} is not supported "
              "(the library has no multi-GPU path)", file=sys.stderr)
        sys.exit(2)

    import torch
    import precision_dense_gemm_tiled_amd as mp
    from precision_dense_gemm_tiled_amd import inputs
    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a gfx950 GPU")
    mp.lib()
    torch.cuda.set_device(0)

    if args.calib_copy:
        src = torch.empty(256 << 20, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        torch.cuda.empty_cache()
        log("[bench] calibration copy of 268435456 bytes done")

    if args.only:
        precs = [args.only]
        out = {}
        for prec in precs:
            sizes = {"w4a16": W4A16_M, "quantize": QUANT_NK, "w4a4": W4A4_SIZES, "w4a4lr": W4A4_SIZES}.get(prec, SQUARE_SIZES)
            if args.sizes:
                sizes = [int(v) for v in args.sizes.split(",")]
            out[prec] = []
            for s in sizes:
                M, N, K = (s, W4A16_NK, W4A16_NK) if prec == "w4a16" else ((1, s, s) if prec == "quantize" else (s, s, s))
                seed = inputs.config_seed(CONFIG_INDEX[prec], s)
                layout = args.b_layout if prec in ("f16", "i8", "i4") else "nk"
                e = sweep_entry(prec, M, N, K, seed, args.steps, args.warmup, args.eager, layout,
                                args.launches)
                log(prec, e)
                out[prec].append(e)
            if prec == "w4a16" and not args.no_floor:
                annotate_w4a16(out[prec], args.steps)
        print(json.dumps(out))
        return

    # The per-precision sweep runs first, so the headline steps are timed on a
    # GPU under sustained load (the clock has settled), then the headline's
    # own W warm-up steps and K timed steps.
    n = 8192
    log(f"[bench] FP16 {n}^3: generating inputs")
    head = Problem("f16", n, n, n, inputs.config_seed(CONFIG_INDEX["f16"], n))
    extra = {}
    if not args.no_sweep:
        per = {}
        for prec in ["f16", "i8", "i4", "w4a16", "w4a4", "w4a4lr", "quantize"]:
            sizes = {"w4a16": W4A16_M, "quantize": QUANT_NK, "w4a4": W4A4_SIZES, "w4a4lr": W4A4_SIZES}.get(prec, SQUARE_SIZES)
            per[prec] = []
            for s in sizes:
                M, N, K = (s, W4A16_NK, W4A16_NK) if prec == "w4a16" else ((1, s, s) if prec == "quantize" else (s, s, s))
                idx = CONFIG_INDEX["i8_512"] if (prec == "i8" and s == 512) else CONFIG_INDEX[prec]
                e = sweep_entry(prec, M, N, K, inputs.config_seed(idx, s), 5, 2, args.eager)
                warm = f", warm {e['us_warm']} us" if "us_warm" in e else ""
                log(f"[bench] {prec} {M}x{N}x{K}: {e['us']} us, {e['throughput']} {e['unit']}, "
                    f"{e['roofline_bound']} frac {e['roofline_frac']}{warm}")
                per[prec].append(e)
            if prec == "w4a16":
                annotate_w4a16(per[prec], 5)
                for e in per[prec]:
                    log(f"[bench] w4a16 M={e['M']}: cold-read floor {e['cold_read_floor_us']} us, "
                        f"call {e['us']} us ({e['us_over_floor']}x), kernel trace {e['kernel_trace_us']} us")
        extra["per_precision"] = per

        # one pass of the whole hot path at the largest sizes
        probs = [Problem(p, n, n, n, inputs.config_seed(CONFIG_INDEX[p], n)) for p in ["f16", "i8", "i4"]]
        probs += [Problem("w4a16", m, W4A16_NK, W4A16_NK, inputs.config_seed(4, m)) for m in W4A16_M]

        def hot_path():
            for p in probs:
                p.launch()
        t_hp = time_launches(hot_path, 5, 1)
        ops = sum(2.0 * p.M * p.N * p.K for p in probs)
        extra["hot_path"] = {"ops_per_pass": ops, "ms_per_pass": round(t_hp * 1e3, 4),
                             "mixed_TOPS": round(ops / t_hp / 1e12, 3),
                             "ops": "f16/i8/i4 8192^3 + w4a16 4096x4096 M=1,16,128"}
        del probs
        torch.cuda.empty_cache()

    # ---- headline: FP16 8192^3, inputs resident, W warm-up + K timed steps.
    # First about settle_ms of untimed launches of the same GEMM: after the
    # sweep's small and memory-bound entries the clock has dropped, and with
    # a few warm-up steps the timed steps would measure its ramp back up.
    settled = 0
    if args.settle_ms > 0:
        t_settle = time.time()
        while (time.time() - t_settle) * 1e3 < args.settle_ms:
            for _ in range(8):
                head.launch()
            torch.cuda.synchronize()
            settled += 8
        log(f"[bench] FP16 {n}^3: {settled} untimed launches to settle the clock")
    log(f"[bench] FP16 {n}^3: {args.warmup} warm-up + {args.steps} timed steps")
    t_step = time_launches(head.launch, args.steps, args.warmup)
    flops = 2.0 * n * n * n
    value = flops / t_step / 1e12
    rf = roofline("f16", n, n, n, t_step)
    del head
    torch.cuda.empty_cache()
    log(f"[bench] FP16 {n}^3: {t_step * 1e3:.3f} ms/step, {value:.1f} TFLOP/s")

    result = {
        "metric": "TFLOPS/TOPS per precision at N=512..8192 + % of MFMA/HBM roofline",
        "value": round(value, 3), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(t_step * 1e3, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f16", "data": "synthetic",
        "config": {"workload": "fp16_gemm_square_n8192", "M": n, "N": n, "K": n,
                   "A": "fp16 U[-1,1) 8192x8192 row-major", "B": "fp16 U[-1,1) 8192x8192 stored NxK",
                   "C": "fp32 8192x8192", "parallelism": "single_gpu",
                   "timed_after": ("the per-precision sweep" if not args.no_sweep else "process start") +
                                  (f", then {settled} untimed launches of this GEMM ({args.settle_ms:.0f} ms)"
                                   if settled else "")},
        "roofline": {"bound": rf["bound"], "achieved": rf["achieved"], "peak": rf["peak"],
                     "unit": rf["unit"], "frac": rf["frac"], "traffic": measured_traffic(),
                     "kernel": "mpg::gemm_tile_kernel<f16, 256x256 tile, BK 128 B, 2-stage LDS ring>",
                     "algorithmic": f"2*M*N*K = {flops:.4e} flop per launch; compulsory bytes "
                                    f"{algorithmic_bytes('f16', n, n, n)} (A + B read once, C written once)"},
    }
    result.update(extra)

    if not args.no_cpu_baseline:
        log("[bench] CPU oracle baseline")
        result["cpu_baseline"] = cpu_baseline()
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
