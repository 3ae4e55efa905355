"""Benchmark of the MatMul-family hot path on one MI355X.

One step = one call of each of the five workloads through the C ABI, in order,
on one stream (all inputs resident in HBM before timing starts):
  1. Gemm fp32   transA=transB=1, A[48,64] B[32,48] C[1,32], alpha .75 beta 1.5
  2. MatMul bf16 A[8,1,512,1024] x B[1,16,1024,768]
  3. Gemm bf16   8192^3, transB=1, C[8192]
  4. QLinearMatMul int8 4096^3, per-row a / per-column b parameters
  5. GroupedMatMul bf16, M=16384 K=4096 N=2048 G=64 S=8
`value` is the step's algorithmic operations (2*M*N*K per product; int8
multiply-adds counted like flops) divided by the step time.  Each workload is
also timed on its own (median of HIP-event intervals around its call) and
reported against the MI355X dense MFMA peak of its type under `per_config`;
`cold_ms` there is the median of calls issued right after a 512 MiB write that
evicts the last-level cache (operands start in HBM only), and `graph_ms` the
per-call time when the calls are replayed from a captured HIP graph (no host
launch work between kernels; `graph_ms_per_step` likewise for a whole step).  `next_rows` times
workloads outside the step the same way (GroupedMatMul over int8 weights with
the dequantisation fused, an fp64 Gemm, uint8 QLinearMatMul, decode-like
skinny Gemms against the HBM peak, warm and, as `hbm_ms`, cycling over copies
of B larger than the last-level cache); they are not part of `value`.

Usage: python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu] [--only NAME]
       python bench.py --copy-calibration      (1 GiB device-to-device copies, for
                                                 scaling the L2 byte counters)

`roofline.traffic` comes from profiles/traffic_grouped_bf16_moe.txt (FETCH_SIZE and
WRITE_SIZE of the grouped kernel, scaled by the same counters on a plain copy): bytes
between the XCDs' L2 caches and the memory side, last-level-cache hits included (HBM
bytes alone are not observable with the profiler's counters); it is null when the
kernel sources differ from the ones the counters were taken on.
"""
import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "TFLOP/s (int8: TOPS) per config and % of MI355X dense MFMA peak, 1 GPU"
UNIT = "TFLOP/s (int8: TOPS)"
# MI355X datasheet dense peaks (TFLOP/s or TOPS) and HBM bandwidth (GB/s)
PEAK = {"bf16": 2516.6, "f16": 2516.6, "f32": 157.3, "int8": 5033.2, "f64": 78.6}
HBM_GBS = 8000.0


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def build_workloads(torch, synth, dev, only=None):
    """Host draws -> device tensors.  Returns name -> dict(run=callable, ops, dtype, bytes, ...)."""
    W = {}

    def want(n):
        return only is None or n in only

    if want("gemm_f32_64x32x48"):
        c = synth.gemm_f32_64x32x48()
        d = dict(A=dev(c["A"]), B=dev(c["B"]), C=dev(c["C"]))
        d["Y"] = torch.empty((64, 32), dtype=torch.float32, device="cuda")
        W["gemm_f32_64x32x48"] = dict(host=c, dev=d, ops=2 * 64 * 32 * 48, dtype="f32",
                                      bytes=(48 * 64 + 32 * 48 + 32 + 64 * 32) * 4)
    if want("matmul_bf16_bcast"):
        c = synth.matmul_bf16_bcast()
        d = dict(A=dev(c["A"], "bf16"), B=dev(c["B"], "bf16"))
        d["Y"] = torch.empty((8, 16, 512, 768), dtype=torch.bfloat16, device="cuda")
        W["matmul_bf16_bcast"] = dict(host=c, dev=d, ops=2 * 128 * 512 * 768 * 1024, dtype="bf16",
                                      bytes=(8 * 512 * 1024 + 16 * 1024 * 768 + 128 * 512 * 768) * 2)
    if want("gemm_bf16_8192"):
        c = synth.gemm_bf16_8192()
        d = dict(A=dev(c["A"], "bf16"), B=dev(c["B"], "bf16"), C=dev(c["C"], "bf16"))
        d["Y"] = torch.empty((8192, 8192), dtype=torch.bfloat16, device="cuda")
        W["gemm_bf16_8192"] = dict(host=c, dev=d, ops=2 * 8192 ** 3, dtype="bf16",
                                   bytes=(3 * 8192 * 8192 + 8192) * 2)
    if want("qlinear_i8_4096"):
        c = synth.qlinear_i8_4096()
        d = {k: dev(c[k]) for k in ("a", "a_scale", "a_zero_point", "b", "b_scale", "b_zero_point", "y_scale",
                                    "y_zero_point")}
        d["y"] = torch.empty((4096, 4096), dtype=torch.int8, device="cuda")
        W["qlinear_i8_4096"] = dict(host=c, dev=d, ops=2 * 4096 ** 3, dtype="int8",
                                    bytes=3 * 4096 * 4096 + 4096 * 10)
    if want("grouped_bf16_moe"):
        c = synth.grouped_bf16_moe()
        d = dict(input=dev(c["input"], "bf16"), weights=dev(c["weights"], "bf16"), idx=dev(c["group_indices"]),
                 bias=dev(c["bias"], "bf16"))
        d["out"] = torch.empty((16384, 8, 2048), dtype=torch.bfloat16, device="cuda")
        W["grouped_bf16_moe"] = dict(host=c, dev=d, ops=2 * 16384 * 8 * 4096 * 2048, dtype="bf16",
                                     bytes=(16384 * 4096 + 64 * 4096 * 2048 + 64 * 2048 + 16384 * 8 * 2048) * 2
                                     + 16384 * 8 * 4)
    return W


def make_runner(om, name, w, torch):
    d, c = w["dev"], w["host"]
    if name == "gemm_f32_64x32x48":
        return lambda: om.gemm(d["A"], d["B"], d["C"], c["alpha"], c["beta"], 1, 1, d["Y"])
    if name == "matmul_bf16_bcast":
        return lambda: om.matmul(d["A"], d["B"], d["Y"])
    if name == "gemm_bf16_8192":
        return lambda: om.gemm(d["A"], d["B"], d["C"], 1.0, 1.0, 0, 1, d["Y"])
    if name == "qlinear_i8_4096":
        return lambda: om.qlinear_matmul(d["a"], d["a_scale"], d["a_zero_point"], d["b"], d["b_scale"],
                                         d["b_zero_point"], d["y_scale"], d["y_zero_point"], d["y"])
    if name == "grouped_bf16_moe":
        ws = torch.empty(om.grouped_matmul_workspace_size(16384, 8, 64), dtype=torch.uint8, device="cuda")
        return lambda: om.grouped_matmul(d["input"], d["weights"], d["idx"], d["bias"], d["out"], ws)
    raise KeyError(name)


def time_each(torch, fn, reps):
    """Median of HIP-event intervals around single calls, on torch's current stream (the call's stream)."""
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for s, e in evs:
        s.record()
        fn()
        e.record()
    torch.cuda.synchronize()
    ms = sorted(s.elapsed_time(e) for s, e in evs)
    return ms[len(ms) // 2], ms


def capture(torch, fn, calls):
    """A HIP graph of `calls` back-to-back calls of fn (captured on torch's graph
    stream after one eager call there, as torch requires)."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(calls):
            fn()
    torch.cuda.synchronize()
    return g


def time_graph(torch, g, calls, reps):
    """Milliseconds per call: `reps` replays of a graph of `calls` calls between two
    HIP events (no host launch work between the kernels)."""
    g.replay()
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(reps):
        g.replay()
    e.record()
    torch.cuda.synchronize()
    return s.elapsed_time(e) / (reps * calls)


def next_rows(torch, om, synth, dev, reps):
    """Workloads beyond the five-workload step, timed the same way but not part
    of `value`: GroupedMatMul over int8 weights with the dequantisation fused
    (the grouped workload's shapes, block 128)."""
    c = synth.grouped_dq_int8_moe()
    M, S = c["group_indices"].shape
    G, K, N = c["qweights"].shape
    d = dict(input=dev(c["input"], "bf16"), q=dev(c["qweights"]), scale=dev(c["scale"], "bf16"),
             zp=dev(c["zero_point"]), idx=dev(c["group_indices"]), bias=dev(c["bias"], "bf16"))
    out = torch.empty((M, S, N), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(om.grouped_matmul_workspace_size(M, S, G), dtype=torch.uint8, device="cuda")
    fn = lambda: om.grouped_matmul_dequant(d["input"], d["q"], d["scale"], d["zp"], c["block_size"], d["idx"],
                                           d["bias"], out, ws)
    for _ in range(3):
        fn()
    torch.cuda.synchronize()
    med, _ = time_each(torch, fn, reps)
    ops = 2 * M * S * K * N
    byts = M * K * 2 + G * K * N + c["scale"].size * 2 + c["zero_point"].size + G * N * 2 + M * S * N * 2 + M * S * 4
    rate = ops / (med * 1e-3) / 1e12
    log("%-20s %9.4f ms  %8.1f T/s  %5.1f%% of bf16 peak (not in the step)" % ("grouped_dq_int8_moe", med, rate,
                                                                               100 * rate / PEAK["bf16"]))
    rows = [dict(workload="grouped_dq_int8_moe", desc=synth.GROUPED_DQ_WORKLOAD, dtype="bf16 x int8-dequant",
                 ms=round(med, 4), tflops=round(rate, 2), frac_peak=round(rate / PEAK["bf16"], 4),
                 hbm_gbs=round(byts / (med * 1e-3) / 1e9, 1))]
    del d, out, ws
    # fp32 / fp64 GroupedMatMul on the matrix cores (4096 tokens x 4 of 16 experts, K = N = 1024)
    for dt in ("f32", "f64"):
        c = synth.grouped_fp_moe(dt)
        M, S = c["group_indices"].shape
        G, K, N = c["weights"].shape
        d = dict(input=dev(c["input"]), w=dev(c["weights"]), idx=dev(c["group_indices"]), bias=dev(c["bias"]))
        out = torch.empty((M, S, N), dtype=torch.float64 if dt == "f64" else torch.float32, device="cuda")
        ws = torch.empty(om.grouped_matmul_workspace_size(M, S, G), dtype=torch.uint8, device="cuda")
        fn = lambda: om.grouped_matmul(d["input"], d["w"], d["idx"], d["bias"], out, ws)
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        med, _ = time_each(torch, fn, reps)
        es = 8 if dt == "f64" else 4
        rate = 2 * M * S * K * N / (med * 1e-3) / 1e12
        name = "grouped_%s_moe" % dt
        log("%-20s %9.4f ms  %8.1f T/s  %5.1f%% of %s peak (not in the step)" % (name, med, rate,
                                                                               100 * rate / PEAK[dt], dt))
        rows.append(dict(workload=name, desc=synth.GROUPED_FP_WORKLOAD % dt, dtype=dt, ms=round(med, 4),
                         tflops=round(rate, 2), frac_peak=round(rate / PEAK[dt], 4),
                         hbm_gbs=round(((M * K + G * K * N + G * N + M * S * N) * es + M * S * 4) / (med * 1e-3)
                                       / 1e9, 1)))
        del d, out, ws
    # fp64 Gemm (MFMA f64), 4096^3, N(0,1) operands, C[4096], alpha=beta=1
    n = 4096
    rng = np.random.default_rng(6)
    A64 = torch.from_numpy(rng.standard_normal((n, n))).cuda()
    B64 = torch.from_numpy(rng.standard_normal((n, n))).cuda()
    C64 = torch.from_numpy(rng.standard_normal(n)).cuda()
    Y64 = torch.empty((n, n), dtype=torch.float64, device="cuda")
    fn = lambda: om.gemm(A64, B64, C64, 1.0, 1.0, 0, 1, Y64)
    fn()
    torch.cuda.synchronize()
    med, _ = time_each(torch, fn, max(5, reps // 3))
    rate = 2 * n ** 3 / (med * 1e-3) / 1e12
    log("%-20s %9.4f ms  %8.1f T/s  %5.1f%% of f64 peak (not in the step)" % ("gemm_f64_4096", med, rate,
                                                                              100 * rate / PEAK["f64"]))
    rows.append(dict(workload="gemm_f64_4096", desc="Gemm fp64 4096^3, transB=1, C[4096], alpha=beta=1, N(0,1), seed 6",
                     dtype="f64", ms=round(med, 4), tflops=round(rate, 2), frac_peak=round(rate / PEAK["f64"], 4),
                     hbm_gbs=round((3 * n * n + n) * 8 / (med * 1e-3) / 1e9, 1)))
    del A64, B64, C64, Y64
    # QLinearMatMul with uint8 operands and output at the int8 workload's size
    q = 4096
    a8 = torch.from_numpy(rng.integers(0, 256, (q, q)).astype(np.uint8)).cuda()
    b8 = torch.from_numpy(rng.integers(0, 256, (q, q)).astype(np.uint8)).cuda()
    asc = torch.from_numpy(synth.uniform(rng, (q, 1), 0.002, 0.01)).cuda()
    bsc = torch.from_numpy(synth.uniform(rng, (1, q), 0.002, 0.01)).cuda()
    az = torch.from_numpy(rng.integers(112, 145, (q, 1)).astype(np.uint8)).cuda()
    bz = torch.from_numpy(rng.integers(112, 145, (1, q)).astype(np.uint8)).cuda()
    ys = torch.tensor(0.05, device="cuda")
    yz = torch.tensor(128, dtype=torch.uint8, device="cuda")
    y8 = torch.empty((q, q), dtype=torch.uint8, device="cuda")
    fn = lambda: om.qlinear_matmul(a8, asc, az, b8, bsc, bz, ys, yz, y8)
    fn()
    torch.cuda.synchronize()
    med, _ = time_each(torch, fn, reps)
    rate = 2 * q ** 3 / (med * 1e-3) / 1e12
    log("%-20s %9.4f ms  %8.1f T/s  %5.1f%% of int8 peak (not in the step)" % ("qlinear_u8_4096", med, rate,
                                                                               100 * rate / PEAK["int8"]))
    rows.append(dict(workload="qlinear_u8_4096", desc="QLinearMatMul uint8 x uint8 -> uint8 4096^3, per-row / per-column "
                     "scales U(0.002,0.01), zero points U[112,144], y_scale 0.05, y_zp 128, seed 6", dtype="uint8",
                     ms=round(med, 4), tflops=round(rate, 2), frac_peak=round(rate / PEAK["int8"], 4),
                     hbm_gbs=round(3 * q * q / (med * 1e-3) / 1e9, 1)))
    del a8, b8, y8
    # decode-like skinny Gemm (B-streaming kernels): HBM-bound, reported against the
    # HBM peak. B (128 MiB) fits the 256 MB last-level cache, so repeated calls are
    # served partly from it; hbm_ms times the same calls cycling over 4 copies of B
    # (512 MiB), so that each call's B comes from HBM (a cache-evicting write before
    # the call, as cold_ms does elsewhere, would add that write's write-backs)
    for M, tB in ((1, 1), (16, 1), (1, 0)):
        N = K = 8192
        A = torch.from_numpy(synth.store(synth.normal(rng, (M, K)), "bf16").view(np.int16)).cuda().view(torch.bfloat16)
        B = torch.from_numpy(synth.store(synth.normal(rng, (N, K), 0.02), "bf16").view(np.int16)).cuda().view(
            torch.bfloat16)
        Y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
        fn = lambda: om.gemm(A, B, None, 1.0, 0.0, 0, tB, Y)
        fn()
        torch.cuda.synchronize()
        med, _ = time_each(torch, fn, reps)
        byts = 2 * (M * K + N * K + M * N)
        gbs = byts / (med * 1e-3) / 1e9
        name = "gemm_bf16_skinny_m%d_%s" % (M, "nk" if tB else "kn")
        row = dict(workload=name,
                   desc="Gemm bf16 M=%d N=K=8192, B stored %s (transB=%d), no C, seed 6"
                   % (M, "(N, K)" if tB else "(K, N)", tB), dtype="bf16",
                   ms=round(med, 4), tflops=round(2 * M * N * K / (med * 1e-3) / 1e12, 2),
                   hbm_gbs=round(gbs, 1), frac_hbm=round(gbs / HBM_GBS, 4))
        Bs = [B] + [B.clone() for _ in range(3)]
        nxt = [0]

        def fn_hbm():
            nxt[0] = (nxt[0] + 1) % len(Bs)
            om.gemm(A, Bs[nxt[0]], None, 1.0, 0.0, 0, tB, Y)
        hms, _ = time_each(torch, fn_hbm, max(reps, 8))
        row.update(hbm_ms=round(hms, 4), hbm_frac_hbm=round(byts / (hms * 1e-3) / 1e9 / HBM_GBS, 4))
        log("%-20s %9.4f ms  %8.1f GB/s  %5.1f%% of HBM peak; B from HBM %.4f ms, %.1f%% (not in the step)"
            % (name, med, gbs, 100 * gbs / HBM_GBS, hms, 100 * row["hbm_frac_hbm"]))
        rows.append(row)
        del Bs
    return rows


def time_cold(torch, fn, reps, flush):
    """Median of HIP-event intervals around single calls, each issued right after a
    write of `flush` (larger than the 256 MB last-level cache), so the call starts
    with none of its operands cached."""
    ms = []
    for i in range(reps):
        flush.fill_(i & 0xFF)
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        fn()
        e.record()
        torch.cuda.synchronize()
        ms.append(s.elapsed_time(e))
    ms.sort()
    return ms[len(ms) // 2]


def kernel_source_hash():
    """sha256 over the kernel sources (csrc/*.hip, *.hpp): identifies the build the counters describe."""
    d = os.path.join(ROOT, "onnx_matmul_family_amd", "csrc")
    h = hashlib.sha256()
    for f in sorted(os.listdir(d)):
        if f.endswith((".hip", ".hpp")):
            with open(os.path.join(d, f), "rb") as fh:
                h.update(f.encode() + b"\0" + fh.read())
    return h.hexdigest()


def measured_traffic(kernel_key):
    """Bytes per launch between the XCDs' L2 caches and the memory side (FETCH_SIZE +
    WRITE_SIZE, scaled by the same counters on a plain copy) from the committed counter
    summary, or None if stale/missing.  The memory side includes the 256 MB last-level
    cache: no counter the profiler offers on this GPU separates its hits from HBM
    reads, so this is an upper bound on HBM traffic, not HBM traffic itself."""
    path = os.path.join(ROOT, "profiles", "traffic_%s.txt" % kernel_key)
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
    try:
        if kv.get("source_sha256") != kernel_source_hash():
            return None
        fetch = float(kv["fetch_kib_per_launch"]) * 1024 * float(kv["copy_fetch_factor"])
        write = float(kv["write_kib_per_launch"]) * 1024 * float(kv["copy_write_factor"])
        return fetch + write
    except (KeyError, ValueError):
        return None


def cpu_baseline(W, budget_s):
    """The oracle as it stands, timed on a bounded sample of each workload's outputs."""
    import oracle
    nth = oracle.threads()
    total_ops, total_t, parts = 0.0, 0.0, []
    per = budget_s / max(1, len(W))
    for name, w in W.items():
        c = w["host"]
        K = {"gemm_f32_64x32x48": 48, "matmul_bf16_bcast": 1024, "gemm_bf16_8192": 8192,
             "qlinear_i8_4096": 4096, "grouped_bf16_moe": 4096}[name]
        nout = w["ops"] // (2 * K)

        def call(sel):
            if name == "gemm_f32_64x32x48":
                return oracle.gemm(c["A"], c["B"], c["C"], c["alpha"], c["beta"], 1, 1, sel=sel)
            if name == "matmul_bf16_bcast":
                return oracle.matmul(c["A"], c["B"], dt="bf16", sel=sel)
            if name == "gemm_bf16_8192":
                return oracle.gemm(c["A"], c["B"], c["C"], 1.0, 1.0, 0, 1, dt="bf16", sel=sel)
            if name == "qlinear_i8_4096":
                return oracle.qlinear_matmul(*(c[k] for k in ("a", "a_scale", "a_zero_point", "b", "b_scale",
                                                              "b_zero_point", "y_scale", "y_zero_point")), sel=sel)
            return oracle.grouped_matmul(c["input"], c["weights"], c["group_indices"], c["bias"], dt="bf16",
                                         sel=sel)

        rng = np.random.default_rng(0)
        n = min(nout, 256)
        # grow the sample until it takes about a tenth of this workload's share,
        # then run the sample sized to fill the share, and time that run
        while n < nout:
            sel = rng.integers(0, nout, n).astype(np.int64)
            t0 = time.perf_counter()
            call(sel)
            dt = time.perf_counter() - t0
            if dt >= per * 0.1:
                break
            n = min(nout, n * 4)
        n = int(min(nout, max(1, n * per / max(dt, 1e-6)))) if n < nout else nout
        sel = rng.integers(0, nout, n).astype(np.int64)
        t0 = time.perf_counter()
        call(sel)
        dt = time.perf_counter() - t0
        total_ops += 2.0 * K * n
        total_t += dt
        parts.append("%s: %d outputs (%.2fs)" % (name, n, dt))
    return dict(value=total_ops / total_t / 1e12, unit=UNIT, cores=nth, kind="oracle",
                sample="random output elements of each workload, computed one by one: " + "; ".join(parts))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--reps", type=int, default=30, help="timed calls per workload for the per-config medians")
    ap.add_argument("--cold-reps", type=int, default=5,
                    help="calls per workload timed right after a 512 MiB cache-flush write (0: skip)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU-oracle baseline")
    ap.add_argument("--no-next", action="store_true",
                    help="skip the workloads outside the step (quantised experts), reported under next_rows")
    ap.add_argument("--cpu-budget", type=float, default=15.0, help="seconds of oracle work for the baseline")
    ap.add_argument("--no-graph", action="store_true", help="skip the HIP-graph replay timings")
    ap.add_argument("--only", default=None, help="comma-separated workload names")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run 1 GiB device-to-device copies (reference for the HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py: this library runs on one GPU only (no multi-GPU path); use --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    if args.copy_calibration:
        X = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        Z = torch.empty_like(X)
        for _ in range(max(1, args.steps)):
            Z.copy_(X)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration": {"bytes_read_per_copy": 1 << 30, "bytes_written_per_copy": 1 << 30,
                                               "copies": max(1, args.steps)}}))
        return
    from onnx_matmul_family_amd import _omm as om
    from onnx_matmul_family_amd import synth
    from onnx_matmul_family_amd.hostdev import dev

    assert torch.cuda.is_available(), "bench needs a GPU"
    om.lib()
    only = set(args.only.split(",")) if args.only else None
    t0 = time.time()
    W = build_workloads(torch, synth, dev, only)
    torch.cuda.synchronize()
    log("inputs ready in %.1fs" % (time.time() - t0))
    runs = {n: make_runner(om, n, w, torch) for n, w in W.items()}

    def step():
        for fn in runs.values():
            fn()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    step_s = (time.perf_counter() - t0) / args.steps
    total_ops = sum(w["ops"] for w in W.values())
    log("step %.3f ms" % (step_s * 1e3))

    per = []
    flush = torch.empty(512 << 20, dtype=torch.uint8, device="cuda") if args.cold_reps > 0 else None
    for n, fn in runs.items():
        med, _ = time_each(torch, fn, args.reps)
        w = W[n]
        rate = w["ops"] / (med * 1e-3) / 1e12
        per.append(dict(workload=n, dtype=w["dtype"], ms=round(med, 4), tflops=round(rate, 2),
                        frac_peak=round(rate / PEAK[w["dtype"]], 4),
                        hbm_gbs=round(w["bytes"] / (med * 1e-3) / 1e9, 1)))
        if flush is not None:
            per[-1]["cold_ms"] = round(time_cold(torch, fn, args.cold_reps, flush), 4)
        log("%-20s %9.4f ms  %8.1f T/s  %5.1f%% of %s peak" % (n, med, rate, 100 * rate / PEAK[w["dtype"]],
                                                               w["dtype"]))

    # the same calls replayed from HIP graphs: per-call time without the host's
    # launch work between kernels (what a captured serving loop sees); one graph
    # per workload holds enough calls to fill about 0.2 ms
    if not args.no_graph:
        for p in per:
            calls = max(1, int(0.2 / max(p["ms"], 1e-3)))
            g = capture(torch, runs[p["workload"]], calls)
            p["graph_ms"] = round(time_graph(torch, g, calls, max(3, args.reps // calls)), 4)
            del g
        g = capture(torch, step, 1)
        graph_step_ms = time_graph(torch, g, 1, args.steps)
        del g
        log("graph replay: step %.3f ms; per call %s" % (graph_step_ms, ", ".join(
            "%s %.4f" % (p["workload"], p["graph_ms"]) for p in per)))

    dom = max(per, key=lambda p: p["ms"])
    wd = W[dom["workload"]]
    ach = wd["ops"] / (dom["ms"] * 1e-3) / 1e12
    roof = dict(bound="mfma", achieved=round(ach, 2), peak=PEAK[wd["dtype"]], unit="TFLOP/s",
                frac=round(ach / PEAK[wd["dtype"]], 4), traffic=measured_traffic(dom["workload"]),
                kernel=dom["workload"], launch_ms=dom["ms"])

    out = {
        "metric": METRIC, "value": round(total_ops / step_s / 1e12, 2), "unit": UNIT, "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(step_s * 1e3, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16/int8/f32",
        "data": "synthetic (seeded numpy draws with the specified shapes and distributions)",
        "config": {"workload": "onnx_matmul_family five-workload step: " + ", ".join(W.keys()),
                   "ops_per_step": total_ops},
        "roofline": roof, "per_config": per,
    }
    if not args.no_graph:
        out["graph_ms_per_step"] = round(graph_step_ms, 4)
    if not args.no_next and only is None:
        out["next_rows"] = next_rows(torch, om, synth, dev, args.reps)
    if not args.no_cpu:
        log("timing the CPU oracle baseline ...")
        out["cpu_baseline"] = cpu_baseline(W, args.cpu_budget)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
