#!/usr/bin/env python3
"""Benchmark of the packed-int4 weight GEMM library on one MI355X.

One step = one call of the hot path on the primary workload: qgemm_w4a16 with
the asymmetric delta term fused (a single kernel launch), decode shape M=16,
K=5120, N=17408, group 128, inputs already resident in HBM.  The packed
weights are rotated over enough copies (>= 512 MB in total) that they cannot
stay in the 256 MB last-level cache between calls, so the weight reads are HBM
reads.

Prints ONE JSON line on stdout:
  value      TFLOP/s (2*M*N*K per call) of the primary workload
  roofline   the primary kernel against the HBM roofline: algorithmic weight
             bytes (0.5 B per code + 2 B scale + 2 B delta per group and
             column) per launch / average launch duration (HIP events on the
             launch stream over the timed region)
  cpu_baseline  the CPU oracle timed on this host on the same workload
  achievable what this GPU sustains in the same run (an HBM streaming-read
             probe at the primary weight size and at 1 GiB, fp16 and int8 MFMA
             loop probes, best of a small launch-shape sweep each); every
             fraction is given against it beside the published peak
  cases      every other configuration measured the same way (decode shapes,
             mid-batch, prefill M=4096, grouped W4A8, the load-time pack)
Logs go to stderr.
"""
import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E, published
FP16_PEAK_TFLOPS = 2516.6       # dense fp16 MFMA (256 CU x 2.4 GHz x 4096 flop/clk)
INT8_PEAK_TOPS = 5033.2         # dense int8 MFMA
ROTATE_BYTES = 512 * 1024 * 1024


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--only-primary", action="store_true", help="skip the secondary cases")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-sample", action="store_true",
                   help="run the oracle on the first rows of the large workloads only")
    p.add_argument("--cpu-only", action="store_true",
                   help="only the CPU oracle baseline (no GPU needed)")
    p.add_argument("--cases", default="all", help="comma list of case names, or 'all'")
    p.add_argument("--eager", action="store_true", help="time plain launches instead of a graph replay")
    p.add_argument("--no-probes", action="store_true", help="skip the achievable-peak probes")
    p.add_argument("--calibrate-copy", action="store_true",
                   help="only run a 256 MiB device-to-device copy 20 times (counter calibration)")
    return p.parse_args()


def weight_bytes(K, N, g, asym):
    G = K // g
    return K * N // 2 + G * N * 2 * (2 if asym else 1)


def time_calls(fn, n_copies, steps, warmup, graph=True):
    """Average ms per call of fn(i) over `steps` calls, rotating i over the
    copies.  With graph=True the `steps` calls are captured once into a HIP
    graph and the timed region is one replay, so host-side launch overhead is
    not measured; HIP events are recorded on the stream the calls are launched
    on (torch's current stream, which the library uses)."""
    import torch
    for i in range(warmup):
        fn(i % n_copies)
    torch.cuda.synchronize()
    st = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    if not graph:
        e0.record(st)
        for i in range(steps):
            fn(i % n_copies)
        e1.record(st)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(steps):
            fn(i % n_copies)
    g.replay()                      # warm replay
    torch.cuda.synchronize()
    e0.record(st)
    g.replay()
    e1.record(st)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


GRAPH = True


def time_best(fn, n_copies, steps, warmup):
    """(ms, ms_graph, ms_eager) per call: the same `steps` calls timed as one
    graph replay and as eager launches; the faster is reported.  Graph replay
    removes the host launch cost, which dominates calls of a few us, but on
    this stack adds a per-node cost of its own (about 1.5 us at ~16 us calls),
    so eager launches win there.  ms_graph is None with --eager."""
    ms_graph = time_calls(fn, n_copies, steps, warmup, True) if GRAPH else None
    ms_eager = time_calls(fn, n_copies, steps, warmup if not GRAPH else 2, False)
    return (min(ms_graph, ms_eager) if ms_graph else ms_eager), ms_graph, ms_eager


def bench_w4a16(name, steps, warmup, flags=0, label=None, case=None):
    import numpy as np
    import torch

    import int4_weight_only_uint32_amd as qg
    import synth

    c = case if case is not None else synth.workload(name)
    M, K, N, g = c.M, c.K, c.N, c.g
    asym = c.z is not None
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    q, s = dev(c.q), dev(c.s)
    z = dev(c.z) if asym else None
    wb = weight_bytes(K, N, g, asym)
    # load-time pack, timed once per case (not part of the step)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    pw = qg.pack(q, s, z, g, fold=True)
    torch.cuda.synchronize()
    pack_ms = (time.perf_counter() - t0) * 1e3
    R = max(1, math.ceil(ROTATE_BYTES / wb))
    copies = [pw] + [qg.PackedWeight(w=pw.w.clone(), scale=pw.scale.clone(),
                                     delta=None if pw.delta is None else pw.delta.clone(),
                                     K=K, N=N, group_size=g) for _ in range(R - 1)]
    del q, s, z
    A = dev(c.A)
    C = torch.empty((M, N), dtype=torch.float16, device="cuda")
    # zero-filled once (its split-K counters must start at zero; every call
    # leaves them at zero)
    ws = None
    nws = qg.qg_workspace_bytes(qg.QG_OP_W4A16, M, N, K, g, 1, flags if asym else 0)
    if nws:
        ws = torch.zeros(nws, dtype=torch.uint8, device="cuda")

    def call(i):
        p = copies[i]
        qg.qgemm_w4a16(A, p.w, p.scale, p.delta, C, M, N, K, g, flags, ws)

    ms, ms_graph, ms_eager = time_best(call, R, steps, warmup)
    flops = 2.0 * M * N * K
    alg = wb + M * K * 2 + M * N * 2
    res = dict(name=label or name, M=M, K=K, N=N, group=g, mode="asym" if asym else "sym-fold",
               flags=flags, us_per_call=ms * 1e3, tflops=flops / (ms * 1e-3) / 1e12,
               weight_gbps=wb / (ms * 1e-3) / 1e9, total_alg_gbps=alg / (ms * 1e-3) / 1e9,
               weight_bytes=wb, rotated_copies=R, pack_ms_first_call=pack_ms,
               us_per_call_graph=ms_graph * 1e3 if ms_graph else None,
               us_per_call_eager=ms_eager * 1e3)
    res["pct_hbm_weight"] = 100.0 * res["weight_gbps"] / HBM_PEAK_GBPS
    res["pct_fp16_mfma"] = 100.0 * res["tflops"] / FP16_PEAK_TFLOPS
    del copies, A, C
    torch.cuda.empty_cache()
    return res, c


def bench_w4a8(name, steps, warmup, case=None):
    import numpy as np
    import torch

    import int4_weight_only_uint32_amd as qg
    import synth

    c = case if case is not None else synth.workload(name)
    asym = c.z is not None
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    packs = [qg.pack(dev(c.q[e]), dev(c.s[e]), dev(c.z[e]) if asym else None, c.g, fold=True)
             for e in range(c.E)]
    W = torch.stack([p.w for p in packs]).contiguous()
    S = torch.stack([p.scale for p in packs]).contiguous()
    D = torch.stack([p.delta for p in packs]).contiguous() if asym else None
    wb = c.E * weight_bytes(c.K, c.N, c.g, asym)
    R = max(1, math.ceil(ROTATE_BYTES / wb))
    Ws = [W] + [W.clone() for _ in range(R - 1)]
    Ss = [S] + [S.clone() for _ in range(R - 1)]
    Ds = [D] + [D.clone() for _ in range(R - 1)] if asym else [None] * R
    Aq, asc, off = dev(c.Aq), dev(c.a_scale), dev(c.offsets)
    C = torch.empty((c.M_total, c.N), dtype=torch.float16, device="cuda")
    mr = int(np.max(np.diff(c.offsets)))

    def call(i):
        qg.qgemm_w4a8(Aq, asc, Ws[i], Ss[i], off, c.E, c.M_total, mr, c.N, c.K, c.g, C,
                      w_delta=Ds[i])

    ms, ms_graph, ms_eager = time_best(call, R, steps, warmup)
    ops = 2.0 * c.M_total * c.N * c.K
    alg = wb + c.M_total * c.K + c.M_total * 4 + c.M_total * c.N * 2
    res = dict(name=name, E=c.E, rows_per_expert=mr, K=c.K, N=c.N, group=c.g,
               mode="asym" if asym else "sym",
               us_per_call=ms * 1e3, tops=ops / (ms * 1e-3) / 1e12,
               weight_gbps=wb / (ms * 1e-3) / 1e9, total_alg_gbps=alg / (ms * 1e-3) / 1e9,
               weight_bytes=wb, rotated_copies=R,
               us_per_call_graph=ms_graph * 1e3 if ms_graph else None,
               us_per_call_eager=ms_eager * 1e3)
    res["pct_hbm_weight"] = 100.0 * res["weight_gbps"] / HBM_PEAK_GBPS
    res["pct_int8_mfma"] = 100.0 * res["tops"] / INT8_PEAK_TOPS
    del Ws, Ss, Ds, W, S, D
    torch.cuda.empty_cache()
    return res


def _committed(name):
    """A committed rocprofv3 counter record under profiles/, if neither the
    kernel sources nor the build script have changed since it was taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", name)

    def sha(rel):
        with open(os.path.join(ROOT, rel), "rb") as f:
            return hashlib.sha256(f.read()).hexdigest()[:16]
    try:
        with open(path) as f:
            rec = json.load(f)
        same = all(sha(p) == h for p, h in {**rec["sources"], **rec["build"]}.items())
    except (OSError, ValueError, KeyError):
        return None
    return rec if same else None


# case name -> committed counter record of the kernels it runs
COUNTER_RECORDS = {
    "w4a16-decode-M16-K5120-N17408-g128-asym": "w4a16_decode_M16_K5120_N17408_counters.json",
    "w4a16-decode-M64-K5120-N17408-g128-asym": "w4a16_decode_M64_K5120_N17408_counters.json",
    "w4a16-midbatch-M256-K4096-N8192-g256-asym": "w4a16_mid_M256_K4096_N8192_counters.json",
    "w4a16-midbatch-M256-K4096-N8192-percol-asym": "w4a16_mid_M256_K4096_N8192_counters.json",
    "w4a16-prefill-M4096-K5120-N17408-g128-sym-signed": "w4a16_prefill_M4096_K5120_N17408_counters.json",
    "w4a8-moe-E8x64-K2048-N7168-g128": "w4a8_E8x64_K2048_N7168_counters.json",
    "w4a8-moe-asym-E8x64-K2048-N7168-g128": "w4a8_E8x64_K2048_N7168_counters.json",
    "w4a16-swiglu-decode-M16-K5120-N17408x2-g128-asym": "w4a16_swiglu_decode_M16_K5120_N17408x2_counters.json",
    "quantize-rows-int8-M4096-K5120": "quantize_rows_int8_M4096_K5120_counters.json",
}
COUNTER_FIELDS = ("duration_us_under_counters", "mfma_busy_of_grbm_cycles", "grbm_clock_ghz",
                  "other_valu_per_mfma", "traffic_bytes", "algorithmic_bytes",
                  "traffic_over_algorithmic")


def case_counters(name):
    """Counter figures (rocprofv3 --pmc) of the kernels a case runs, from the
    committed record while its sources are unchanged, else None."""
    fn = COUNTER_RECORDS.get(name)
    rec = _committed(fn) if fn else None
    if not rec:
        return None
    out = {k: {f: v[f] for f in COUNTER_FIELDS if f in v} for k, v in rec["kernels"].items()}
    out["source"] = "profiles/" + fn[:-5] + ".md"
    return out


def measured_traffic():
    """HBM bytes per launch of the decode kernel (FETCH_SIZE + WRITE_SIZE,
    copy-calibrated) from the committed counter record, or None."""
    rec = _committed(COUNTER_RECORDS["w4a16-decode-M16-K5120-N17408-g128-asym"])
    return next(iter(rec["kernels"].values()))["traffic_bytes"] if rec else None


def achievable(primary_bytes):
    """Best sustained rates of the probe kernels (libqgprobe.so) over a small
    sweep of launch shapes, HIP events on the launch stream."""
    import torch
    from int4_weight_only_uint32_amd import probe
    res = {"sweeps": {}}

    def sweep(key, fn, shapes):
        vals = {}
        for sh in shapes:
            vals["/".join(map(str, sh))] = fn(*sh)
        res["sweeps"][key] = vals
        best = max(vals, key=vals.get)
        return vals[best], best

    # HBM reads, rotated over copies so nothing is served from the caches
    for key, size in (("hbm_read_gbps_primary_size", primary_bytes), ("hbm_read_gbps_1GiB", 1 << 30)):
        size = size // 1024 * 1024
        n = max(2, math.ceil(ROTATE_BYTES / size))
        bufs = [torch.ones(size, dtype=torch.uint8, device="cuda") for _ in range(n)]
        best, at = sweep(key, lambda G, U: probe.hbm_read_gbps(bufs, G, U),
                         [(G, U) for G in (1024, 2048, 4096) for U in (1, 2, 4)])
        res[key] = best
        res[key + "_at"] = "workgroups/unroll " + at
        del bufs
        torch.cuda.empty_cache()
    # about 1 ms per launch at the published rates
    for key, fn, shapes in (
            ("mfma_f16_16x16x32_tflops", lambda G: probe.mfma_f16_tflops(16, G, 2048 * 1024 // G), [(512,), (1024,), (2048,)]),
            ("mfma_f16_32x32x16_tflops", lambda G: probe.mfma_f16_tflops(32, G, 4096 * 1024 // G), [(512,), (1024,), (2048,)]),
            ("mfma_i8_16x16x64_tops", lambda G: probe.mfma_i8_tops(G, 2048 * 1024 // G), [(512,), (1024,), (2048,)])):
        best, at = sweep(key, fn, shapes)
        res[key] = best
        res[key + "_at"] = "workgroups " + at
    res["hbm_read_gbps"] = max(res["hbm_read_gbps_primary_size"], res["hbm_read_gbps_1GiB"])
    res["mfma_f16_tflops"] = max(res["mfma_f16_16x16x32_tflops"], res["mfma_f16_32x32x16_tflops"])
    return res


def add_fractions(r, ach):
    """Fractions of one case against the measured achievable rates."""
    if ach is None:
        return
    if "weight_gbps" in r:
        r["frac_achievable_hbm_weight"] = r["weight_gbps"] / ach["hbm_read_gbps"]
    else:
        r["frac_achievable_hbm"] = r["alg_gbps"] / ach["hbm_read_gbps"]
    if "tflops" in r:
        r["frac_achievable_fp16_mfma"] = r["tflops"] / ach["mfma_f16_tflops"]
    if "tops" in r:
        r["frac_achievable_int8_mfma"] = r["tops"] / ach["mfma_i8_16x16x64_tops"]


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def _oracle_case(oracle, nm, rows, full):
    """One oracle call on a named workload: every row when `full` or when the
    workload has at most `rows` rows, else its first `rows` rows (W4A8: the
    first rows of each expert).  Returns the per-case record."""
    import numpy as np
    import synth
    c = synth.workload(nm)
    if nm.startswith("w4a8"):
        per = np.diff(c.offsets)
        take = per if full else np.minimum(per, rows)
        idx = np.concatenate([np.arange(o, o + t) for o, t in zip(c.offsets[:-1], take)])
        off = np.concatenate([[0], np.cumsum(take)]).astype(np.int32)
        M, total, K, N = int(take.sum()), int(per.sum()), c.K, c.N
        wb = c.E * (K * N // 2 + (K // c.g) * N * 2)
        t0 = time.perf_counter()
        oracle.w4a8(c.Aq[idx], c.a_scale[idx], c.q, c.s, off, c.g, fold=True, want_acc=False)
        dt = time.perf_counter() - t0
    else:
        total, K, N = c.M, c.K, c.N
        M = total if full else min(total, rows)
        wb = weight_bytes(K, N, c.g, c.z is not None)
        t0 = time.perf_counter()
        oracle.w4a16(c.A[:M], c.q, c.s, c.z, c.g, fold=True)
        dt = time.perf_counter() - t0
    flops = 2.0 * M * N * K
    return {"case": nm, "rows": M, "rows_total": total, "s": round(dt, 3),
            "gflops": round(flops / dt / 1e9, 3),
            "weight_gbps": round(wb / dt / 1e9, 3),
            "full_call_s_linear": round(dt * total / M, 2)}


def cpu_baseline(case, full=True):
    """The oracle (fp64 dequant + naive loop, OpenMP) on this host.  Primary
    workload: whole calls repeated until at least 8 s have passed (at most 40
    calls); returns the mean TFLOP/s and the thread count it used.  Then one
    whole oracle call per named workload (about 20 s in all on a 16-core
    host; with full=False only the first 64 rows for M >= 256 and the first 8
    rows of every expert of the W4A8 batch), each with its seconds, GFLOP/s,
    weight GB/s and the seconds a whole call takes (measured, or linear in the
    rows for a sample)."""
    import oracle
    import synth
    oracle.build(force=False)
    threads = int(os.environ.get("OMP_NUM_THREADS", "0")) or len(os.sched_getaffinity(0))
    calls = 0
    t0 = time.perf_counter()
    while True:
        oracle.w4a16(case.A, case.q, case.s, case.z, case.g, fold=True)
        calls += 1
        dt = time.perf_counter() - t0
        if dt >= 8.0 or calls >= 40:
            break
    flops = 2.0 * case.M * case.N * case.K * calls
    per_case = []
    for nm in synth.WORKLOADS:
        if nm == case.name:
            continue
        r = _oracle_case(oracle, nm, 8 if nm.startswith("w4a8") else 64, full)
        log(json.dumps(r))
        per_case.append(r)
    return dict(value=flops / dt / 1e12, unit="TFLOP/s", cores=threads, kind="oracle",
                cpu=cpu_model(),
                sample=f"{calls} whole oracle calls on M={case.M} K={case.K} N={case.N} g={case.g} "
                       f"asym ({dt:.1f} s wall, {dt / calls:.2f} s per call; fp64 dequant + "
                       f"naive m-k-n loop)",
                cases=per_case)


def bench_swiglu(name, steps, warmup, M, K, N, g, asym=True):
    """SwiGLU of a gate/up pair (one packed [K, 2N] weight) against the plain
    GEMM of the same pair (its [M, 2N] product, no activation)."""
    import numpy as np
    import torch

    import int4_weight_only_uint32_amd as qg
    import synth

    c = synth.w4a16_case(M, K, 2 * N, g, asym=asym, signed_scales=not asym, stream=91, case_id=99)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    pair = qg.pack(dev(c.q), dev(c.s), dev(c.z) if asym else None, g)
    wb = weight_bytes(K, 2 * N, g, asym)
    R = max(1, math.ceil(ROTATE_BYTES / wb))
    copies = [pair] + [qg.PackedWeight(w=pair.w.clone(), scale=pair.scale.clone(),
                                       delta=None if pair.delta is None else pair.delta.clone(),
                                       K=K, N=2 * N, group_size=g)
                       for _ in range(R - 1)]
    A = dev(c.A)
    H = torch.empty((M, N), dtype=torch.float16, device="cuda")
    Y = torch.empty((M, 2 * N), dtype=torch.float16, device="cuda")
    n = max(qg.qg_workspace_bytes(qg.QG_OP_W4A16_SWIGLU, M, N, K, g, 1, 0),
            qg.qg_workspace_bytes(qg.QG_OP_W4A16, M, 2 * N, K, g, 1, 0), 256)
    ws = torch.zeros(n, dtype=torch.uint8, device="cuda")

    def fused(i):
        p = copies[i]
        qg.qgemm_w4a16_swiglu(A, p.w, p.scale, p.delta, H, M, N, K, g, 0, ws)

    def gemm(i):
        p = copies[i]
        qg.qgemm_w4a16(A, p.w, p.scale, p.delta, Y, M, 2 * N, K, g, 0, ws)

    ms, ms_graph, ms_eager = time_best(fused, R, steps, warmup)
    ms_gemm, _, _ = time_best(gemm, R, steps, warmup)
    res = dict(name=name, M=M, K=K, N=N, group=g, mode="asym" if asym else "sym-fold",
               us_per_call=ms * 1e3,
               weight_bytes=wb, weight_gbps=wb / (ms * 1e-3) / 1e9,
               tflops=4.0 * M * N * K / (ms * 1e-3) / 1e12, rotated_copies=R,
               us_pair_gemm_only=ms_gemm * 1e3,
               us_per_call_graph=ms_graph * 1e3 if ms_graph else None,
               us_per_call_eager=ms_eager * 1e3)
    res["pct_hbm_weight"] = 100.0 * res["weight_gbps"] / HBM_PEAK_GBPS
    res["pct_fp16_mfma"] = 100.0 * res["tflops"] / FP16_PEAK_TFLOPS
    del copies, A, H, Y, ws
    torch.cuda.empty_cache()
    return res


def bench_quantize(name, steps, warmup, A16, gemm=None):
    """Per-row int8 quantization of the fp16 activations A16 [M,K]; with
    `gemm` (the W4A8 case) also the quantizer followed by the W4A8 GEMM, the
    step of an fp16-input W4A8 layer.  Inputs rotate over >= ROTATE_BYTES of
    copies, so the rate is HBM's and not a cache's."""
    import numpy as np
    import torch

    import int4_weight_only_uint32_amd as qg

    M, K = A16.shape
    alg = M * K * 2 + M * K + M * 4
    R = max(1, math.ceil(ROTATE_BYTES / alg))
    A0 = torch.from_numpy(np.ascontiguousarray(A16)).cuda()
    As = [A0] + [A0.clone() for _ in range(R - 1)]
    Qs = [torch.empty((M, K), dtype=torch.int8, device="cuda") for _ in range(R)]
    Ss = [torch.empty((M,), dtype=torch.float32, device="cuda") for _ in range(R)]

    def call(i):
        qg.quantize_rows_int8(As[i], M, K, Qs[i], Ss[i])

    ms, ms_graph, ms_eager = time_best(call, R, steps, warmup)
    res = dict(name=name, M=M, K=K, us_per_call=ms * 1e3, alg_bytes=alg,
               alg_gbps=alg / (ms * 1e-3) / 1e9, rotated_copies=R,
               us_per_call_graph=ms_graph * 1e3 if ms_graph else None,
               us_per_call_eager=ms_eager * 1e3)
    res["pct_hbm"] = 100.0 * res["alg_gbps"] / HBM_PEAK_GBPS
    if gemm is not None:
        W, S, off, E, mr, N, g, C = gemm

        def step(i):
            qg.quantize_rows_int8(As[i], M, K, Qs[i], Ss[i])
            qg.qgemm_w4a8(Qs[i], Ss[i], W, S, off, E, M, mr, N, K, g, C)

        ms2, _, _ = time_best(step, R, steps, warmup)
        res["us_quantize_plus_w4a8"] = ms2 * 1e3
    del As, Qs, Ss
    torch.cuda.empty_cache()
    return res


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: this library runs on one GPU; --gpus {args.gpus} is not supported "
              f"(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import synth
    if args.cpu_only:
        print(json.dumps({"cpu_baseline": cpu_baseline(
            synth.workload("w4a16-decode-M16-K5120-N17408-g128-asym"), full=not args.cpu_sample)}),
              flush=True)
        return
    import torch
    import int4_weight_only_uint32_amd as qg
    global GRAPH
    GRAPH = not args.eager
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    if not qg.qg_device_supported(0):
        print("bench.py: cuda:0 is not gfx950", file=sys.stderr)
        sys.exit(1)
    props = torch.cuda.get_device_properties(0)
    log(f"device: {props.name} {getattr(props, 'gcnArchName', '')} CUs={props.multi_processor_count}")

    if args.calibrate_copy:
        n = 256 * 1024 * 1024
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(20):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copied {n} bytes x 20")
        return
    steps, warmup = args.steps, args.warmup
    primary_name = "w4a16-decode-M16-K5120-N17408-g128-asym"
    primary, pcase = bench_w4a16(primary_name, steps, warmup)
    log(json.dumps(primary))

    cases = []
    want = None if args.cases == "all" else set(args.cases.split(","))
    if not args.only_primary:
        plan = (synth.names("w4a16-small") + synth.names("w4a16-decode") +
                synth.names("w4a16-midbatch") + synth.names("w4a16-prefill"))
        for nm in plan:
            if nm == primary_name or (want and nm not in want):
                continue
            M = synth.WORKLOADS[nm]["spec"]["M"]
            st = steps if M <= 256 else max(10, steps // 10)
            r, _ = bench_w4a16(nm, st, min(warmup, st))
            log(json.dumps(r))
            cases.append(r)
        sep = primary_name + "+separate-correction"
        if not want or sep in want:
            r, _ = bench_w4a16(primary_name, steps, warmup, flags=qg.QG_CORR_SEPARATE, label=sep)
            log(json.dumps(r))
            cases.append(r)
        for nm in synth.names("w4a8"):
            if not want or nm in want:
                r = bench_w4a8(nm, steps, warmup)
                log(json.dumps(r))
                cases.append(r)
        an = "w4a8-moe-asym-E8x64-K2048-N7168-g128"
        if not want or an in want:
            # the expert batch's A, codes and scales, with AWQ-style zero-points
            ca = synth.w4a8_case(8, 64, 2048, 7168, 128, stream=4, case_id=0, asym=True, name=an)
            r = bench_w4a8(an, steps, warmup, case=ca)
            log(json.dumps(r))
            cases.append(r)
            del ca
        vn = "w4a16-vocab-head-M16-K5120-N50257-g128-asym"
        if not want or vn in want:
            # a vocabulary of 50257 (N padded to 50304 in the pack, C cropped)
            cv = synth.w4a16_case(16, 5120, 50257, 128, asym=True, stream=92, case_id=1016)
            r, _ = bench_w4a16(vn, steps, warmup, case=cv)
            log(json.dumps(r))
            cases.append(r)
            del cv
        sn = "w4a16-swiglu-decode-M16-K5120-N17408x2-g128-asym"
        if not want or sn in want:
            r = bench_swiglu(sn, steps, warmup, 16, 5120, 17408, 128)
            log(json.dumps(r))
            cases.append(r)
        sn = "w4a16-swiglu-prefill-M4096-K5120-N17408x2-g128-sym-signed"
        if not want or sn in want:
            st = max(5, steps // 20)
            r = bench_swiglu(sn, st, min(warmup, st), 4096, 5120, 17408, 128, asym=False)
            log(json.dumps(r))
            cases.append(r)
        qn = "quantize-rows-int8-E8x64-K2048+w4a8"
        if not want or qn in want:
            c = synth.workload("w4a8-moe-E8x64-K2048-N7168-g128")
            dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
            packs = [qg.pack(dev(c.q[e]), dev(c.s[e]), None, c.g, fold=True) for e in range(c.E)]
            W = torch.stack([p.w for p in packs]).contiguous()
            S = torch.stack([p.scale for p in packs]).contiguous()
            C = torch.empty((c.M_total, c.N), dtype=torch.float16, device="cuda")
            mr = int(np.max(np.diff(c.offsets)))
            gemm = (W, S, dev(c.offsets), c.E, mr, c.N, c.g, C)
            r = bench_quantize(qn, steps, warmup, c.A16, gemm)
            log(json.dumps(r))
            cases.append(r)
            del packs, W, S, C, gemm
        qn = "quantize-rows-int8-M16-K5120"
        if not want or qn in want:
            r = bench_quantize(qn, steps, warmup, pcase.A)
            log(json.dumps(r))
            cases.append(r)
        qn = "quantize-rows-int8-M4096-K5120"
        if not want or qn in want:
            r = bench_quantize(qn, steps, warmup, synth.activations(4096, 5120))
            log(json.dumps(r))
            cases.append(r)

    for r in [primary] + cases:
        cc = case_counters(r["name"])
        if cc:
            r["counters"] = cc

    ach = None
    if not args.no_probes:
        ach = achievable(primary["weight_bytes"])
        log(json.dumps(ach))
        for r in [primary] + cases:
            add_fractions(r, ach)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(pcase, full=not args.cpu_sample)
        log(json.dumps(cpu))

    launch_us = primary["us_per_call"]
    achieved = primary["weight_bytes"] / (launch_us * 1e-6) / 1e9
    out = {
        "metric": "W4A16 g128 GEMM TFLOPS + weight GB/s (%roofline) at M=16 and M=4096",
        "value": primary["tflops"],
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": primary["us_per_call"] / 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp16",
        "data": "synthetic (seeded; A~N(0,1) fp16, q~U{0..15}, |s|~U[1e-3,2e-2], "
                "z=-8s+N(0,1e-3)); weights rotated over >=512 MB of copies",
        "timing": ("per case the faster of one graph replay of the timed calls and eager "
                   "launches of the same calls (HIP events on the launch stream)")
                  if GRAPH else "eager launches (HIP events on the launch stream)",
        "config": {"workload": "w4a16-decode M=16 K=5120 N=17408 group=128 asymmetric, "
                               "delta fused (one launch per step)",
                   "M": 16, "K": 5120, "N": 17408, "group": 128},
        "weight_gbps": primary["weight_gbps"],
        "pct_hbm_roofline_weight": primary["pct_hbm_weight"],
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBPS, "traffic": measured_traffic(),
                     "kernel": "w4a16_decode_kernel (split-K, fused delta)",
                     "traffic_unit": "bytes per launch (rocprofv3 FETCH_SIZE+WRITE_SIZE, copy-calibrated)",
                     "algorithmic_bytes_per_launch": primary["weight_bytes"],
                     "achievable": ach["hbm_read_gbps_primary_size"] if ach else None,
                     "frac_of_achievable": achieved / ach["hbm_read_gbps_primary_size"] if ach else None},
        "achievable": ach,
        "cpu_baseline": cpu,
        "cases": cases,
    }
    prefill = [c for c in cases if c["name"].startswith("w4a16-prefill")]
    if prefill:
        out["prefill_M4096"] = {"tflops": prefill[0]["tflops"],
                                "pct_fp16_mfma": prefill[0]["pct_fp16_mfma"],
                                "frac_achievable_fp16_mfma": prefill[0].get("frac_achievable_fp16_mfma"),
                                "us_per_call": prefill[0]["us_per_call"],
                                "counters": prefill[0].get("counters")}
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
