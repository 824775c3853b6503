"""Benchmark of the FP8 block-scaled NT GEMM on one MI355X.

One step = one pass over the dense DeepSeek-V3-like shape list (M in {64, 128, 4096}
x (N,K) in {(2112,7168), (24576,1536), (32768,512), (7168,16384), (4096,7168),
(7168,2048)}), A ~ N(0,1) and B ~ N(0,0.02) quantised to e4m3 with 1x128 / 128x128
FP32 scales, BF16 output. Every shape has its own resident operands (no operand is
reused within a step, so each GEMM streams its inputs from HBM). Prints one JSON line.

  value     = total algorithmic FP8 FLOPs of a step / measured step time (TFLOP/s)
  per_shape = per-GEMM kernel time from HIP events on the launch stream, FP8 TFLOP/s,
              HBM GB/s of the algorithmic bytes, and the fraction of the binding roofline:
              the 18 dense shapes (the step), then, timed separately, the small dense
              128x256x512 case (per-call latency, no roofline fraction), the two
              contiguous grouped cases, the ten masked decode cases and the MoE FFN pair
  roofline  = the same for the shape that takes the most time, its mean launch time from
              HIP events on the launch stream (avg_us), traffic from the rocprofv3 counter
              table of the same kernel sources (null when the sources have changed)
  cpu_baseline = the CPU oracle timed on one full shape on this host (median of 3) and
              single-threaded on the small case
"""
import argparse
import csv
import glob
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_FP8_TFLOPS = 5000.0   # MI355X dense FP8 MFMA
PEAK_HBM_GBS = 8000.0      # MI355X HBM3E
METRIC = "FP8 TFLOPS & GB/s per shape, 1×MI355X, % of FP8 MFMA peak / HBM roofline"
CONFIG2 = [(m, n, k) for m in (64, 128, 4096)
           for (n, k) in ((2112, 7168), (24576, 1536), (32768, 512), (7168, 16384), (4096, 7168), (7168, 2048))]


def algo_work(M, N, K, G=1, scale_bytes=4.0):
    """Algorithmic FLOPs and HBM bytes of one dense call (each operand read once, D written
    once); scale_bytes per block scale: 4 (FP32) or 1 (packed UE8M0, four codes a word)."""
    flops = 2.0 * M * N * K
    kb = K // 128
    nbytes = int(M * K + G * N * K + M * N * 2 + (M * kb + G * ((N + 127) // 128) * kb) * scale_bytes)
    return flops, nbytes


def classify(flops, nbytes):
    t_mfma = flops / (PEAK_FP8_TFLOPS * 1e12)
    t_hbm = nbytes / (PEAK_HBM_GBS * 1e9)
    return ("mfma", t_mfma) if t_mfma >= t_hbm else ("hbm", t_hbm)


def kernel_source_hash():
    """sha256 of the HIP sources: counter-derived traffic is only valid for this kernel."""
    h = hashlib.sha256()
    for f in sorted(glob.glob(os.path.join(ROOT, "moe_grouped_gemm_fp32_amd", "csrc", "*"))):
        with open(f, "rb") as fh:
            h.update(os.path.basename(f).encode())
            h.update(fh.read())
    return h.hexdigest()[:16]


def read_counter_csv(d, counter):
    """Per-dispatch values of `counter` from a rocprofv3 --pmc csv directory: list of (kernel, value)."""
    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    rows = []
    for f in files:
        with open(f) as fh:
            for r in csv.DictReader(fh):
                if r["Counter_Name"] == counter:
                    rows.append((int(r["Dispatch_Id"]), r["Kernel_Name"], float(r["Counter_Value"])))
    rows.sort()
    return [(k, v) for _, k, v in rows]


N_SMALL, SMALL_REPS = 200, 5   # the small dense case: SMALL_REPS groups of N_SMALL back-to-back calls


def dispatch_blocks(n, shapes, steps, warmup):
    """GEMM-kernel dispatch indices (in dispatch order) of one case each, for a profiled
    default run of `steps` / `warmup`: the dense shapes step by step, then the small dense
    case (one checking call, then its timed calls), then the untimed gate+up call that
    makes the MoE down GEMM's input and the grouped cases step by step. A run with
    --no-grouped holds the dense block only. The last `steps` dispatches of a case are the
    ones its HIP-event time covers. Returns (dense, small, grouped) index lists."""
    per = warmup + 2 * steps + 1
    nd = len(shapes) * per
    dense = [list(range(i, nd, len(shapes))) for i in range(len(shapes))]
    if n == nd:
        return dense, [], []
    ng = len(GROUPED_CASES)
    g0 = nd + 1 + N_SMALL * SMALL_REPS + 1
    if n != g0 + ng * per:
        sys.exit("%d GEMM dispatches in the trace; a run of --steps %d --warmup %d makes %d (dense only) or %d"
                 % (n, steps, warmup, nd, g0 + ng * per))
    small = list(range(nd + 1, nd + 1 + N_SMALL * SMALL_REPS))
    grouped = [list(range(g0 + i, g0 + ng * per, ng)) for i in range(ng)]
    return dense, small, grouped


def pmc_summary(args, shapes):
    """Build the HBM-traffic table from FETCH_SIZE / WRITE_SIZE runs of this benchmark and of
    the plain copy (--copy-mb). Counters are KiB per dispatch; each is scaled by the ratio
    (known copy bytes) / (counter bytes of the copy)."""
    fetch_dir, write_dir, cfetch_dir, cwrite_dir = args.pmc_summary
    copy_bytes = args.copy_mb * (1 << 20)

    def copy_factor(d, counter):
        vals = [v for k, v in read_counter_csv(d, counter) if "fp8_gemm" not in k]
        big = max(vals)  # the copy kernel moves the most bytes of its process
        return copy_bytes / (big * 1024.0)

    ff = copy_factor(cfetch_dir, "FETCH_SIZE")
    fw = copy_factor(cwrite_dir, "WRITE_SIZE")
    fetch = [v for k, v in read_counter_csv(fetch_dir, "FETCH_SIZE") if "fp8_gemm_kernel" in k]
    write = [v for k, v in read_counter_csv(write_dir, "WRITE_SIZE") if "fp8_gemm_kernel" in k]
    dense, _, _ = dispatch_blocks(len(fetch), shapes, args.steps, args.warmup)
    table = {}
    for i, (M, N, K) in enumerate(shapes):
        f = [fetch[j] for j in dense[i]]
        w = [write[j] for j in dense[i]]
        fk = sum(f) / len(f)
        wk = sum(w) / len(w)
        _, algo = algo_work(M, N, K)
        traffic = fk * 1024.0 * ff + wk * 1024.0 * fw
        table["%d,%d,%d" % (M, N, K)] = {"fetch_kib": round(fk, 1), "write_kib": round(wk, 1),
                                         "bytes_per_launch": round(traffic), "algo_bytes": algo,
                                         "traffic_over_algo": round(traffic / algo, 3)}
    out = {"kernel_sha": kernel_source_hash(), "copy_mb": args.copy_mb, "fetch_factor": round(ff, 4),
           "write_factor": round(fw, 4), "shapes": table}
    with open(args.traffic_file, "w") as fh:
        json.dump(out, fh, indent=1)
    print(json.dumps(out))


def kg_pmc_summary(args):
    """HBM traffic of the K-grouped kernel from FETCH_SIZE / WRITE_SIZE runs of
    --workload kgrouped, scaled by the copy-kernel factors stored in the dense traffic
    table (measured in the same session); dispatch i belongs to case i mod 2."""
    fetch_dir, write_dir = args.kg_pmc_summary
    with open(args.traffic_file) as fh:
        dense = json.load(fh)
    ff, fw = dense["fetch_factor"], dense["write_factor"]
    fetch = [v for k, v in read_counter_csv(fetch_dir, "FETCH_SIZE") if "k_grouped" in k]
    write = [v for k, v in read_counter_csv(write_dir, "WRITE_SIZE") if "k_grouped" in k]
    import synth
    ks = [(t + 127) // 128 * 128 for t in synth.k_grouped_tokens(KGROUP_EXPERTS, seed=9600)]
    table = {}
    for i, (M, N) in enumerate(KGROUP_CASES):
        f, w = fetch[i::len(KGROUP_CASES)], write[i::len(KGROUP_CASES)]
        fk, wk = sum(f) / len(f), sum(w) / len(w)
        _, algo = kgrouped_work(M, N, ks)
        traffic = fk * 1024.0 * ff + wk * 1024.0 * fw
        table["%d,%d" % (M, N)] = {"fetch_kib": round(fk, 1), "write_kib": round(wk, 1),
                                   "bytes_per_launch": round(traffic), "algo_bytes": algo,
                                   "traffic_over_algo": round(traffic / algo, 3)}
    out = {"kernel_sha": kernel_source_hash(), "fetch_factor": ff, "write_factor": fw, "ks": ks, "cases": table}
    with open(os.path.join(ROOT, "profiles", "traffic_kgrouped.json"), "w") as fh:
        json.dump(out, fh, indent=1)
    print(json.dumps(out))


def read_trace(d, kernel):
    """(dispatch id, kernel name, duration ns) of every dispatch whose name contains
    `kernel` in a rocprofv3 --kernel-trace csv directory, in dispatch order."""
    files = glob.glob(os.path.join(d, "**", "*kernel_trace.csv"), recursive=True)
    rows = []
    for f in files:
        with open(f) as fh:
            for r in csv.DictReader(fh):
                if kernel in r["Kernel_Name"]:
                    rows.append((int(r["Dispatch_Id"]), r["Kernel_Name"],
                                 int(r["End_Timestamp"]) - int(r["Start_Timestamp"])))
    rows.sort()
    return rows


def trace_summary(d, shapes, steps, warmup, kernel="fp8_gemm_kernel"):
    """Per-case GEMM kernel durations from a rocprofv3 --kernel-trace csv directory of a
    run with the same --steps / --warmup (the default run, or a dense-only one such as
    --workload ue8m0 or --layout tn with kernel="fp8_k_grouped_tn_kernel"): the mean over
    all of a case's dispatches and over the event-timed ones (the last `steps`), which the
    run's own HIP-event figures cover."""
    rows = read_trace(d, kernel)
    dense, small, grouped = dispatch_blocks(len(rows), shapes, steps, warmup)

    def stats(idx):
        sel = [rows[j] for j in idx]
        timed = sel[-steps:]
        return {"kernel": sel[0][1].replace("void fp8gemm::", ""), "dispatches": len(sel),
                "avg_us": round(sum(r[2] for r in sel) / len(sel) / 1e3, 2),
                "timed_avg_us": round(sum(r[2] for r in timed) / len(timed) / 1e3, 2)}

    for i, (M, N, K) in enumerate(shapes):
        o = {"M": M, "N": N, "K": K}
        o.update(stats(dense[i]))
        flops, nbytes = algo_work(M, N, K)
        o.update({"tflops": round(flops / o["timed_avg_us"] / 1e6, 1),
                  "gbs": round(nbytes / o["timed_avg_us"] / 1e3, 1)})
        print(json.dumps(o))
    if small:
        sel = [rows[j][2] for j in small]
        print(json.dumps({"case": "dense small 128x256x512", "dispatches": len(sel),
                          "avg_us": round(sum(sel) / len(sel) / 1e3, 2)}))
    for name, idx in zip(GROUPED_CASES, grouped):
        o = {"case": name}
        o.update(stats(idx))
        print(json.dumps(o))


GROUPED_CASES = (["contiguous G=4 x 8192 rows N=4096 K=7168", "contiguous G=8 x 4096 rows N=7168 K=2048"] +
                 ["masked G=%d N=%d K=%d" % (g, n, k) for (n, k) in ((4096, 7168), (7168, 2048)) for g in (1, 2, 4, 8, 16)] +
                 ["moe gate+up N=4096 K=7168", "moe down N=7168 K=2048"])


def trace_summary_cases(rows, names, steps):
    """Per-case mean kernel duration over all dispatches and over the event-timed ones (the
    last `steps` of each case) when dispatch i belongs to case i mod len(names)."""
    for i, name in enumerate(names):
        sel = rows[i::len(names)]
        timed = sel[-steps:]
        print(json.dumps({"case": name, "kernel": sel[0][1].replace("void fp8gemm::", ""),
                          "dispatches": len(sel), "avg_us": round(sum(r[2] for r in sel) / len(sel) / 1e3, 2),
                          "timed_avg_us": round(sum(r[2] for r in timed) / len(timed) / 1e3, 2)}))


def trace_summary_grouped(d, steps):
    """Per-case GEMM kernel durations of a --workload grouped run from a rocprofv3
    --kernel-trace csv directory. The first GEMM dispatch is the untimed gate+up call that
    produces the down GEMM's input; after it, dispatch i belongs to case i mod 14."""
    trace_summary_cases(read_trace(d, "fp8_gemm_kernel")[1:], GROUPED_CASES, steps)


def read_counters(d, kernel):
    """({(dispatch id, counter): value summed over the counter's hardware instances},
    sorted dispatch ids, sorted counter names) of the dispatches whose kernel name
    contains `kernel` in a rocprofv3 --pmc csv directory."""
    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    per = {}
    for f in files:
        with open(f) as fh:
            for r in csv.DictReader(fh):
                if kernel not in r["Kernel_Name"]:
                    continue
                key = (int(r["Dispatch_Id"]), r["Counter_Name"])
                per[key] = per.get(key, 0.0) + float(r["Counter_Value"])
    return per, sorted({k[0] for k in per}), sorted({k[1] for k in per})


def counter_row(per, names, sel, row):
    for c in names:
        vals = [per[(x, c)] for x in sel if (x, c) in per]
        row[c] = sum(vals) / len(vals) if vals else None
    return row


def counter_summary(d, shapes, steps, warmup, kernel="fp8_gemm_kernel"):
    """Per-shape mean of every counter in a rocprofv3 --pmc csv directory of a run with
    the same --steps / --warmup (the default run's dense shapes, or a dense-only run);
    values are summed over the counter's hardware instances within a dispatch."""
    per, dispatches, names = read_counters(d, kernel)
    dense, _, _ = dispatch_blocks(len(dispatches), shapes, steps, warmup)
    for i, (M, N, K) in enumerate(shapes):
        sel = [dispatches[j] for j in dense[i]]
        print(json.dumps(counter_row(per, names, sel, {"M": M, "N": N, "K": K, "dispatches": len(sel)})))


def counter_summary_cases(d, kernel, cases, skip=0):
    """Per-case counter means when, after the first `skip` dispatches, dispatch i belongs
    to case i mod len(cases)."""
    per, dispatches, names = read_counters(d, kernel)
    dispatches = dispatches[skip:]
    for i, name in enumerate(cases):
        sel = dispatches[i::len(cases)]
        print(json.dumps(counter_row(per, names, sel, {"case": name, "dispatches": len(sel)})))


def copy_only(args):
    """A plain device copy of --copy-mb MiB, the calibration kernel for the byte counters."""
    import torch
    n = args.copy_mb * (1 << 20)
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": n}))


def parse_shapes(text):
    out = []
    for item in text.split(";"):
        m, n, k = (int(x) for x in item.split(","))
        out.append((m, n, k))
    return out


def blas_threads():
    """Threads the oracle's matrix products use (numpy's BLAS pool), else the usable cores."""
    try:
        from threadpoolctl import threadpool_info
        blas = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        if blas:
            return int(blas[0].get("num_threads"))
    except Exception:  # pragma: no cover
        pass
    return len(os.sched_getaffinity(0))


def cpu_baseline(runs=3):
    """The CPU oracle, as it stands, on the full M=4096, N=7168, K=16384 dense shape (the
    dominant shape of the timed step; ~8 s per run on a 16-thread host): median of `runs`
    runs on the host's cores, plus the median of three single-thread runs of the small
    128x256x512 case."""
    import numpy as np
    import oracle
    import synth
    from threadpoolctl import threadpool_limits
    M, N, K = 4096, 7168, 16384
    c = synth.dense_case(M, N, K, seed=99, device="cpu")
    args = [c[k].numpy() for k in ("A", "sa", "B", "sb")]
    times = []
    for _ in range(runs):
        t0 = time.perf_counter()
        oracle.gemm_nt(*args)
        times.append(time.perf_counter() - t0)
    dt = float(np.median(times))
    threads = blas_threads()
    small = synth.dense_case(128, 256, 512, seed=98, device="cpu")
    sargs = [small[k].numpy() for k in ("A", "sa", "B", "sb")]
    st = []
    with threadpool_limits(limits=1):
        for _ in range(3):
            t0 = time.perf_counter()
            oracle.gemm_nt(*sargs)
            st.append(time.perf_counter() - t0)
    sdt = float(np.median(st))
    return {"value": round(2.0 * M * N * K / dt / 1e12, 6), "unit": "TFLOP/s", "cores": threads,
            "kind": "oracle", "seconds": round(dt, 3), "runs_seconds": [round(t, 3) for t in times],
            "sample": "full oracle (e4m3 decode, per-128-K FP64 block matmul, scaling, BF16 RNE) of the "
                      "dense M=4096 N=7168 K=16384 shape, 962 GFLOP, median of %d runs" % runs,
            "single_thread_small": {"shape": "128x256x512", "seconds": round(sdt, 5),
                                    "tflops": round(2.0 * 128 * 256 * 512 / sdt / 1e12, 6), "cores": 1}}


def grouped_work(m_live, g_active, N, K, m_padded=None):
    """Algorithmic FLOPs and HBM bytes of one grouped call: live rows only, each active
    group's B and sb read once, D written once for live rows."""
    kb = K // 128
    flops = 2.0 * m_live * N * K
    nbytes = (m_live * K + g_active * N * K + m_live * N * 2 + m_live * kb * 4 +
              g_active * ((N + 127) // 128) * kb * 4)
    padded = 2.0 * m_padded * N * K if m_padded is not None else flops
    return flops, nbytes, padded


def time_cases(fns, steps, warmup):
    """Run every callable once per step: `warmup` untimed steps, then `steps` timed steps
    (wall time, bracketed by synchronisations), then per-call durations from HIP events on
    the launch stream over `steps` more steps (one untimed step first and a single
    synchronisation at the end, so the host stays ahead of the GPU and no event pair
    includes host launch latency). Returns (ms per step, [mean ms per call])."""
    import torch

    def step(events=None):
        for i, fn in enumerate(fns):
            if events is not None:
                events[i][0].record()
            fn()
            if events is not None:
                events[i][1].record()

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    ms_per_step = (time.perf_counter() - t0) / steps * 1e3
    step()
    all_ev = []
    for _ in range(steps):
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in fns]
        step(ev)
        all_ev.append(ev)
    torch.cuda.synchronize()
    per = [0.0] * len(fns)
    for ev in all_ev:
        for i, (a, b) in enumerate(ev):
            per[i] += a.elapsed_time(b)
    return ms_per_step, [v / steps for v in per]


def grouped_cases(dev, ue=False):
    """The M-grouped workloads with their resident operands: contiguous (4 experts x 8192
    rows, N=4096, K=7168; 8 experts x 4096 rows, N=7168, K=2048), masked decode (G in 1, 2,
    4, 8, 16 at (N, K) = (4096, 7168) and (7168, 2048), M_max 4096, masked_m uniform in
    [179, 333], expected_m 256) and the MoE FFN pair (4096 tokens, 256 experts, top-8
    Zipf(1.1) routing, padded to 128 rows per expert; the down GEMM's input is the SwiGLU
    of the gate+up output re-quantised 1x128, untimed glue). ue: power-of-two scales
    through the *_ue8m0 calls. Returns a list of dicts (name, group, fn, flops, bytes,
    padded_flops, extra)."""
    import torch
    import moe_grouped_gemm_fp32_amd as fg
    import synth

    cases = []
    kind = "pow2" if ue else "normal"

    def add(name, group, fn, m_live, g_active, N, K, m_padded=None, extra=None):
        flops, nbytes, padded = grouped_work(m_live, g_active, N, K, m_padded)
        cases.append(dict(name=name, group=group, fn=fn, flops=flops, bytes=nbytes, padded_flops=padded,
                          extra=extra or {}))

    # contiguous, groups of equal size (multiples of 128 rows: no padding rows)
    for G, rows, N, K in ((4, 8192, 4096, 7168), (8, 4096, 7168, 2048)):
        c = synth.contiguous_case([rows] * G, N, K, seed=3000 + G, device=dev, kind=kind)
        ws = fg.make_workspace(fg.KIND_CONTIGUOUS, c["M"], N, K, G, device=dev)
        cfg = fg.query_config(fg.KIND_CONTIGUOUS, c["M"], N, K, G)
        add("contiguous G=%d x %d rows N=%d K=%d" % (G, rows, N, K), "contiguous",
            (lambda c=c, ws=ws: fg.fp8_grouped_gemm_nt_contiguous(c["A"], c["sa"], c["B"], c["sb"], c["D"],
                                                                  c["m_indices"], ws, ue8m0=ue)),
            G * rows, G, N, K, extra={"tile": "%dx%d" % (cfg["block_m"], cfg["block_n"]), "split_k": cfg["split_k"]})
    # masked decode
    for N, K in ((4096, 7168), (7168, 2048)):
        for G in (1, 2, 4, 8, 16):
            c = synth.masked_case(G, 4096, N, K, seed=4000 + G + N, device=dev, expected_m=256, kind=kind)
            mm = c["masked_m_list"]
            cfg = fg.query_config(fg.KIND_MASKED, 4096, N, K, G, expected_m=256)
            add("masked G=%d N=%d K=%d" % (G, N, K), "masked decode",
                (lambda c=c: fg.fp8_grouped_gemm_nt_masked(c["A"], c["sa"], c["B"], c["sb"], c["D"],
                                                           c["masked_m"], 256, ue8m0=ue)),
                sum(mm), sum(1 for v in mm if v > 0), N, K,
                extra={"masked_m_sum": sum(mm), "tile": "%dx%d" % (cfg["block_m"], cfg["block_n"])})
    # MoE FFN pair
    c1 = synth.moe_case(seed=5000, device=dev, N=4096, K=7168, kind=kind)
    mi = c1["m_indices"]
    m_live = int((mi >= 0).sum())
    g_act = sum(1 for v in c1["counts"] if v > 0)
    ws1 = fg.make_workspace(fg.KIND_CONTIGUOUS, c1["M"], 4096, 7168, 256, device=dev)
    fn1 = lambda: fg.fp8_grouped_gemm_nt_contiguous(c1["A"], c1["sa"], c1["B"], c1["sb"], c1["D"], mi, ws1, ue8m0=ue)
    fn1()
    torch.cuda.synchronize()
    A2, sa2 = synth.swiglu_requant(c1["D"].view(torch.bfloat16).float().nan_to_num(0.0), mi, pow2=ue)
    g2 = synth.make_generator(5001, dev)
    B2 = torch.empty(256, 7168, 2048, dtype=torch.uint8, device=dev)
    sb2 = torch.empty(256, 56, 16, dtype=torch.float32, device=dev)
    for e in range(256):
        b, sc = synth.make_weight(7168, 2048, kind, g2, dev)
        B2[e] = b
        sb2[e] = sc
    D2 = synth.sentinel_output((c1["M"], 7168), dev)
    ws2 = fg.make_workspace(fg.KIND_CONTIGUOUS, c1["M"], 7168, 2048, 256, device=dev)
    fn2 = lambda: fg.fp8_grouped_gemm_nt_contiguous(A2, sa2, B2, sb2, D2, mi, ws2, ue8m0=ue)
    add("moe gate+up (256 experts, %d live / %d padded rows) N=4096 K=7168" % (m_live, c1["M"]), "MoE FFN pair",
        fn1, m_live, g_act, 4096, 7168, m_padded=c1["M"])
    add("moe down (256 experts, %d live / %d padded rows) N=7168 K=2048" % (m_live, c1["M"]), "MoE FFN pair",
        fn2, m_live, g_act, 7168, 2048, m_padded=c1["M"])
    torch.cuda.synchronize()
    return cases


def grouped_rows(cases, per_ms):
    rows = []
    for c, ms in zip(cases, per_ms):
        bound, t_ideal = classify(c["flops"], c["bytes"])
        tflops = c["flops"] / (ms * 1e-3) / 1e12
        gbs = c["bytes"] / (ms * 1e-3) / 1e9
        frac = tflops / PEAK_FP8_TFLOPS if bound == "mfma" else gbs / PEAK_HBM_GBS
        r = {"config": c["group"], "case": c["name"], "us": round(ms * 1e3, 2), "tflops": round(tflops, 1),
             "gbs": round(gbs, 1), "bound": bound, "frac": round(frac, 4), "ideal_us": round(t_ideal * 1e6, 2),
             "padded_tflops": round(c["padded_flops"] / (ms * 1e-3) / 1e12, 1),
             "algo_bytes": c["bytes"], "algo_flops": c["flops"]}
        r.update(c["extra"])
        rows.append(r)
    return rows


def plan_sweep(args):
    """--plan-sweep dense|masked: time every tile / split (/ whole-tile-round) plan of each
    dense shape or masked decode case, forced for that call only, inside the benchmark's
    sequence of calls (the other calls keep their own plans). Rounds are enqueued without
    synchronising, so the GPU stays busy as in the benchmark; the median event time over
    `--rounds` rounds (after one untimed round) is printed per plan, one JSON line per case.
    The planner's cost constants are fitted to these tables (--plan-table)."""
    import numpy as np
    import torch
    import moe_grouped_gemm_fp32_amd as fg
    import synth
    dev = torch.device("cuda:0")
    WS = torch.zeros(1 << 30, dtype=torch.uint8, device=dev)   # one workspace, shared by every call in turn
    if args.plan_sweep == "dense":
        cases = []
        for i, (M, N, K) in enumerate(CONFIG2):
            c = synth.dense_case(M, N, K, seed=2000 + i, device=dev, a_std=1.0, b_std=0.02)
            cases.append(dict(key=[M, N, K], M=M, N=N, K=K, G=1, kind=fg.KIND_DENSE,
                              fn=(lambda c=c: fg.fp8_gemm_nt(c["A"], c["sa"], c["B"], c["sb"], c["D"], WS))))
    elif args.plan_sweep == "layout":   # the TN call: both operands K-major
        cases = []
        for i, (M, N, K) in enumerate(CONFIG2):
            c = synth.dense_case(M, N, K, seed=2000 + i, device=dev, a_std=1.0, b_std=0.02)
            At = torch.zeros(K, (M + 15) // 16 * 16, dtype=torch.uint8, device=dev)
            At[:, :M] = c["A"].t()
            Bt = torch.zeros(K, (N + 15) // 16 * 16, dtype=torch.uint8, device=dev)
            Bt[:, :N] = c["B"].t()
            cases.append(dict(key=[M, N, K], M=M, N=N, K=K, G=1, kind=fg.KIND_LAYOUT,
                              fn=(lambda c=c, At=At, Bt=Bt: fg.fp8_gemm_tn(At, c["sa"], Bt, c["sb"], c["D"],
                                                                           workspace=WS))))
            del c["A"], c["B"]
    else:
        cases = []
        for N, K in ((4096, 7168), (7168, 2048)):
            for G in (1, 2, 4, 8, 16):
                c = synth.masked_case(G, 4096, N, K, seed=4000 + G + N, device=dev, expected_m=256)
                cases.append(dict(key=[G, N, K], M=4096, N=N, K=K, G=G, kind=fg.KIND_MASKED,
                                  fn=(lambda c=c: fg.fp8_grouped_gemm_nt_masked(c["A"], c["sa"], c["B"], c["sb"],
                                                                                c["D"], c["masked_m"], 256, WS))))
    torch.cuda.synchronize()
    layout = args.plan_sweep == "layout"
    tiles = [(128, 128), (256, 256), (64, 128), (128, 64)] if layout else [(64, 64), (128, 64), (64, 128), (128, 128), (256, 128),
                                                      (128, 256), (64, 96), (128, 96)]
    for ti, t in enumerate(cases):
        nkb = t["K"] // 128
        masked = t["kind"] == fg.KIND_MASKED
        cands = [None]
        for bm, bn in tiles if layout else ():
            ntiles = -(-t["M"] // bm) * -(-t["N"] // bn)
            for sp in range(1, 17):
                if -(-nkb // -(-nkb // sp)) == sp and (sp == 1 or ntiles * sp <= 512):
                    cands.append((bm, bn, sp, 0))
        for bm, bn in () if layout else tiles:
            if not masked and ((t["M"] <= 128 and bm > 128) or (t["M"] > 128 and bm < 128)):
                continue
            ntiles = -(-t["M"] // bm) * -(-t["N"] // bn)
            rem = ntiles % 256
            for sp in ((1, 2, 3, 4, 6, 8) if masked else range(1, 9)):
                if -(-nkb // -(-nkb // sp)) != sp:
                    continue
                if masked or ntiles * sp <= 1024 or sp == 1:
                    cands.append((bm, bn, sp, 0))
                if not masked and sp > 1 and ntiles > 256 and rem > 0 and rem * sp <= 256:
                    cands.append((bm, bn, sp, ntiles - rem))
        res = {}
        for cfg in cands:
            if cfg is not None:
                try:
                    with fg.force_config(*cfg[:3], full_tiles=cfg[3]):
                        t["fn"]()
                except Exception:
                    continue   # a plan the library rejects (too many split tiles)
            evs = []
            for r in range(args.rounds + 1):
                ev = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                for ci, c in enumerate(cases):
                    if ci == ti:
                        ev[0].record()
                        if cfg is None:
                            c["fn"]()
                        else:
                            with fg.force_config(*cfg[:3], full_tiles=cfg[3]):
                                c["fn"]()
                        ev[1].record()
                    else:
                        c["fn"]()
                evs.append(ev)
            torch.cuda.synchronize()
            ms = float(np.median([a.elapsed_time(b) for a, b in evs[1:]]))
            key = "auto" if cfg is None else ("%dx%d s%d" % cfg[:3] if masked or layout else "%dx%d s%d f%d" % cfg)
            res[key] = round(ms * 1e3, 2)
        print(json.dumps({"kind": args.plan_sweep, "case": t["key"], "all": res}), flush=True)


def plan_table(args):
    """--plan-table LOG...: average (geometric mean) the --plan-sweep logs of several runs
    into profiles/planner_sweep.json, the measured table the planner is checked against."""
    import math
    import platform
    acc = {"dense": {}, "masked": {}, "layout": {}}
    runs = {"dense": 0, "masked": 0, "layout": 0}
    for f in args.plan_table:
        with open(f) as fh:
            kinds = set()
            for line in fh:
                if not line.startswith("{"):
                    continue
                d = json.loads(line)
                kinds.add(d["kind"])
                tab = acc[d["kind"]].setdefault(",".join(str(x) for x in d["case"]), {})
                for k, v in d["all"].items():
                    if k != "auto":
                        tab.setdefault(k, []).append(v)
            for k in kinds:
                runs[k] += 1
    out = {"what": "event time (us) of every plan of each case, forced for that call only inside the benchmark's "
                   "sequence of calls; geometric mean over the runs",
           "command": "python bench.py --plan-sweep dense --rounds 12 > LOG (twice, likewise --plan-sweep masked "
                      "and layout); python bench.py --plan-table LOG...",
           "kernel_sha": kernel_source_hash(), "runs": runs}
    for kind in ("dense", "masked", "layout"):
        out[kind] = {case: {k: round(math.exp(sum(math.log(x) for x in v) / len(v)), 2) for k, v in tab.items()}
                     for case, tab in acc[kind].items()}
    with open(os.path.join(ROOT, "profiles", "planner_sweep.json"), "w") as fh:
        json.dump(out, fh, indent=1, sort_keys=True)
    print(json.dumps({k: out[k] for k in ("what", "runs", "kernel_sha")}))


def grouped_bench(args):
    """--workload grouped: the M-grouped workloads alone (one step = every case once).
    Prints one JSON line (not the default benchmark, which includes these cases too)."""
    import torch
    dev = torch.device("cuda:0")
    ue = bool(args.ue8m0)
    cases = grouped_cases(dev, ue)
    ms_per_step, per = time_cases([c["fn"] for c in cases], args.steps, args.warmup)
    total = sum(c["flops"] for c in cases)
    out = {"metric": METRIC, "value": round(total / (ms_per_step * 1e-3) / 1e12, 2), "unit": "TFLOP/s",
           "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "e4m3",
           "data": "synthetic",
           "config": {"workload": ("UE8M0-scaled " if ue else "") + "M-grouped FP8 NT GEMMs: contiguous (4x8192 rows "
                                  "N=4096 K=7168; 8x4096 rows N=7168 K=2048), masked decode (G in 1..16, M_max 4096, "
                                  "masked_m in [179,333]), MoE FFN pair (4096 tokens, 256 experts, top-8 Zipf 1.1)"},
           "per_case": grouped_rows(cases, per)}
    print(json.dumps(out), flush=True)


QUANT_CASES = [(4096, 7168, "bf16"), (4096, 2048, "bf16"), (4096, 16384, "bf16"), (32768, 7168, "bf16"),
               (53376, 2048, "bf16"), (4096, 7168, "fp32"), (53376, 2048, "swiglu-bf16")]


def quant_bench(args):
    """--workload quant: the 1x128 activation quantiser on the activation shapes that feed
    the GEMMs (dense M=4096 at K = 7168, 2048, 16384; the MoE gate+up input of 32768
    routed rows at K=7168; the MoE down input of 53376 padded rows at K=2048; one FP32
    input; and SwiGLU fused with the quantisation on the MoE down input, reading the
    53376 x 4096 BF16 gate+up output). HBM-bound: bytes = input once + e4m3 codes + FP32
    scales. One JSON line."""
    import torch
    import moe_grouped_gemm_fp32_amd as fg

    dev = torch.device("cuda:0")
    cases = []
    for i, (M, K, dt) in enumerate(QUANT_CASES):
        g = torch.Generator(device=dev)
        g.manual_seed(7000 + i)
        swiglu = dt.startswith("swiglu")
        X = torch.randn(M, 2 * K if swiglu else K, generator=g, device=dev, dtype=torch.float32)
        if dt.endswith("bf16"):
            X = X.to(torch.bfloat16)
        Q = torch.empty(M, K, dtype=torch.uint8, device=dev)
        sa = torch.empty(K // 128, fg.scale_ld(M), dtype=torch.float32, device=dev)
        nbytes = X.numel() * X.element_size() + M * K + M * (K // 128) * 4
        if swiglu:
            fn = lambda X=X, Q=Q, sa=sa: fg.swiglu_quantize_1x128(X, None, Q, sa)
        else:
            fn = lambda X=X, Q=Q, sa=sa: fg.quantize_1x128(X, Q, sa)
        cases.append(dict(name="%s %dx%d" % (dt, M, K), fn=fn, bytes=nbytes))
    torch.cuda.synchronize()

    def step(events=None):
        for i, c in enumerate(cases):
            if events is not None:
                events[i][0].record()
            c["fn"]()
            if events is not None:
                events[i][1].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    ms_per_step = (time.perf_counter() - t0) / args.steps * 1e3
    step()
    all_ev = []
    for _ in range(args.steps):
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in cases]
        step(ev)
        all_ev.append(ev)
    torch.cuda.synchronize()
    per = [0.0] * len(cases)
    for ev in all_ev:
        for i, (a, b) in enumerate(ev):
            per[i] += a.elapsed_time(b)
    rows, total = [], 0
    for i, c in enumerate(cases):
        ms = per[i] / args.steps
        total += c["bytes"]
        gbs = c["bytes"] / (ms * 1e-3) / 1e9
        rows.append({"case": c["name"], "us": round(ms * 1e3, 2), "gbs": round(gbs, 1),
                     "frac": round(gbs / PEAK_HBM_GBS, 4), "ideal_us": round(c["bytes"] / PEAK_HBM_GBS / 1e3, 2),
                     "algo_bytes": c["bytes"]})
    out = {"metric": "1x128 activation quantisation HBM GB/s, 1xMI355X, % of HBM roofline",
           "value": round(total / (ms_per_step * 1e-3) / 1e9, 1), "unit": "GB/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "e4m3", "data": "synthetic",
           "config": {"workload": "1x128 FP32-scaled e4m3 quantisation of N(0,1) activations feeding the GEMMs",
                      "cases": [c["name"] for c in cases]},
           "per_case": rows}
    print(json.dumps(out), flush=True)


# MoE weight-gradient shapes of the K-grouped TN GEMM: per local expert, dW_gate+up [4096,
# 7168] = dH^T X and dW_down [7168, 2048] = dY^T H, reduced over that expert's tokens
KGROUP_CASES = [(4096, 7168), (7168, 2048)]
KGROUP_EXPERTS = 8


def kgrouped_work(M, N, ks, accumulate=False):
    """Algorithmic FLOPs and HBM bytes of one K-grouped call: every operand byte and scale
    read once, D written once (and read once when accumulating)."""
    K = sum(ks)
    flops = 2.0 * M * N * K
    nbytes = K * (M + N) + (K // 128) * (M + N) * 4 + len(ks) * M * N * 4 * (2 if accumulate else 1)
    return flops, nbytes


def kgrouped_cpu_baseline(ks, M, N):
    """The oracle (as it stands) on a bounded sample: M x N outputs of every group."""
    import numpy as np
    import oracle
    import synth
    c = synth.k_grouped_case([k for k in ks], M, N, seed=98, device="cpu")
    args = [c[k].numpy() for k in ("A", "sa", "B", "sb")]
    t0 = time.perf_counter()
    oracle.k_grouped_tn(*args, c["ks"])
    dt = time.perf_counter() - t0
    flops = 2.0 * M * N * sum(c["ks"])
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": blas_threads(),
            "kind": "oracle", "seconds": round(dt, 3),
            "sample": "oracle k_grouped_tn on the same %d expert segments (K=%d) at M=%d, N=%d" % (
                len(ks), sum(c["ks"]), M, N)}


def kgrouped_bench(args):
    """--workload kgrouped: the K-grouped TN GEMM (MoE weight gradient) on the two expert
    projections, 8 local experts with 1024..3072 tokens each (K ~ 16.5K), FP32 output
    (--ue8m0: power-of-two scales through the UE8M0 call). One JSON line; value = FP8
    TFLOP/s over both calls."""
    import torch
    import moe_grouped_gemm_fp32_amd as fg
    import synth

    dev = torch.device("cuda:0")
    tokens = synth.k_grouped_tokens(KGROUP_EXPERTS, seed=9600)
    cases = []
    for i, (M, N) in enumerate(KGROUP_CASES):
        c = synth.k_grouped_case(tokens, M, N, seed=9700 + i, device=dev, kind="pow2" if args.ue8m0 else "normal")
        D = torch.zeros(len(c["ks"]), M, N, dtype=torch.float32, device=dev)
        flops, nbytes = kgrouped_work(M, N, c["ks"], args.accumulate)
        fn = (lambda c=c, D=D: fg.k_grouped_fp8_gemm_tn_contiguous(c["A"], c["sa"], c["B"], c["sb"], D, c["ks"],
                                                                    accumulate=args.accumulate, ue8m0=args.ue8m0))
        cases.append(dict(name="wgrad %dx%d G=%d K=%d" % (M, N, len(c["ks"]), c["K"]), fn=fn, flops=flops,
                          bytes=nbytes, ks=c["ks"]))
    torch.cuda.synchronize()

    def step(events=None):
        for i, c in enumerate(cases):
            if events is not None:
                events[i][0].record()
            c["fn"]()
            if events is not None:
                events[i][1].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    ms_per_step = (time.perf_counter() - t0) / args.steps * 1e3
    step()
    all_ev = []
    for _ in range(args.steps):
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in cases]
        step(ev)
        all_ev.append(ev)
    torch.cuda.synchronize()
    per = [0.0] * len(cases)
    for ev in all_ev:
        for i, (a, b) in enumerate(ev):
            per[i] += a.elapsed_time(b)
    rows, total = [], 0.0
    for i, c in enumerate(cases):
        ms = per[i] / args.steps
        total += c["flops"]
        tf = c["flops"] / (ms * 1e-3) / 1e12
        gbs = c["bytes"] / (ms * 1e-3) / 1e9
        rows.append({"case": c["name"], "us": round(ms * 1e3, 2), "tflops": round(tf, 1),
                     "frac": round(tf / PEAK_FP8_TFLOPS, 4), "hbm_gbs": round(gbs, 1),
                     "algo_flops": c["flops"], "algo_bytes": c["bytes"]})
    dom = max(range(len(cases)), key=lambda i: per[i])
    r = rows[dom]
    traffic = None
    tpath = os.path.join(ROOT, "profiles", "traffic_kgrouped.json")
    if os.path.exists(tpath) and not args.accumulate and not args.ue8m0:
        with open(tpath) as fh:
            tk = json.load(fh)
        key = "%d,%d" % KGROUP_CASES[dom]
        if tk.get("kernel_sha") == kernel_source_hash() and key in tk["cases"]:  # this very kernel only
            traffic = tk["cases"][key]["bytes_per_launch"]
    out = {"metric": "K-grouped FP8 GEMM (MoE weight gradient) TFLOP/s, 1xMI355X, % of FP8 dense MFMA peak",
           "value": round(total / (ms_per_step * 1e-3) / 1e12, 1), "unit": "TFLOP/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "e4m3", "data": "synthetic",
           "config": {"workload": "K-grouped TN GEMM, 8 experts x 1024..3072 tokens, dW gate+up 4096x7168 and "
                                  "dW down 7168x2048, FP32 out%s%s" % (", accumulating" if args.accumulate else "",
                                                            ", UE8M0 scales" if args.ue8m0 else ""),
                      "cases": [c["name"] for c in cases]},
           "roofline": {"bound": "mfma", "achieved": r["tflops"], "peak": PEAK_FP8_TFLOPS, "unit": "TFLOP/s",
                        "frac": r["frac"], "traffic": traffic, "kernel": "fp8_k_grouped_tn_kernel",
                        "case": r["case"]},
           "per_case": rows}
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = kgrouped_cpu_baseline(cases[0]["ks"], 5120, 5120)
    print(json.dumps(out), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--workload", choices=("dense", "ue8m0", "grouped", "quant", "kgrouped"), default="dense",
                    help="dense: the 18 DeepSeek-V3-like shapes (default); ue8m0: the same shapes with "
                         "power-of-two (UE8M0) scales through fp8_gemm_nt_ue8m0; grouped: contiguous, masked, "
                         "MoE; quant: the 1x128 activation quantiser; kgrouped: the K-grouped TN GEMM "
                         "(MoE weight gradient)")
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--shapes", type=str, default=None, help="'M,N,K;M,N,K' instead of the default list")
    ap.add_argument("--plan-sweep", choices=("dense", "masked", "layout"),
                    help="time every plan of each dense shape / masked decode case / dense shape in the TN "
                         "layout (planner fitting)")
    ap.add_argument("--rounds", type=int, default=12, help="rounds per plan of --plan-sweep")
    ap.add_argument("--plan-table", nargs="+", metavar="LOG",
                    help="average --plan-sweep logs into profiles/planner_sweep.json")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-grouped", action="store_true",
                    help="default run without the small dense case and the grouped (contiguous, masked, MoE) rows")
    ap.add_argument("--with-c", action="store_true",
                    help="dense workload as D = C + A B^T with a BF16 C per shape (fp8_gemm_nt_c)")
    ap.add_argument("--packed", action="store_true",
                    help="with --workload ue8m0: the scales packed four UE8M0 codes a word through "
                         "fp8_gemm_nt_ue8m0_packed")
    ap.add_argument("--ue8m0", action="store_true",
                    help="with --workload grouped or kgrouped: power-of-two (UE8M0) scales through the *_ue8m0 calls")
    ap.add_argument("--accumulate", action="store_true", help="with --workload kgrouped: D += A^T B")
    ap.add_argument("--layout", choices=("nt", "tn", "nn", "tt"), default="nt",
                    help="dense workload in another memory layout: the K-major operands stored [K, rows] "
                         "and fp8_gemm_tn / fp8_gemm_nn / fp8_gemm_tt called")
    ap.add_argument("--kg-pmc-summary", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="build profiles/traffic_kgrouped.json from rocprofv3 --pmc runs of --workload kgrouped")
    ap.add_argument("--traffic-file", default=os.path.join(ROOT, "profiles", "traffic_dense_shapes.json"))
    ap.add_argument("--copy-mb", type=int, default=0, help="only run a plain copy of this many MiB")
    ap.add_argument("--trace-summary", metavar="TRACE_DIR", help="per-shape durations from a rocprofv3 trace")
    ap.add_argument("--counter-summary", metavar="PMC_DIR", help="per-shape counter means from a rocprofv3 --pmc run")
    ap.add_argument("--pmc-summary", nargs=4, metavar=("FETCH_DIR", "WRITE_DIR", "COPY_FETCH_DIR", "COPY_WRITE_DIR"),
                    help="build the traffic table from rocprofv3 --pmc output directories")
    args = ap.parse_args()

    if args.plan_table:
        plan_table(args)
        return
    if args.plan_sweep:
        plan_sweep(args)
        return
    if args.pmc_summary:
        pmc_summary(args, parse_shapes(args.shapes) if args.shapes else CONFIG2)
        return
    if args.kg_pmc_summary:
        kg_pmc_summary(args)
        return
    if args.counter_summary:
        if args.workload == "kgrouped":
            counter_summary_cases(args.counter_summary, "k_grouped_tn_kernel",
                                  ["wgrad %dx%d" % mn for mn in KGROUP_CASES])
        elif args.workload == "grouped":   # the first dispatch is the untimed gate+up call
            counter_summary_cases(args.counter_summary, "fp8_gemm_kernel", GROUPED_CASES, skip=1)
        else:
            counter_summary(args.counter_summary, parse_shapes(args.shapes) if args.shapes else CONFIG2,
                            args.steps, args.warmup,
                            "fp8_gemm_kernel" if args.layout == "nt" else "fp8_k_grouped_tn_kernel")
        return
    if args.trace_summary:
        if args.workload == "grouped":
            trace_summary_grouped(args.trace_summary, args.steps)
        elif args.workload == "kgrouped":
            trace_summary_cases(read_trace(args.trace_summary, "k_grouped_tn_kernel"),
                                ["wgrad %dx%d" % mn for mn in KGROUP_CASES], args.steps)
        else:
            trace_summary(args.trace_summary, parse_shapes(args.shapes) if args.shapes else CONFIG2,
                          args.steps, args.warmup,
                          "fp8_gemm_kernel" if args.layout == "nt" else "fp8_k_grouped_tn_kernel")
        return
    if args.copy_mb:
        copy_only(args)
        return

    if args.gpus != 1:
        print(json.dumps({"error": "the benchmark and the library run on one GPU; --gpus %d is not supported" % args.gpus}))
        sys.exit(2)

    if args.workload == "grouped":
        grouped_bench(args)
        return
    if args.workload == "quant":
        quant_bench(args)
        return
    if args.workload == "kgrouped":
        kgrouped_bench(args)
        return

    import torch
    import moe_grouped_gemm_fp32_amd as fg
    import synth

    dev = torch.device("cuda:0")
    shapes = parse_shapes(args.shapes) if args.shapes else CONFIG2
    ue8m0 = args.workload == "ue8m0"
    tn = args.layout != "nt"   # one of the other memory layouts
    if tn and args.with_c:
        sys.exit("--layout %s takes no C" % args.layout)
    layout_fn = {"tn": "fp8_gemm_tn", "nn": "fp8_gemm_nn", "tt": "fp8_gemm_tt"}.get(args.layout)
    packed = ue8m0 and args.packed
    if args.packed and not ue8m0:
        sys.exit("--packed goes with --workload ue8m0")
    gemm = fg.fp8_gemm_nt_ue8m0_packed if packed else fg.fp8_gemm_nt_ue8m0 if ue8m0 else fg.fp8_gemm_nt
    cases = []
    for i, (M, N, K) in enumerate(shapes):
        c = synth.dense_case(M, N, K, seed=2000 + i, device=dev, a_std=1.0, b_std=0.02,
                             kind="pow2" if ue8m0 else "normal")
        if packed:  # sa [K/128, M] -> [ceil(K/512), M], sb [N/128, K/128] -> [N/128, ceil(K/512)]
            c["sa"] = synth.pack_ue8m0(c["sa"], 0)
            c["sb"] = synth.pack_ue8m0(c["sb"], 1)
        c["ws"] = fg.make_workspace(fg.KIND_DENSE, M, N, K, device=dev)
        c["C"] = (torch.randn(M, N, generator=synth.make_generator(2500 + i, dev), device=dev) * 0.1).to(
            torch.bfloat16) if args.with_c else None
        c["cfg"] = fg.query_config(fg.KIND_DENSE, M, N, K)
        if tn:  # the same operands, those the layout makes K-major stored [K, rows] (padded to 16 bytes)
            if args.layout in ("tn", "tt"):
                At = torch.zeros(K, (M + 15) // 16 * 16, dtype=torch.uint8, device=dev)
                At[:, :M] = c["A"].t()
                c["A"] = At
            if args.layout in ("tn", "nn"):
                Bt = torch.zeros(K, (N + 15) // 16 * 16, dtype=torch.uint8, device=dev)
                Bt[:, :N] = c["B"].t()
                c["B"] = Bt
            c["ws"] = fg.make_workspace(fg.KIND_LAYOUT, M, N, K, device=dev)
            c["cfg"] = fg.query_config(fg.KIND_LAYOUT, M, N, K)
        cases.append(c)
    torch.cuda.synchronize()

    def call(c):
        if tn:
            getattr(fg, layout_fn)(c["A"], c["sa"], c["B"], c["sb"], c["D"], ue8m0=ue8m0, workspace=c["ws"])
        elif c["C"] is not None:
            fg.fp8_gemm_nt(c["A"], c["sa"], c["B"], c["sb"], c["D"], c["ws"], C=c["C"])
        else:
            gemm(c["A"], c["sa"], c["B"], c["sb"], c["D"], c["ws"])

    ms_per_step, per_ms = time_cases([(lambda c=c: call(c)) for c in cases], args.steps, args.warmup)
    per = [[ms * args.steps] for ms in per_ms]
    traffic = {}
    if os.path.exists(args.traffic_file):
        with open(args.traffic_file) as f:
            tr = json.load(f)
        if tr.get("kernel_sha") == kernel_source_hash() and not ue8m0 and not args.with_c and not tn:  # this very kernel only
            traffic = tr.get("shapes", {})

    total_flops = 0.0
    rows = []
    for i, ((M, N, K), c) in enumerate(zip(shapes, cases)):
        flops, nbytes = algo_work(M, N, K, scale_bytes=1.0 if packed else 4.0)
        if args.with_c:
            nbytes += 2 * M * N  # C read once
        total_flops += flops
        ms = per[i][0] / args.steps
        bound, t_ideal = classify(flops, nbytes)
        tflops = flops / (ms * 1e-3) / 1e12
        gbs = nbytes / (ms * 1e-3) / 1e9
        frac = (tflops / PEAK_FP8_TFLOPS) if bound == "mfma" else (gbs / PEAK_HBM_GBS)
        rows.append({"M": M, "N": N, "K": K, "us": round(ms * 1e3, 2), "tflops": round(tflops, 1),
                     "gbs": round(gbs, 1), "bound": bound, "frac": round(frac, 4),
                     "ideal_us": round(t_ideal * 1e6, 2), "tile": "%dx%d" % (c["cfg"]["block_m"], c["cfg"]["block_n"]),
                     "split_k": c["cfg"]["split_k"], "algo_bytes": nbytes, "algo_flops": flops})
    value = total_flops / (ms_per_step * 1e-3) / 1e12

    dom = max(rows, key=lambda r: r["us"])
    key = "%d,%d,%d" % (dom["M"], dom["N"], dom["K"])
    tr = traffic.get(key)
    if dom["bound"] == "mfma":
        roof = {"bound": "mfma", "achieved": dom["tflops"], "peak": PEAK_FP8_TFLOPS, "unit": "TFLOP/s",
                "frac": round(dom["tflops"] / PEAK_FP8_TFLOPS, 4)}
    else:
        roof = {"bound": "hbm", "achieved": dom["gbs"], "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(dom["gbs"] / PEAK_HBM_GBS, 4)}
    roof["traffic"] = tr["bytes_per_launch"] if tr else None
    roof["kernel"] = "%s M=%d N=%d K=%d tile %s split %d" % (
        "fp8_k_grouped_tn_kernel (dense %s)" % args.layout.upper() if tn else "fp8_gemm_kernel", dom["M"], dom["N"], dom["K"], dom["tile"],
        dom["split_k"])
    roof["avg_us"] = dom["us"]
    roof["algo_per_launch"] = dom["algo_flops"] if dom["bound"] == "mfma" else dom["algo_bytes"]

    roof["avg_us_source"] = ("mean of HIP event pairs around each launch, recorded on the launch stream over "
                             "the timed steps")

    extra_rows = []
    default_run = not ue8m0 and not args.with_c and not tn and not args.shapes
    if default_run:
        for r in rows:
            r["config"] = "dense DeepSeek-V3 shape list"
        # the small dense case: launch-latency-bound (its ideal time is ~0.03 us), so its
        # row reports the per-call time and no roofline fraction
        sm = synth.dense_case(128, 256, 512, seed=1001, device=dev)
        f_s, b_s = algo_work(128, 256, 512)
        # 200 back-to-back calls through the C ABI with pre-bound arguments between two
        # events: the host issues a call in a few microseconds, so the GPU sets the pace
        import ctypes
        vp = ctypes.c_void_p
        cargs = (vp(sm["A"].data_ptr()), sm["A"].stride(0), vp(sm["sa"].data_ptr()), sm["sa"].stride(0),
                 vp(sm["B"].data_ptr()), sm["B"].stride(0), vp(sm["sb"].data_ptr()), vp(sm["D"].data_ptr()),
                 sm["D"].stride(0), 128, 256, 512, None, 0, vp(torch.cuda.current_stream().cuda_stream))
        raw = fg.lib().fp8_gemm_nt
        assert raw(*cargs) == 0
        n_small, reps = N_SMALL, []
        for _ in range(SMALL_REPS):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            e0.record()
            for _ in range(n_small):
                raw(*cargs)
            e1.record()
            torch.cuda.synchronize()
            reps.append(e0.elapsed_time(e1) / n_small)
        sm_ms = sorted(reps)[len(reps) // 2]
        extra_rows.append({"config": "dense small", "M": 128, "N": 256, "K": 512, "us": round(sm_ms * 1e3, 2),
                           "tflops": round(f_s / sm_ms / 1e9, 2), "gbs": round(b_s / sm_ms / 1e6, 1),
                           "bound": "latency", "frac": None,
                           "note": "launch-latency-bound (ideal %.3f us): per-call time of 200 back-to-back calls, "
                                   "no roofline fraction" % (b_s / 8e12 * 1e6),
                           "algo_bytes": b_s, "algo_flops": f_s})
        if not args.no_grouped:
            gcases = grouped_cases(dev)
            _, gper = time_cases([c["fn"] for c in gcases], args.steps, args.warmup)
            extra_rows += grouped_rows(gcases, gper)

    cpu = None
    if not args.no_cpu_baseline and default_run:
        cpu = cpu_baseline()

    out = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "e4m3",
        "data": "synthetic",
        "config": {"workload": "dense FP8 %s GEMM with 1x128/128x128 %s scales and BF16 output over %d "
                               "DeepSeek-V3-like shapes (M in {64,128,4096} x (N,K) list)"
                               % (args.layout.upper(), "packed UE8M0 (four codes a word)" if packed else
                                  "UE8M0 (power-of-two)" if ue8m0 else "FP32", len(shapes))
                               + (", D = C + A B^T with a BF16 C" if args.with_c else "")
                               + (" (%s)" % layout_fn if tn else ""),
                   "shapes": ["%dx%dx%d" % s for s in shapes]},
        "roofline": roof,
        "cpu_baseline": cpu,
        "per_shape": rows + extra_rows,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
