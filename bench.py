#!/usr/bin/env python3
"""Benchmark of libwqmm on one MI355X.

Headline workload (one JSON line on stdout): the f16-weight decode GEMV suite
at hidden 2048, M = 1, (N, K) = (6144, 2048) gate/up, (2048, 6144) down,
(2048, 2048) o_proj and (151936, 2048) LM head; A ~ N(0,1) f32, B ~ N(0,0.02)
cast to f16 on the GPU, seed 0.  One step runs the four GEMVs once through
wq_matmul.  ``value`` = weight bytes of all timed steps / timed wall time
(GB/s), inputs resident in HBM.  Every weight matrix is rotated over enough
distinct copies (>= 1 GiB in total) that each launch reads cold from HBM
rather than from the 256 MB Infinity Cache.

``roofline`` is for the dominant kernel, the LM-head GEMV: its algorithmic
bytes (N*K*2 weight bytes) over its average launch duration, measured with
HIP events on the stream it runs on around a burst of back-to-back LM-head
launches (the suite's rotated weights) right after the timed region; the
per-launch event pairs inside the timed region are reported beside it (they
add a marker and a dispatch latency per launch).  ``cpu_baseline`` times the CPU oracle (all host cores it uses) on the
same suite.  ``secondary`` reports the other configurations: the Q8_0 and
Q4_0 decode suites, the f16 prefill GEMM at M = 512, the Q8_0 and Q4_0 M
sweeps, the fused residual and SwiGLU epilogues against the same product
followed by separate element-wise kernels, the fused LM-head GEMV + top-k
against the GEMV alone and the GEMV followed by a top-k pass, the split-KV decode
attention (KV bytes GB/s at 4K-128K tokens), the 1024x1024 f16 GEMV, a plain
device copy, and ``read_ceiling``: a read-only kernel (wq_read_probe, the
GEMVs' 128-bit non-temporal loads and nothing else) timed on every byte size
a bandwidth-bound row reads, rotated over >= 1 GiB of copies like the
weights.  Every decode GEMV is reported against both the 8 TB/s peak and the
plain read of its own byte count.  Q4_0
weights are synthetic bytes (random codes and scales) since no Q4_0 encoder is
given.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "decode GEMV weight GB/s (% HBM peak); prefill GEMM TFLOP/s (% MFMA peak)"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
FP32_MFMA_PEAK_TFLOPS = 157.3  # MI355X dense fp32 matrix
# The f16 matrix-core routes (stream, f16 matrix-core GEMM) issue two f16
# products (A's hi and lo halves) per product of the f32 problem: their compute
# roofline is half the MI355X dense f16 matrix peak (2.5 PFLOP/s).
F16_PAIR_PEAK_TFLOPS = 2500.0 / 2
ROTATE_BYTES = 1 << 30
WARM_GPU_S = 0.05  # sustained GPU time before a timed burst
DECODE = [("gate_up", 6144, 2048), ("down", 2048, 6144), ("o_proj", 2048, 2048), ("lm_head", 151936, 2048)]
PREFILL = [(512, 6144, 2048), (512, 2048, 6144)]
SWEEP_SHAPES = [(11008, 4096), (4096, 11008)]
SWEEP_M = [1, 2, 4, 8, 16, 64, 512]
ROUTE_NAMES = {1: "gemv", 2: "gemm", 3: "small_m", 4: "stream", 5: "gemm_f16_pair"}
F16_PAIR_ROUTES = (4, 5)


def compute_peak(route):
    """Matrix peak (TFLOP/s) of the products a route issues."""
    return F16_PAIR_PEAK_TFLOPS if route in F16_PAIR_ROUTES else FP32_MFMA_PEAK_TFLOPS


TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "gemv_f16_lm_head_151936x2048.md")
GEMV_SOURCES = [os.path.join(ROOT, "gemm_wq_gemv_amd", "csrc", f) for f in ("gemv.hip", "wq_internal.h")]


def gemv_source_hash() -> str:
    import hashlib
    h = hashlib.sha256()
    for path in GEMV_SOURCES:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def recorded_traffic():
    """HBM bytes per LM-head launch from the committed rocprofv3 PMC summary
    (FETCH_SIZE + WRITE_SIZE, copy-calibrated), if it was taken on the current
    kernel sources; otherwise None."""
    try:
        text = open(TRAFFIC_PROFILE).read()
    except OSError:
        return None
    fields = dict(line.split(":", 1) for line in text.splitlines() if line.startswith(("source_sha256:", "traffic_bytes_per_launch:")))
    if fields.get("source_sha256", "").strip() != gemv_source_hash():
        return None
    try:
        return int(fields["traffic_bytes_per_launch"].strip())
    except (KeyError, ValueError):
        return None


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--seed", type=int, default=0)
    p.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    p.add_argument("--no-secondary", action="store_true", help="headline suite only")
    p.add_argument("--only", choices=["f16", "q8", "q4", "prefill", "sweep", "epi", "topk", "attn", "counters"],
                   default=None, help="run one workload only (for profiling); prints no headline line")
    p.add_argument("--summarize", nargs="+", metavar="CSV", default=None,
                   help="print per-kernel medians (a rocprofv3 kernel_trace.csv) or counter tables "
                        "(counter_collection.csv files, with the kernel_trace.csv of the same runs) and exit")
    return p.parse_args()


# ------------------------------------------------------------ profiling aids --
# COUNTER_WORKLOAD: (label, launcher) pairs run by `--only counters`, a fixed
# set of launches of every kernel family whose counters the profiles summarise,
# each on weights rotated over >= 1 GiB, plus a 1 GiB device copy whose
# FETCH_SIZE / WRITE_SIZE calibrate the byte counters.
COUNTER_REPEAT = 12


def counter_workload(torch, wq, wqgen, seed):
    F16, Q8, Q4 = wq.WQ_FMT_F16, wq.WQ_FMT_Q8_0, wq.WQ_FMT_Q4_0

    def rotated(n, k, fmt):
        if fmt == F16:
            b0 = wq.pack_f16(torch.from_numpy(wqgen.weights(n, k, seed)).cuda())
        elif fmt == Q4:
            b0 = torch.from_numpy(wqgen.q4_0_bytes(n, k, seed)).cuda()
        else:
            b0 = wq.quantize_q8_0(torch.from_numpy(wqgen.weights(n, k, seed)).cuda())
        nb = wq.weight_bytes(n, k, fmt)
        return [b0] + [b0.clone() for _ in range(max(1, math.ceil(ROTATE_BYTES / nb)) - 1)]

    def product(label, m, n, k, fmt, route=wq.WQ_ROUTE_AUTO):
        bs = rotated(n, k, fmt)
        a = torch.from_numpy(wqgen.activations(m, k, seed)).cuda()
        c = torch.empty((m, n), device="cuda")
        log(f"counters: {label}")
        prev = wq.wq_set_forced_route(route)
        for i in range(COUNTER_REPEAT):
            wq.wq_matmul(a, bs[i % len(bs)], c, m, n, k, fmt)
        torch.cuda.synchronize()
        wq.wq_set_forced_route(prev)
        del bs

    nb = 1 << 30
    src = torch.empty(nb // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    log("counters: 1 GiB device copy (byte-counter calibration)")
    for _ in range(4):
        dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst
    product("f16 LM head 151936x2048", 1, 151936, 2048, F16)
    product("Q8_0 LM head 151936x2048 (register chunks)", 1, 151936, 2048, Q8)
    product("Q8_0 GEMV 4096x11008 (register chunks)", 1, 4096, 11008, Q8)
    product("Q8_0 GEMV 11008x4096 (register chunks)", 1, 11008, 4096, Q8)
    product("Q8_0 GEMV 6144x2048 (staged)", 1, 6144, 2048, Q8)
    product("Q4_0 LM head 151936x2048 (staged)", 1, 151936, 2048, Q4)
    product("Q4_0 GEMV 11008x4096 (register chunks)", 1, 11008, 4096, Q4)
    product("Q4_0 GEMV 4096x11008 (register chunks)", 1, 4096, 11008, Q4)
    product("Q8_0 stream 2x11008x4096", 2, 11008, 4096, Q8)
    product("Q8_0 stream 8x4096x11008", 8, 4096, 11008, Q8)
    product("Q8_0 stream 16x4096x11008", 16, 4096, 11008, Q8)
    product("Q8_0 stream 16x11008x4096", 16, 11008, 4096, Q8)
    product("Q8_0 small-M (fp32) 8x4096x11008", 8, 4096, 11008, Q8, wq.WQ_ROUTE_SKINNY)
    product("f16 small-M 4x11008x4096", 4, 11008, 4096, F16)
    product("Q8_0 GEMM 16x11008x4096", 16, 11008, 4096, Q8, wq.WQ_ROUTE_GEMM)
    product("f16 GEMM 512x6144x2048 (f16 matrix cores)", 512, 6144, 2048, F16)
    product("Q8_0 GEMM 512x4096x11008 (f16 matrix cores)", 512, 4096, 11008, Q8)
    product("f16 GEMM 512x6144x2048 (fp32 MFMA)", 512, 6144, 2048, F16, wq.WQ_ROUTE_GEMM)
    for fmt, key in ((F16, "f16"), (Q8, "Q8_0")):
        bs = rotated(151936, 2048, fmt)
        a = torch.from_numpy(wqgen.activations(1, 2048, seed)).cuda()
        vals = torch.empty(50, device="cuda")
        ids = torch.empty(50, dtype=torch.int32, device="cuda")
        log(f"counters: {key} LM-head top-50")
        for i in range(COUNTER_REPEAT):
            wq.wq_lm_head_topk(a, bs[i % len(bs)], 151936, 2048, fmt, 50, vals, ids)
        torch.cuda.synchronize()
        del bs
    D, hq, hkv, L = 256, 8, 2, 32768
    gen = torch.Generator(device="cuda")
    gen.manual_seed(seed)
    q = torch.randn((hq, D), device="cuda", generator=gen)
    out = torch.empty((hq, D), device="cuda")
    copies = max(2, math.ceil(ROTATE_BYTES / (2 * L * hkv * D * 2)))
    ks = [torch.randn((L, hkv * D), device="cuda", generator=gen).half().view(torch.int16) for _ in range(copies)]
    vs = [torch.randn((L, hkv * D), device="cuda", generator=gen).half().view(torch.int16) for _ in range(copies)]
    log("counters: decode attention f16 L=32768")
    for i in range(COUNTER_REPEAT):
        wq.wq_decode_attention(q, ks[i % copies], vs[i % copies], out, L, D, hq, hkv, wq.WQ_KV_F16, 0.0625)
    torch.cuda.synchronize()


def _kernel_short(name: str) -> str:
    """`ns::(anonymous namespace)::kernel<args>(params)` -> `kernel<args>`."""
    name = name.split("(")[0] if "(anonymous" not in name else name
    for pre in ("void ", "wq::", "(anonymous namespace)::"):
        name = name.replace(pre, "")
    if "(" in name:
        name = name[:name.index("(")]
    return name.strip()


def summarize(paths):
    """Markdown tables from rocprofv3 CSV output: per-kernel duration statistics
    (median first) from a kernel_trace.csv; from counter_collection.csv files, the
    per-dispatch counter means per (kernel, grid) -- FETCH_SIZE / WRITE_SIZE in
    bytes (KiB x 1024) -- next to the median duration of the same dispatches."""
    import csv
    import statistics
    from collections import defaultdict
    traces = [p for p in paths if p.endswith("kernel_trace.csv")]
    counters = [p for p in paths if p.endswith("counter_collection.csv")]
    for path in traces:
        dur = defaultdict(list)
        for r in csv.DictReader(open(path)):
            key = (_kernel_short(r["Kernel_Name"]), int(r["Grid_Size_X"]) // max(1, int(r["Workgroup_Size_X"])),
                   int(r["Workgroup_Size_X"]))
            dur[key].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
        print(f"Kernel durations from {os.path.basename(path)} (us; workgroups, lanes per workgroup)\n")
        print("| kernel | workgroups | lanes | dispatches | median | mean | min | max |")
        print("|---|---:|---:|---:|---:|---:|---:|---:|")
        for (k, g, w), v in sorted(dur.items(), key=lambda x: -sum(x[1])):
            print(f"| `{k}` | {g} | {w} | {len(v)} | {statistics.median(v):.2f} | {statistics.mean(v):.2f} | "
                  f"{min(v):.2f} | {max(v):.2f} |")
        print()
    for path in counters:
        vals = defaultdict(lambda: defaultdict(list))
        for r in csv.DictReader(open(path)):
            key = (_kernel_short(r["Kernel_Name"]), int(r["Grid_Size"]) // max(1, int(r["Workgroup_Size"])))
            vals[key][r["Counter_Name"]].append(float(r["Counter_Value"]))
        names = sorted({c for v in vals.values() for c in v})
        print(f"Counters from {os.path.basename(path)} (mean per dispatch; *_SIZE in bytes)\n")
        print("| kernel | workgroups | dispatches | " + " | ".join(names) + " |")
        print("|---|---:|---:|" + "---:|" * len(names))
        for (k, g), cs in sorted(vals.items()):
            n = max(len(x) for x in cs.values())
            cells = []
            for c in names:
                x = statistics.mean(cs[c]) if cs.get(c) else float("nan")
                cells.append(f"{x * 1024:,.0f}" if c.endswith("_SIZE") else f"{x:,.0f}")
            print(f"| `{k}` | {g} | {n} | " + " | ".join(cells) + " |")
        print()
        # Byte-counter calibration: the workload's first four 256-workgroup copy
        # dispatches, the 1 GiB device copies it makes before anything else.
        rows = sorted(csv.DictReader(open(path)), key=lambda r: int(r["Dispatch_Id"]))
        for c in names:
            if not c.endswith("_SIZE"):
                continue
            big = [float(r["Counter_Value"]) for r in rows
                   if r["Counter_Name"] == c and "copyBuffer" in r["Kernel_Name"]
                   and int(r["Grid_Size"]) // max(1, int(r["Workgroup_Size"])) == 256][:4]
            if big:
                print(f"1 GiB copy calibration: {c} = {statistics.mean(big):,.1f} KiB per dispatch over "
                      f"{len(big)} dispatches (1,048,576 KiB moved; scale factor "
                      f"{1_048_576 / statistics.mean(big):.4f})\n")


class Suite:
    """Decode GEMV suite in one format with rotated weight copies."""

    def __init__(self, wq, wqgen, torch, fmt, seed, host_weights):
        self.fmt = fmt
        self.items = []
        for name, n, k in DECODE:
            if fmt == wq.WQ_FMT_Q4_0:
                b0 = torch.from_numpy(wqgen.q4_0_bytes(n, k, seed)).cuda()
            else:
                wd = torch.from_numpy(host_weights[(n, k)]).cuda()
                b0 = wq.pack_f16(wd) if fmt == wq.WQ_FMT_F16 else wq.quantize_q8_0(wd)
                del wd
            nbytes = wq.weight_bytes(n, k, fmt)
            copies = max(2, math.ceil(ROTATE_BYTES / nbytes))
            bs = [b0] + [b0.clone() for _ in range(copies - 1)]
            a = torch.from_numpy(wqgen.activations(1, k, seed)).cuda()
            c = torch.empty((1, n), dtype=torch.float32, device="cuda")
            self.items.append(dict(name=name, n=n, k=k, bs=bs, a=a, c=c, bytes=nbytes))
        self.bytes_per_step = sum(it["bytes"] for it in self.items)
        torch.cuda.synchronize()

    def step(self, wq, i, events=None):
        """One pass over the suite; `events` = {item index: (start, end)} to bracket."""
        for j, it in enumerate(self.items):
            b = it["bs"][i % len(it["bs"])]
            ev = events.get(j) if events else None
            if ev is not None:
                ev[0].record()
            wq.wq_matmul(it["a"], b, it["c"], 1, it["n"], it["k"], self.fmt)
            if ev is not None:
                ev[1].record()


_SLEEP_CYCLES_PER_S = None


def hold_stream(torch, seconds):
    """Enqueue a spin kernel that keeps the stream busy for about `seconds`
    (torch.cuda._sleep counts GPU clock cycles; the rate is measured once)."""
    global _SLEEP_CYCLES_PER_S
    if _SLEEP_CYCLES_PER_S is None:
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda._sleep(100_000)
        a.record()
        torch.cuda._sleep(4_000_000)
        b.record()
        torch.cuda.synchronize()
        _SLEEP_CYCLES_PER_S = 4_000_000 / max(a.elapsed_time(b) / 1e3, 1e-4)
    torch.cuda._sleep(int(min(seconds, 0.5) * _SLEEP_CYCLES_PER_S))


def time_suite(torch, wq, suite, steps, warmup, bracket):
    """Times `steps` suite passes back to back on the GPU.  HIP events bracket
    the launches of the items listed in `bracket` only (events between kernels
    cost a few microseconds of GPU time each, so the other launches run back
    to back).  The Python binding validates its arguments on every call (tens
    of microseconds of host time per step), so a spin kernel sized from the
    warmup's host rate holds the stream while all timed steps are enqueued:
    the GPU then runs them without waiting for the host, as a compiled decode
    loop or a captured graph would.  Returns (timed seconds, host wall seconds
    including the hold, {item: mean launch seconds})."""
    t0 = time.perf_counter()
    for i in range(warmup):
        suite.step(wq, i)
    host_step = (time.perf_counter() - t0) / max(warmup, 1)
    torch.cuda.synchronize()
    ev = {j: [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
          for j in bracket}
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    hold = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    hold.record()
    hold_stream(torch, 1.5 * host_step * steps * (1 + len(bracket)) + 1e-3)
    start.record()
    t1 = time.perf_counter()
    for i in range(steps):
        suite.step(wq, warmup + i, {j: e[i] for j, e in ev.items()})
    host = time.perf_counter() - t1
    end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    if host > 0.9 * hold.elapsed_time(start) / 1e3:
        log(f"warning: host enqueue ({host * 1e3:.2f} ms) outlasted the stream hold; GPU time may include gaps")
    total = start.elapsed_time(end) / 1e3
    per = {j: sum(a.elapsed_time(b) for a, b in e) / steps / 1e3 for j, e in ev.items()}
    return total, wall, per


def time_launches(torch, fn, iters, warmup):
    """GPU seconds per launch of fn, at the clock the chip holds under
    sustained load.  The compute clock ramps up over about 20 ms of load and
    drops again after a few milliseconds of idle (the 512x6144x2048 f16 GEMM
    takes about 136 us just after idle and 119 us sustained; HBM-bound kernels
    do not move), so the warmup is W launches and then as many more as make
    about WARM_GPU_S of GPU time.  A spin kernel then holds the stream while
    the host enqueues the timed launches, so that per-call host overhead
    (Python binding and launch, about 10 us) does not leak into the GPU time
    of kernels shorter than that; it is sized from the warmup's host rate,
    so the GPU idles no longer than the enqueue takes."""
    w0, w1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    # One launch first: the first call of a kernel in the process loads its
    # code (milliseconds), which would inflate the per-launch estimate below
    # and cut the clock-ramp warmup short (measured: the 512x6144x2048 GEMM,
    # the first prefill shape, then timed at 135 us instead of 116 us).
    fn(0)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    w0.record()
    for i in range(warmup):
        fn(i)
    w1.record()
    host_call = (time.perf_counter() - t0) / max(warmup, 1)
    torch.cuda.synchronize()
    per = max(w0.elapsed_time(w1) / 1e3 / max(warmup, 1), 1e-6)
    extra = min(math.ceil(WARM_GPU_S / per), 20000)
    t0 = time.perf_counter()
    for i in range(extra):
        fn(i)
    backlog = max(0.0, extra * per - (time.perf_counter() - t0))  # GPU work still queued, at most
    e0, s, e = (torch.cuda.Event(enable_timing=True) for _ in range(3))
    e0.record()
    hold_stream(torch, 2e-4 + 1.5 * host_call * iters)
    s.record()
    t0 = time.perf_counter()
    for i in range(iters):
        fn(warmup + i)
    host = time.perf_counter() - t0
    e.record()
    torch.cuda.synchronize()
    if host > 0.9 * (e0.elapsed_time(s) / 1e3 + backlog):
        log(f"warning: host enqueue ({host * 1e3:.2f} ms) outlasted the stream hold; GPU time may include gaps")
    return s.elapsed_time(e) / 1e3 / iters


def read_ceiling(torch, wq, sizes, iters, warmup):
    """Plain-read time of each byte size in `sizes` (label -> bytes): the read
    probe over rotated copies totalling >= 1 GiB, best of 1, 2, 4 and 8 slabs of
    4 KiB per workgroup."""
    res = {}
    for label, nbytes in sizes.items():
        nb = (nbytes + 15) // 16 * 16
        copies = max(2, math.ceil(ROTATE_BYTES / nb))
        bufs = [torch.empty(nb, dtype=torch.uint8, device="cuda") for _ in range(copies)]
        for b in bufs:
            b.fill_(1)
        out = torch.empty((nb + 1023) // 1024, dtype=torch.int32, device="cuda")
        best = None
        for variant in (0, 1, 2, 3):
            t = time_launches(torch, lambda i: wq.wq_read_probe(bufs[i % copies], nb, out, variant), iters, warmup)
            if best is None or t < best[0]:
                best = (t, variant)
        res[label] = {"bytes": nbytes, "us": round(best[0] * 1e6, 2), "GB/s": round(nbytes / best[0] / 1e9, 1),
                      "slabs_per_workgroup": 1 << best[1]}
        del bufs, out
        torch.cuda.empty_cache()
    return res


def gemv_table(torch, wq, suite, fmt, iters, warmup, ceiling):
    """Each decode GEMV of a suite timed alone as a burst of back-to-back launches
    (rotated weights), against the 8 TB/s peak and the plain read of its bytes."""
    out = {}
    for it in suite.items:
        t = time_launches(torch, lambda i: wq.wq_matmul(it["a"], it["bs"][i % len(it["bs"])], it["c"], 1, it["n"],
                                                        it["k"], fmt), iters, warmup)
        gbs = it["bytes"] / t / 1e9
        ceil_gbs = ceiling.get(it["bytes"])
        out[it["name"]] = {"us": round(t * 1e6, 2), "GB/s": round(gbs, 1), "frac_hbm": round(gbs / HBM_PEAK_GBS, 4),
                           "frac_read_ceiling": round(gbs / ceil_gbs, 4) if ceil_gbs else None}
    return out


def epilogue_bench(torch, wq, wqgen, seed, iters, warmup):
    """Fused epilogues on the suite's FFN shapes (hidden 2048, intermediate 3072):
    gate||up [6144, 2048] with SwiGLU into [m, 3072], and down [2048, 6144] added
    into the residual stream, at M = 1 (decode) and M = 512 (prefill), for every
    format.  `unfused` is the same product through wq_matmul into a buffer
    followed by torch's element-wise silu * up or add (the extra pass over C
    that the fused call saves)."""
    import torch.nn.functional as F
    out = {}
    fmts = ((wq.WQ_FMT_F16, "f16"), (wq.WQ_FMT_Q8_0, "q8"), (wq.WQ_FMT_Q4_0, "q4"))
    for fmt, key in fmts:
        for name, rows, k, epi in (("swiglu_gate_up", 6144, 2048, wq.WQ_EPI_SWIGLU),
                                   ("residual_down", 2048, 6144, wq.WQ_EPI_RESIDUAL)):
            if fmt == wq.WQ_FMT_Q4_0:
                b0 = torch.from_numpy(wqgen.q4_0_bytes(rows, k, seed)).cuda()
            else:
                wd = torch.from_numpy(wqgen.weights(rows, k, seed)).cuda()
                b0 = wq.pack_f16(wd) if fmt == wq.WQ_FMT_F16 else wq.quantize_q8_0(wd)
                del wd
            nbytes = wq.weight_bytes(rows, k, fmt)
            bs = [b0] + [b0.clone() for _ in range(max(1, math.ceil(ROTATE_BYTES / nbytes)) - 1)]
            n = rows // 2 if epi == wq.WQ_EPI_SWIGLU else rows
            for m in (1, 512):
                a = torch.from_numpy(wqgen.activations(m, k, seed)).cuda()
                c = torch.from_numpy(wqgen.residual(m, n, seed)).cuda()
                tmp = torch.empty((m, rows), device="cuda")

                def fused(i):
                    wq.wq_matmul_ex(a, bs[i % len(bs)], c, m, n, k, fmt, epi)

                def unfused(i):
                    wq.wq_matmul(a, bs[i % len(bs)], tmp, m, rows, k, fmt)
                    if epi == wq.WQ_EPI_SWIGLU:
                        torch.mul(F.silu(tmp[:, :n]), tmp[:, n:], out=c)
                    else:
                        c.add_(tmp)

                tf = time_launches(torch, fused, iters, warmup)
                tu = time_launches(torch, unfused, iters, warmup)
                out[f"{key}_{name}_m{m}_{rows}x{k}"] = {
                    "fused_us": round(tf * 1e6, 2), "unfused_us": round(tu * 1e6, 2),
                    "speedup": round(tu / tf, 3), "fused_weight_GB/s": round(nbytes / tf / 1e9, 1),
                    "route": ROUTE_NAMES[wq.wq_route_for(m, n, k, fmt)]}
                del a, c, tmp
            del bs, b0
            torch.cuda.empty_cache()
    return out


def topk_bench(torch, wq, wqgen, seed, iters, warmup):
    """LM-head top-k at vocab 151936, hidden 2048, for every format and k in
    {1, 50}: the fused GEMV + top-k (wq_lm_head_topk) against the GEMV alone
    (wq_matmul writing the logits) and against the GEMV followed by wq_topk."""
    n, k = 151936, 2048
    out = {}
    for fmt, key in ((wq.WQ_FMT_F16, "f16"), (wq.WQ_FMT_Q8_0, "q8"), (wq.WQ_FMT_Q4_0, "q4")):
        if fmt == wq.WQ_FMT_Q4_0:
            b0 = torch.from_numpy(wqgen.q4_0_bytes(n, k, seed)).cuda()
        else:
            wd = torch.from_numpy(wqgen.weights(n, k, seed)).cuda()
            b0 = wq.pack_f16(wd) if fmt == wq.WQ_FMT_F16 else wq.quantize_q8_0(wd)
            del wd
        nbytes = wq.weight_bytes(n, k, fmt)
        bs = [b0] + [b0.clone() for _ in range(max(1, math.ceil(ROTATE_BYTES / nbytes)) - 1)]
        a = torch.from_numpy(wqgen.activations(1, k, seed)).cuda()
        logits = torch.empty((1, n), device="cuda")
        t_gemv = time_launches(torch, lambda i: wq.wq_matmul(a, bs[i % len(bs)], logits, 1, n, k, fmt), iters,
                               warmup)
        for topk in (1, 50):
            vals = torch.empty(topk, device="cuda")
            ids = torch.empty(topk, dtype=torch.int32, device="cuda")
            t_fused = time_launches(
                torch, lambda i: wq.wq_lm_head_topk(a, bs[i % len(bs)], n, k, fmt, topk, vals, ids), iters, warmup)

            def unfused(i):
                wq.wq_matmul(a, bs[i % len(bs)], logits, 1, n, k, fmt)
                wq.wq_topk(logits, n, topk, vals, ids)

            t_unf = time_launches(torch, unfused, iters, warmup)
            out[f"{key}_k{topk}"] = {"fused_us": round(t_fused * 1e6, 2), "gemv_then_topk_us": round(t_unf * 1e6, 2),
                                     "gemv_only_us": round(t_gemv * 1e6, 2),
                                     "fused_weight_GB/s": round(nbytes / t_fused / 1e9, 1)}
        del bs, b0
        torch.cuda.empty_cache()
    return out


ATTN_LENS = [4096, 32768, 131072]


def attention_bench(torch, wq, seed, iters, warmup):
    """Split-KV decode attention at head_dim 256, 8 query heads over 2 KV heads
    (q_dim 2048 = the o_proj input of the decode suite), f32 and f16 caches of
    4096 / 32768 / 131072 tokens; K and V ~ N(0,1) drawn on the device (seeded),
    rotated over copies of >= 1 GiB.  Bytes = the K and V rows read once."""
    D, hq, hkv = 256, 8, 2
    gen = torch.Generator(device="cuda")
    gen.manual_seed(seed)
    q = torch.randn((hq, D), device="cuda", generator=gen)
    out = torch.empty((hq, D), device="cuda")
    res = {}
    for kvfmt, key in ((wq.WQ_KV_F32, "f32"), (wq.WQ_KV_F16, "f16")):
        for L in ATTN_LENS:
            dt = torch.float32 if kvfmt == wq.WQ_KV_F32 else torch.float16
            nbytes = 2 * L * hkv * D * (4 if kvfmt == wq.WQ_KV_F32 else 2)
            copies = max(2, math.ceil(ROTATE_BYTES / nbytes))
            ks = [torch.randn((L, hkv * D), device="cuda", generator=gen).to(dt) for _ in range(copies)]
            vs = [torch.randn((L, hkv * D), device="cuda", generator=gen).to(dt) for _ in range(copies)]
            if kvfmt == wq.WQ_KV_F16:
                ks = [x.view(torch.int16) for x in ks]
                vs = [x.view(torch.int16) for x in vs]
            t = time_launches(torch, lambda i: wq.wq_decode_attention(q, ks[i % copies], vs[i % copies], out, L, D,
                                                                      hq, hkv, kvfmt, 0.0625), iters, warmup)
            res[f"{key}_L{L}"] = {"us": round(t * 1e6, 2), "kv_GB/s": round(nbytes / t / 1e9, 1),
                                  "frac_hbm": round(nbytes / t / 1e9 / HBM_PEAK_GBS, 4), "kv_bytes": nbytes}
            del ks, vs
            torch.cuda.empty_cache()
    return res


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(host_weights, seed, budget_s=8.0):
    """The CPU oracle, timed on this host: the f16 decode suite repeated until the
    time budget is used (the headline value), then one oracle call per other
    configuration -- the 1024x1024 GEMV, the Q8_0 decode suite, the two M = 512 f16
    prefill products and every M of the Q8_0 sweep at both shapes -- and one call
    per fused row (SwiGLU, LM-head top-50, attention over 4096 tokens).  Threads:
    every CPU in the process's affinity mask, unless OMP_NUM_THREADS asks for
    fewer (the GPU machine sets it to the CPU share of one GPU)."""
    import numpy as np

    import oracle
    import wqgen

    affinity = len(os.sched_getaffinity(0))
    threads = affinity
    omp = os.environ.get("OMP_NUM_THREADS", "")
    if omp.isdigit() and 0 < int(omp) < threads:
        threads = int(omp)
    threads = max(1, min(128, threads))
    enc = {(n, k): oracle.encode(host_weights[(n, k)], oracle.FMT_F16) for _, n, k in DECODE}
    acts = {k: wqgen.activations(1, k, seed) for _, _, k in DECODE}
    bytes_done, t_total, passes = 0, 0.0, 0
    while passes == 0 or t_total < budget_s:
        for _, n, k in DECODE:
            t0 = time.perf_counter()
            oracle.matmul(acts[k], enc[(n, k)], oracle.FMT_F16, 1, n, k, threads=threads)
            t_total += time.perf_counter() - t0
            bytes_done += 2 * n * k
        passes += 1

    def timed(fn):
        t0 = time.perf_counter()
        fn()
        return time.perf_counter() - t0

    configs = {}
    # C1: GEMV 1024 x 1024 f16.
    w1 = oracle.encode(wqgen.weights(1024, 1024, seed), oracle.FMT_F16)
    a1 = wqgen.activations(1, 1024, seed)
    dt = timed(lambda: oracle.matmul(a1, w1, oracle.FMT_F16, 1, 1024, 1024, threads=threads))
    configs["gemv_f16_1024x1024"] = {"ms": round(dt * 1e3, 3), "weight_GB/s": round(w1.nbytes / dt / 1e9, 3)}
    # Q8_0 decode suite (same f32 weights, quantised by the oracle).
    q8 = {(n, k): oracle.encode(host_weights[(n, k)], oracle.FMT_Q8_0) for _, n, k in DECODE}
    tq, bq = 0.0, 0
    for name, n, k in DECODE:
        dt = timed(lambda: oracle.matmul(acts[k], q8[(n, k)], oracle.FMT_Q8_0, 1, n, k, threads=threads))
        configs[f"q8_decode_{name}_{n}x{k}"] = {"ms": round(dt * 1e3, 3),
                                                "weight_GB/s": round(q8[(n, k)].nbytes / dt / 1e9, 3)}
        tq += dt
        bq += q8[(n, k)].nbytes
    configs["q8_decode_suite"] = {"ms": round(tq * 1e3, 3), "weight_GB/s": round(bq / tq / 1e9, 3)}
    del q8
    # f16 prefill at M = 512, both shapes, full products.
    for m, n, k in PREFILL:
        w = oracle.encode(wqgen.weights(n, k, seed), oracle.FMT_F16)
        a = wqgen.activations(m, k, seed)
        dt = timed(lambda: oracle.matmul(a, w, oracle.FMT_F16, m, n, k, threads=threads))
        configs[f"f16_prefill_{m}x{n}x{k}"] = {"ms": round(dt * 1e3, 2), "GFLOP/s": round(2.0 * m * n * k / dt / 1e9, 2)}
    # Q8_0 M sweep, every M at both shapes.
    for n, k in SWEEP_SHAPES:
        w = oracle.encode(wqgen.weights(n, k, seed), oracle.FMT_Q8_0)
        a_all = wqgen.activations(max(SWEEP_M), k, seed)
        for m in SWEEP_M:
            a = np.ascontiguousarray(a_all[:m])
            dt = timed(lambda: oracle.matmul(a, w, oracle.FMT_Q8_0, m, n, k, threads=threads))
            configs[f"q8_sweep_{m}x{n}x{k}"] = {"ms": round(dt * 1e3, 2),
                                                "GFLOP/s": round(2.0 * m * n * k / dt / 1e9, 2),
                                                "weight_GB/s": round(w.nbytes / dt / 1e9, 3)}
        del w, a_all
    # The fused rows, one oracle call each (the same shapes as their GPU tables).
    rows = {}
    a = wqgen.activations(1, 2048, seed)
    gu = enc[(6144, 2048)]
    dt = timed(lambda: oracle.matmul_epilogue(a, gu, oracle.FMT_F16, 1, 3072, 2048, oracle.EPI_SWIGLU,
                                              threads=threads))
    rows["swiglu_gate_up_m1_6144x2048"] = {"ms": round(dt * 1e3, 2), "weight_GB/s": round(2 * 6144 * 2048 / dt / 1e9, 3)}
    lm = enc[(151936, 2048)]
    dt = timed(lambda: oracle.lm_head_topk(a, lm, oracle.FMT_F16, 151936, 2048, 50, threads=threads))
    rows["lm_head_topk50_151936x2048"] = {"ms": round(dt * 1e3, 2), "weight_GB/s": round(lm.nbytes / dt / 1e9, 3)}
    L, D, hq, hkv = 4096, 256, 8, 2
    q = wqgen.normal((hq, D), seed=seed, stream=11)
    kc = wqgen.normal((L, hkv * D), seed=seed, stream=12)
    vc = wqgen.normal((L, hkv * D), seed=seed, stream=13)
    dt = timed(lambda: oracle.decode_attention(q, kc, vc, oracle.KV_F32, L, D, hq, hkv, 0.0625))
    rows["decode_attention_f32_L4096"] = {"ms": round(dt * 1e3, 2), "kv_GB/s": round(2 * kc.nbytes / dt / 1e9, 3),
                                          "threads": 1}
    return {"value": round(bytes_done / t_total / 1e9, 3), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": f"{passes} full pass(es) of the f16 decode suite (4 GEMVs, M=1, {bytes_done // passes} "
                      f"weight bytes per pass), f64 accumulation, {t_total:.1f} s; then one oracle call per "
                      f"other configuration (configs)",
            "cpu_model": _cpu_model(), "affinity_cpus": affinity, "configs": configs, "other_rows": rows}


def main():
    args = parse()
    if args.summarize:
        summarize(args.summarize)
        return
    if args.gpus != 1:
        print("bench.py runs on one GPU only: this library has no multi-GPU path (pass --gpus 1)",
              file=sys.stderr)
        sys.exit(2)
    import torch

    import gemm_wq_gemv_amd as wq
    import wqgen

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    torch.cuda.set_device(0)
    F16, Q8, Q4 = wq.WQ_FMT_F16, wq.WQ_FMT_Q8_0, wq.WQ_FMT_Q4_0

    log("drawing inputs")
    host_weights = {(n, k): wqgen.weights(n, k, args.seed) for _, n, k in DECODE}

    secondary = {}
    only = args.only
    result = None
    iters = max(10, args.steps // 2)
    if only == "counters":
        counter_workload(torch, wq, wqgen, args.seed)
        return

    # Plain-read ceilings at every byte size a bandwidth-bound row reads.
    ceiling = {}
    if only in (None, "f16", "q8", "q4", "sweep"):
        log("read ceiling")
        sizes = {"gemv_f16_1024x1024": wq.weight_bytes(1024, 1024, F16)}
        for fmt, key in ((F16, "f16"), (Q8, "q8"), (Q4, "q4")):
            for name, n, k in DECODE:
                sizes[f"{key}_{name}_{n}x{k}"] = wq.weight_bytes(n, k, fmt)
        for fmt, key in ((Q8, "q8"), (Q4, "q4")):
            for n, k in SWEEP_SHAPES:
                sizes[f"{key}_sweep_{n}x{k}"] = wq.weight_bytes(n, k, fmt)
        sizes["1GiB"] = 1 << 30
        rc = read_ceiling(torch, wq, sizes, iters, args.warmup)
        secondary["read_ceiling"] = rc
        ceiling = {v["bytes"]: v["GB/s"] for v in rc.values()}

    if only in (None, "f16"):
        log("f16 decode suite: encoding + rotation copies")
        s16 = Suite(wq, wqgen, torch, F16, args.seed, host_weights)
        log("f16 decode suite: timing")
        lm = [i for i, it in enumerate(s16.items) if it["name"] == "lm_head"][0]
        # The timed steps carry no event markers (each costs GPU time between
        # kernels); per-launch event pairs are taken in a separate pass below.
        total, wall, _ = time_suite(torch, wq, s16, args.steps, args.warmup, bracket=[])
        lm_bytes = s16.items[lm]["bytes"]
        # Average LM-head launch duration: a burst of back-to-back launches of
        # the same kernel on the same stream (the suite's rotated weight copies),
        # bracketed by one event pair while a spin kernel holds the stream, so
        # neither per-launch event markers nor host enqueue time count.
        it = s16.items[lm]
        lm_s = time_launches(torch, lambda i: wq.wq_matmul(it["a"], it["bs"][i % len(it["bs"])], it["c"], 1, it["n"],
                                                           it["k"], F16), max(20, args.steps), 3)
        achieved = lm_bytes / lm_s / 1e9
        value = s16.bytes_per_step * args.steps / total / 1e9
        per_burst = gemv_table(torch, wq, s16, F16, iters, args.warmup, ceiling)
        # Per-kernel times in a separate, untimed pass with every launch bracketed
        # (includes the events' own cost, about 3 us for the small kernels).
        _, _, per_all = time_suite(torch, wq, s16, max(10, args.steps // 2), 2, bracket=range(len(s16.items)))
        lm_pairs_s = per_all[lm]
        result = {
            "metric": METRIC,
            "value": round(value, 2),
            "unit": "GB/s",
            "n_gpus": 1,
            "steps": args.steps,
            "warmup": args.warmup,
            "ms_per_step": round(total / args.steps * 1e3, 5),
            "higher_is_better": True,
            "scaling": "weak",
            "vs_baseline": None,
            "dtype": "f32",
            "data": "synthetic",
            "config": {
                "workload": "f16-weight decode GEMV suite at hidden 2048, M=1: (N,K) = (6144,2048) gate/up, "
                            "(2048,6144) down, (2048,2048) o_proj, (151936,2048) LM head; A ~ N(0,1) f32, "
                            "B ~ N(0,0.02) cast to f16; seed 0",
                "weight_bytes_per_step": s16.bytes_per_step,
                "rotation": {it["name"]: len(it["bs"]) for it in s16.items},
                "frac_of_hbm_peak": round(value / HBM_PEAK_GBS, 4),
                "wall_s": round(wall, 4),
            },
            "roofline": {
                "kernel": "gemv_f16_ksplit (LM head, N=151936, K=2048)",
                "bound": "hbm",
                "achieved": round(achieved, 1),
                "peak": HBM_PEAK_GBS,
                "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": recorded_traffic(),
                "avg_launch_us": round(lm_s * 1e6, 3),
                "avg_launch_us_per_launch_event_pairs_in_suite": round(lm_pairs_s * 1e6, 3),
                "algorithmic_bytes_per_launch": lm_bytes,
                "read_ceiling_GB/s": ceiling.get(lm_bytes),
                "frac_of_read_ceiling": round(achieved / ceiling[lm_bytes], 4) if lm_bytes in ceiling else None,
            },
        }
        secondary["f16_decode_per_kernel"] = per_burst
        secondary["f16_decode_per_kernel_event_timed"] = {
            it["name"]: {"us": round(per_all[j] * 1e6, 3), "GB/s": round(it["bytes"] / per_all[j] / 1e9, 1)}
            for j, it in enumerate(s16.items)}
        del s16
        torch.cuda.empty_cache()

    if not args.no_secondary and only in (None, "f16"):
        log("GEMV f16 1024x1024")
        n, k = 1024, 1024
        b0 = wq.pack_f16(torch.from_numpy(wqgen.weights(n, k, args.seed)).cuda())
        nbytes = wq.weight_bytes(n, k, F16)
        bs = [b0] + [b0.clone() for _ in range(max(1, math.ceil(ROTATE_BYTES / nbytes)) - 1)]
        a = torch.from_numpy(wqgen.activations(1, k, args.seed)).cuda()
        c = torch.empty((1, n), device="cuda")
        t = time_launches(torch, lambda i: wq.wq_matmul(a, bs[i % len(bs)], c, 1, n, k, F16), iters, args.warmup)
        gbs = nbytes / t / 1e9
        secondary["gemv_f16_1024x1024"] = {"us": round(t * 1e6, 2), "GB/s": round(gbs, 1),
                                           "frac_hbm": round(gbs / HBM_PEAK_GBS, 4),
                                           "frac_read_ceiling": round(gbs / ceiling[nbytes], 4) if nbytes in ceiling
                                           else None}
        del bs, b0
        torch.cuda.empty_cache()

    for fmt, key in ((Q8, "q8"), (Q4, "q4")):
        if args.no_secondary or only not in (None, key):
            continue
        log(f"{key} decode suite")
        sq = Suite(wq, wqgen, torch, fmt, args.seed, host_weights)
        lmq = [i for i, it in enumerate(sq.items) if it["name"] == "lm_head"][0]
        total, _, _ = time_suite(torch, wq, sq, args.steps, args.warmup, bracket=[])
        _, _, per_all = time_suite(torch, wq, sq, max(10, args.steps // 2), 2, bracket=range(len(sq.items)))
        it = sq.items[lmq]
        lmq_s = time_launches(torch, lambda i: wq.wq_matmul(it["a"], it["bs"][i % len(it["bs"])], it["c"], 1, it["n"],
                                                            it["k"], fmt), max(20, args.steps), 3)
        secondary[f"{key}_decode_suite"] = {
            "per_kernel": gemv_table(torch, wq, sq, fmt, iters, args.warmup, ceiling),
            "GB/s": round(sq.bytes_per_step * args.steps / total / 1e9, 2),
            "frac_hbm": round(sq.bytes_per_step * args.steps / total / 1e9 / HBM_PEAK_GBS, 4),
            "ms_per_step": round(total / args.steps * 1e3, 5),
            "lm_head_us": round(lmq_s * 1e6, 3),
            "lm_head_GB/s": round(it["bytes"] / lmq_s / 1e9, 1),
            "per_kernel_event_timed": {it["name"]: {"us": round(per_all[j] * 1e6, 3),
                                                    "GB/s": round(it["bytes"] / per_all[j] / 1e9, 1)}
                                       for j, it in enumerate(sq.items)},
        }
        del sq
        torch.cuda.empty_cache()

    if not args.no_secondary and only in (None, "prefill"):
        log("f16 prefill GEMM, M=512")
        out = {}
        for m, n, k in PREFILL:
            b0 = wq.pack_f16(torch.from_numpy(wqgen.weights(n, k, args.seed)).cuda())
            nbytes = wq.weight_bytes(n, k, F16)
            bs = [b0] + [b0.clone() for _ in range(max(1, math.ceil(ROTATE_BYTES / nbytes)) - 1)]
            a = torch.from_numpy(wqgen.activations(m, k, args.seed)).cuda()
            c = torch.empty((m, n), device="cuda")
            t = time_launches(torch, lambda i: wq.wq_matmul(a, bs[i % len(bs)], c, m, n, k, F16),
                              max(10, args.steps // 2), args.warmup)
            tf = 2.0 * m * n * k / t / 1e12
            route = wq.wq_route_for(m, n, k, F16)
            # The same product on the fp32 matrix-core GEMM, for comparison.
            prev = wq.wq_set_forced_route(wq.WQ_ROUTE_GEMM)
            try:
                t32 = time_launches(torch, lambda i: wq.wq_matmul(a, bs[i % len(bs)], c, m, n, k, F16),
                                    max(10, args.steps // 2), args.warmup)
            finally:
                wq.wq_set_forced_route(prev)
            out[f"{m}x{n}x{k}"] = {"us": round(t * 1e6, 2), "TFLOP/s": round(tf, 2), "route": ROUTE_NAMES[route],
                                   "plan": list(wq.wq_hgemm_plan(m, n, k, F16)),
                                   "frac_mfma_fp32": round(tf / FP32_MFMA_PEAK_TFLOPS, 4),
                                   "frac_route_peak": round(tf / compute_peak(route), 4),
                                   "route_peak_TFLOP/s": compute_peak(route),
                                   "fp32_gemm_us": round(t32 * 1e6, 2),
                                   "fp32_gemm_TFLOP/s": round(2.0 * m * n * k / t32 / 1e12, 2)}
            del bs, b0
            torch.cuda.empty_cache()
        secondary["f16_prefill_m512"] = out

    if not args.no_secondary and only in (None, "sweep"):
        for fmt, key in ((Q8, "q8"), (Q4, "q4")):
            log(f"{key} M sweep")
            out = {}
            for n, k in SWEEP_SHAPES:
                if fmt == Q4:
                    b0 = torch.from_numpy(wqgen.q4_0_bytes(n, k, args.seed)).cuda()
                else:
                    b0 = wq.quantize_q8_0(torch.from_numpy(wqgen.weights(n, k, args.seed)).cuda())
                nbytes = wq.weight_bytes(n, k, fmt)
                bs = [b0] + [b0.clone() for _ in range(max(1, math.ceil(ROTATE_BYTES / nbytes)) - 1)]
                a_all = torch.from_numpy(wqgen.activations(max(SWEEP_M), k, args.seed)).cuda()
                for m in SWEEP_M:
                    a = a_all[:m].contiguous()
                    c = torch.empty((m, n), device="cuda")
                    t = time_launches(torch, lambda i: wq.wq_matmul(a, bs[i % len(bs)], c, m, n, k, fmt),
                                      max(10, args.steps // 2), args.warmup)
                    gbs, tf = nbytes / t / 1e9, 2.0 * m * n * k / t / 1e12
                    # Binding roofline: HBM below the ridge, the route's matrix
                    # peak above it (ridge 19.7 flop/B for fp32 MFMA, 156 for
                    # the f16 pairs).
                    route = wq.wq_route_for(m, n, k, fmt)
                    peak = compute_peak(route)
                    hbm_bound = 2.0 * m * n * k / nbytes < peak * 1e12 / (HBM_PEAK_GBS * 1e9)
                    out[f"{m}x{n}x{k}"] = {"us": round(t * 1e6, 2), "weight_GB/s": round(gbs, 1),
                                           "TFLOP/s": round(tf, 2),
                                           "bound": "hbm" if hbm_bound else "mfma",
                                           "frac_of_bound": round(gbs / HBM_PEAK_GBS if hbm_bound else tf / peak, 4),
                                           "frac_mfma_fp32": round(tf / FP32_MFMA_PEAK_TFLOPS, 4),
                                           "frac_read_ceiling": round(gbs / ceiling[nbytes], 4)
                                           if hbm_bound and nbytes in ceiling else None,
                                           "route": ROUTE_NAMES[route]}
                del bs, b0
                torch.cuda.empty_cache()
            secondary[f"{key}_sweep"] = out

    if not args.no_secondary and only in (None, "epi"):
        log("fused epilogues")
        secondary["epilogues"] = epilogue_bench(torch, wq, wqgen, args.seed, max(10, args.steps // 2), args.warmup)

    if not args.no_secondary and only in (None, "topk"):
        log("LM-head top-k")
        secondary["lm_head_topk_151936x2048"] = topk_bench(torch, wq, wqgen, args.seed, max(10, args.steps // 2),
                                                          args.warmup)

    if not args.no_secondary and only in (None, "attn"):
        log("decode attention")
        secondary["decode_attention_h256_q8_kv2"] = attention_bench(torch, wq, args.seed, max(10, args.steps // 2),
                                                                   args.warmup)

    if (not args.no_secondary and only is None) or only == "f16":
        log("device copy reference")
        nb = 1 << 30
        src = torch.empty(nb // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        t = time_launches(torch, lambda i: dst.copy_(src), 10, 3)
        secondary["device_copy_1GiB"] = {"us": round(t * 1e6, 1), "GB/s_read_plus_write": round(2 * nb / t / 1e9, 1)}
        del src, dst

    if result is None:
        log(json.dumps(secondary))
        return
    if not args.no_cpu:
        log("CPU oracle baseline")
        result["cpu_baseline"] = cpu_baseline(host_weights, args.seed)
    else:
        result["cpu_baseline"] = None
    result["secondary"] = secondary
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
