#!/usr/bin/env python3
"""Benchmark of the Q8_0 projection path on one MI355X.

Headline (one JSON line on stdout): the decode projection set at batch 1,
H=7168 -- rmsnorm_quant (ROW) of the row, whose quantized activation feeds
every K=7168 consumer (N=4096/512/512/4096 plus N=12288 and N=96), and the
N=4096 K=128 GEMV on a second f32 vector, quantized in the launch. One step is
one launch of rmsnorm_quant_gemv_shared_multi_plus_f32; `value` is the step's
algorithmic HBM bytes per second. The same work as two launches (rmsnorm_quant,
then q8_gemv_shared_multi_plus_f32) and as six is timed beside it.
Weights rotate over enough distinct copies (>= 1 GB) that no step finds its
weights in the 256 MB Infinity Cache or the L2s. The steps are captured once
in a HIP graph and replayed; inputs are resident in HBM before timing.

Also measured (in "per_config"): the single 2048x2048 GEMV, the prefill
rms-class and swiglu-class producers and q8 GEMMs at T=3325, and the LM head
(GEMV at T=1, GEMM at T=512), each kernel timed with HIP events on its own
stream, reported as GB/s or TOPS and as a fraction of the MI355X peaks.

cpu_baseline: the CPU oracle computing the same decode step on this host,
timed on a bounded number of steps.
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
sys.path.insert(0, ROOT)

METRIC = "Q8_0 GEMV HBM GB/s (batch 1) + q8 GEMM i8 TOPS (prefill) vs roofline"
HBM_PEAK_GBS = 8000.0   # MI355X HBM3E
I8_PEAK_TOPS = 5000.0   # MI355X dense int8 MFMA
EPS = 1e-6
COLD_BYTES = 1.0e9      # rotate weight copies over at least this many bytes


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def ensure_built():
    from int8_quantized_projections_amd import _build
    import synth

    if not os.path.exists(_build.LIB_PATH):
        _build.build()
    if not os.path.exists(synth.LIB_PATH):
        synth.build()


# ---------------------------------------------------------------------------
# Inputs on the device (weights quantized on the GPU by the library itself)
# ---------------------------------------------------------------------------
class Dev:
    def __init__(self):
        import torch
        from int8_quantized_projections_amd import q8lib

        self.torch = torch
        self.q8 = q8lib
        self.dev = torch.device("cuda:0")

    def upload(self, a):
        import numpy as np
        return self.torch.from_numpy(np.ascontiguousarray(a)).to(self.dev)

    def tensor(self, workload, name, rows=None):
        import synth
        return self.upload(synth.tensor(workload, name, rows))

    def weights(self, workload, name, chunk_rows=16384):
        """Q8_0 weights [N, K] from the workload's f32 draw, quantized on the GPU (q8_quantize, ROW)."""
        import synth
        torch, q8 = self.torch, self.q8
        (N, K), _, _, _ = synth.WORKLOADS[workload]["tensors"][name]
        qs = torch.empty((N, K), dtype=torch.int8, device=self.dev)
        d = torch.empty((N, K // 32), dtype=torch.int16, device=self.dev)
        for r0 in range(0, N, chunk_rows):
            r1 = min(N, r0 + chunk_rows)
            wf = self.tensor(workload, name, slice(r0, r1))
            sd = torch.empty((r1 - r0) * (K // 32), dtype=torch.int32, device=self.dev)
            q8.q8_quantize(wf, q8.LAYOUT_ROW, qs[r0:r1].reshape(-1), sd)
            d[r0:r1] = sd.view(torch.int16).view(-1, 2)[:, 0].reshape(r1 - r0, K // 32)  # low half = f16 d
            del wf, sd
        torch.cuda.synchronize()
        return q8.Q8Weights(qs, d)

    def copies(self, W, n):
        return [W] + [self.q8.Q8Weights(W.qs.clone(), W.d.clone()) for _ in range(n - 1)]


def gemv_bytes(N, K):
    """Algorithmic bytes of one batch-1 GEMV: weights (1.0625 B each), activation, output."""
    return N * K + N * (K // 32) * 2 + K + (K // 32) * 4 + N * 4


def gemv_f32_bytes(N, K):
    """Algorithmic bytes of a GEMV on an f32 activation quantized in the launch."""
    return N * K + N * (K // 32) * 2 + K * 4 + N * 4


def quant_bytes(rows, K, layout=0):
    qrows = rows if layout == 0 else (rows + 63) // 64 * 64
    return rows * K * 4 + qrows * K + qrows * (K // 32) * 4


def rms_bytes(rows, K, layout=0):
    return quant_bytes(rows, K, layout) + rows * K * 4 + K * 4


def swiglu_bytes(rows, K, layout=1):
    return quant_bytes(rows, K, layout) + rows * K * 8


def gemm_min_bytes(T, N, K):
    qrows = (T + 63) // 64 * 64
    return qrows * K + qrows * (K // 32) * 4 + N * K + N * (K // 32) * 2 + T * N * 4


def stats(ms_list):
    s = sorted(ms_list)
    n = len(s)
    pick = lambda q: s[min(n - 1, max(0, int(round(q * (n - 1)))))]
    return {"median_us": pick(0.5) * 1e3, "p10_us": pick(0.1) * 1e3, "p90_us": pick(0.9) * 1e3,
            "mean_us": sum(s) / n * 1e3, "reps": n, "reps_us": [round(v * 1e3, 2) for v in ms_list]}


def device_info(torch):
    """The GPU as the runtime reports it."""
    p = torch.cuda.get_device_properties(0)
    return {"name": p.name, "arch": getattr(p, "gcnArchName", None), "compute_units": p.multi_processor_count,
            "memory_GB": round(p.total_memory / 1e9, 1), "clock_kHz": getattr(p, "clock_rate", None)}


def counted_launches(q8, fn):
    """Kernel launches the library enqueues for one call of fn, by its launch counters."""
    q8.launch_counts_reset()
    fn()
    return sum(q8.launch_counts().values())


def time_each(D, fn, reps, warm=3):
    """Device time of each call of fn(i), measured with HIP events on the current stream.
    A spin kernel queued first keeps the stream busy while the host enqueues every
    (event, launch, event) triple, so no host gap falls inside an interval."""
    torch = D.torch
    for i in range(warm):
        fn(i)
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    torch.cuda._sleep(int(2.4e9 * (1e-3 + 60e-6 * reps)))
    for i, (a, b) in enumerate(evs):
        a.record()
        fn(i)
        b.record()
    torch.cuda.synchronize()
    return [a.elapsed_time(b) for a, b in evs]


def time_batch(D, fn, reps, warm=3):
    """Mean device time per call of fn(i) over `reps` back-to-back calls, with one pair of
    HIP events around the whole batch (no event between launches)."""
    torch = D.torch
    for i in range(warm):
        fn(i)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda._sleep(int(2.4e9 * (1e-3 + 40e-6 * reps)))
    a.record()
    for i in range(reps):
        fn(i)
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / reps


def timed(D, fn, reps):
    """Device time per launch of fn(i). mean_us: the mean over a back-to-back batch of 4*reps
    launches with one pair of HIP events around the batch, the kernel's own duration as a trace
    shows it; each: the per-launch event pairs, where every interval also holds that launch's
    dispatch (a few microseconds, the whole time of a tiny kernel)."""
    each = stats(time_each(D, fn, reps))
    batch_us = time_batch(D, fn, 4 * reps) * 1e3
    return {"mean_us": batch_us, "timing": "back-to-back batch of %d launches" % (4 * reps),
            "each": {k: each[k] for k in ("mean_us", "median_us", "p10_us", "p90_us", "reps", "reps_us")}}


# ---------------------------------------------------------------------------
# Headline: decode projection set, H=7168
# ---------------------------------------------------------------------------
DEC_N = {"Wq": 4096, "Wk": 512, "Wv": 512, "Wg": 4096, "W12288": 12288, "W96": 96, "W128": 4096}


DEC_GROUP = ("Wq", "Wk", "Wv", "Wg", "W12288", "W96")  # every consumer of the normed activation


def decode_pair_bytes():
    """The grouped GEMV over the six K=7168 consumers (one read of the q8_0 activation) and
    the K=128 GEMV, its f32 activation quantized in the launch."""
    return decode_grouped_bytes() + gemv_f32_bytes(4096, 128)


def decode_step_bytes():
    """The whole step in one launch: x and w read, y and the q8_0 activation written once,
    every weight byte and output once. The grouped GEMV reads its activation from LDS, so
    the pair's activation read is not counted."""
    H = 7168
    return {"rmsnorm_quant_gemv_shared_multi_plus_f32":
            rms_bytes(1, H) + decode_pair_bytes() - (H + (H // 32) * 4)}


def decode_grouped_bytes():
    H = 7168
    return sum(gemv_bytes(DEC_N[n], H) for n in DEC_GROUP) - (len(DEC_GROUP) - 1) * (H + (H // 32) * 4)


def bench_decode(D, steps, warmup, log_reps):
    torch, q8 = D.torch, D.q8
    wl = "decode_h7168"
    H = 7168
    log("[decode] building inputs")
    x = D.tensor(wl, "x").view(1, H)
    w = D.tensor(wl, "w_norm")
    x128 = D.tensor(wl, "x128").view(1, 128)
    base = {n: D.weights(wl, n) for n in DEC_N}
    set_bytes = sum(W.qs.numel() + W.d.numel() * 2 for W in base.values())
    ncopy = max(2, math.ceil(COLD_BYTES / set_bytes))
    sets = [dict(zip(base, ws)) for ws in zip(*(D.copies(base[n], ncopy) for n in base))]
    log(f"[decode] {ncopy} weight copies of {set_bytes / 1e6:.1f} MB")
    y = torch.empty((1, H), device=D.dev)
    aq, asd = q8.alloc_act(1, H, q8.LAYOUT_ROW)
    bq, bsd = q8.alloc_act(1, 128, q8.LAYOUT_ROW)
    outs = {n: torch.empty(DEC_N[n], device=D.dev) for n in DEC_N}

    def launches(c):
        S = sets[c % ncopy]
        return [
            # the producer and every GEMV of the step in one launch; the K=128 activation has
            # one consumer and is quantized inside the launch
            ("rmsnorm_quant_gemv_shared_multi_plus_f32", lambda: q8.rmsnorm_quant_gemv_shared_multi_plus_f32(
                x, w, EPS, [S[n] for n in DEC_GROUP], S["W128"], x128.view(-1), y, aq, asd,
                [outs[n] for n in DEC_GROUP], outs["W128"])),
        ]

    def standalone(c):  # the same work as separate launches, for comparison
        S = sets[c % ncopy]
        return {
            # the step as two launches: the producer, then both GEMVs in one launch
            "rmsnorm_quant_row": (lambda: q8.rmsnorm_quant(x, w, EPS, q8.LAYOUT_ROW, y, aq, asd), rms_bytes(1, H)),
            "q8_gemv_shared_multi_plus_f32": (lambda: q8.q8_gemv_shared_multi_plus_f32(
                [S[n] for n in DEC_GROUP], aq, asd, S["W128"], x128.view(-1), [outs[n] for n in DEC_GROUP],
                outs["W128"]), decode_pair_bytes()),
            # the step's GEMVs as two launches
            "q8_gemv_shared_multi_x6": (lambda: q8.q8_gemv_shared_multi(
                [S[n] for n in DEC_GROUP], aq, asd, [outs[n] for n in DEC_GROUP]), decode_grouped_bytes()),
            "q8_gemv_f32_4096x128": (lambda: q8.q8_gemv_f32(S["W128"], x128.view(-1), outs["W128"]),
                                     gemv_f32_bytes(4096, 128)),
            # and as six
            "q8_gemv_shared_multi_x4": (lambda: q8.q8_gemv_shared_multi(
                [S[n] for n in DEC_GROUP[:4]], aq, asd, [outs[n] for n in DEC_GROUP[:4]]),
                sum(gemv_bytes(DEC_N[n], H) for n in DEC_GROUP[:4]) - 3 * (H + (H // 32) * 4)),
            "q8_gemv_12288x7168": (lambda: q8.q8_gemv(S["W12288"], aq, asd, outs["W12288"]), gemv_bytes(12288, H)),
            "q8_gemv_96x7168": (lambda: q8.q8_gemv(S["W96"], aq, asd, outs["W96"]), gemv_bytes(96, H)),
            "q8_quantize_128": (lambda: q8.q8_quantize(x128, q8.LAYOUT_ROW, bq, bsd), quant_bytes(1, 128)),
            "q8_gemv_4096x128": (lambda: q8.q8_gemv(S["W128"], bq, bsd, outs["W128"]), gemv_bytes(4096, 128)),
        }

    def step(c):
        for _, f in launches(c):
            f()

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()

    # capture all timed steps in one graph (each step uses the next weight copy)
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(0)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    # the library's launch counters over the capture: launches per step, counted
    q8.launch_counts_reset()
    with torch.cuda.graph(g):
        for i in range(steps):
            step(i)
    counted = {k: v / steps for k, v in q8.launch_counts().items() if v}
    g.replay()  # untimed: graph upload / first replay
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    g.replay()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1)
    parts = decode_step_bytes()
    step_bytes = sum(parts.values())

    # per-kernel device time, HIP events around every launch (eager, rotating copies)
    comp = {}
    for idx, name in enumerate(parts):
        t = time_each(D, lambda i, idx=idx: launches(i)[idx][1](), log_reps)
        st = stats(t)
        gbs = parts[name] / (st["mean_us"] * 1e-6) / 1e9
        comp[name] = {**st, "bytes": parts[name], "GBps": gbs, "frac_hbm": gbs / HBM_PEAK_GBS,
                      "launches_per_step": 1}
        tb = time_batch(D, lambda i, idx=idx: launches(i)[idx][1](), 4 * log_reps)
        comp[name]["batch_mean_us"] = tb * 1e3
        comp[name]["batch_GBps"] = parts[name] / (tb * 1e-3) / 1e9
    for name in standalone(0):
        st = timed(D, lambda i, name=name: standalone(i)[name][0](), log_reps)
        b = standalone(0)[name][1]
        comp["separate_" + name] = {**st, "bytes": b, "GBps": b / (st["mean_us"] * 1e-6) / 1e9,
                                    "frac_hbm": b / (st["mean_us"] * 1e-6) / 1e9 / HBM_PEAK_GBS,
                                    "launches_per_step": 0}
        if name.startswith("q8_gemv") and b > 10e6 and PRACTICAL is not None:
            # a weight stream: the read ceiling at its own size (outputs are under 0.1% of it)
            c = PRACTICAL.ceiling(b, 0)
            comp["separate_" + name]["practical"] = c
            comp["separate_" + name]["frac_of_practical"] = comp["separate_" + name]["GBps"] / c["GBps"]
    del g
    # the same step with one weight copy, resident in the 256 MB Infinity Cache ("warm")
    gw = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gw):
        for i in range(steps):
            for _, f in launches(0):
                f()
    gw.replay()
    torch.cuda.synchronize()
    e0.record()
    gw.replay()
    e1.record()
    torch.cuda.synchronize()
    warm_ms = e0.elapsed_time(e1)
    del gw
    return {"ms_per_step": ms / steps, "step_bytes": step_bytes, "value_GBps": step_bytes * steps / (ms * 1e-3) / 1e9,
            "slice_tok_per_s": steps / (ms * 1e-3),
            "copies": ncopy, "components": comp, "launches_per_step": sum(counted.values()),
            "launches_per_step_predicted": 1,
            "warm": {"ms_per_step": warm_ms / steps, "GBps": step_bytes * steps / (warm_ms * 1e-3) / 1e9,
                     "note": "one weight copy, resident in the Infinity Cache; not the headline"},
            "launch_counts_per_step": counted}


# ---------------------------------------------------------------------------
# Other workloads (each kernel: HIP events around a back-to-back batch, see timed)
# ---------------------------------------------------------------------------
def launch_floor(D, reps):
    """The back-to-back time per launch of a kernel that does almost nothing (the read probe over
    16 KB, one workgroup): the floor under any kernel's time in a batch of launches."""
    torch, q8 = D.torch, D.q8
    buf = torch.zeros(16384, dtype=torch.uint8, device=D.dev)
    out = torch.empty(1, dtype=torch.int32, device=D.dev)
    us = time_batch(D, lambda i: q8.hbm_read_probe(buf, 1, 1, out), 4 * reps) * 1e3
    return {"mean_us": us, "kernel": "k_read_probe<1>, 16 KB, one workgroup",
            "timing": "back-to-back batch of %d launches" % (4 * reps)}


def bench_gemv2048(D, reps):
    torch, q8 = D.torch, D.q8
    wl = "gemv_2048"
    x = D.tensor(wl, "x").view(1, 2048)
    W = D.weights(wl, "W")
    n = max(2, math.ceil(COLD_BYTES / (W.qs.numel() * 1.0625)))
    Ws = D.copies(W, n)
    aq, asd = q8.alloc_act(1, 2048, q8.LAYOUT_ROW)
    y = torch.empty(2048, device=D.dev)
    tq = timed(D, lambda i: q8.q8_quantize(x, q8.LAYOUT_ROW, aq, asd), reps)
    tg = timed(D, lambda i: q8.q8_gemv(Ws[i % n], aq, asd, y), reps)
    tf = timed(D, lambda i: q8.q8_gemv_f32(Ws[i % n], x.view(-1), y), reps)
    # back-to-back replay of many distinct-weight GEMVs: aggregate bytes / aggregate time
    R = min(n, 200)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(R):
            q8.q8_gemv(Ws[i], aq, asd, y)
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    g.replay()
    e1.record()
    torch.cuda.synchronize()
    agg_us = e0.elapsed_time(e1) * 1e3 / R
    gb = gemv_bytes(2048, 2048)
    fb = gemv_f32_bytes(2048, 2048)
    return {
        "slice_launches": {"predicted": 1, "counted": counted_launches(q8, lambda: q8.q8_gemv_f32(Ws[0], x.view(-1), y))},
        "q8_gemv_f32_2048x2048": {**hbm_entry(tf, fb, read_b=fb - 2048 * 4), "launches": 1},
        "q8_quantize_2048": {**tq, "bytes": quant_bytes(1, 2048), "GBps": quant_bytes(1, 2048) / tq["mean_us"] / 1e3},
        "q8_gemv_2048x2048": hbm_entry(tg, gb, read_b=gb - 2048 * 4),
        "launch_floor": launch_floor(D, reps),
        "q8_gemv_2048x2048_graph_back_to_back": {"us_per_gemv": agg_us, "GBps": gb / agg_us / 1e3,
                                                 "frac_hbm": gb / agg_us / 1e3 / HBM_PEAK_GBS, "gemvs": R},
    }


# The q8_0 GEMM's vector-ALU bound: every output element takes its two block scales once
# per 32-value K block, two non-packed f32 instructions (a wave64 instruction holds its SIMD
# for 4 cycles), against one 32x32x32 i8 MFMA of 32 matrix-core cycles per 32x32 tile and
# block: 65536 ops per 128 VALU cycles per SIMD, 512 ops per cycle, 1024 SIMDs at 2.4 GHz.
VALU_CEILING_TOPS = 512 * 4 * 256 * 2.4e9 / 1e12  # 1258 TOPS, 25% of the i8 MFMA peak


def gemm_entry(t, T, N, K):
    ops = 2.0 * T * N * K
    tops = ops / (t["mean_us"] * 1e-6) / 1e12
    mb = gemm_min_bytes(T, N, K)
    return {**t, "ops": ops, "TOPS": tops, "frac_i8_peak": tops / I8_PEAK_TOPS,
            "valu_ceiling_TOPS": VALU_CEILING_TOPS, "frac_valu_ceiling": tops / VALU_CEILING_TOPS,
            "min_bytes": mb, "GBps_min_bytes": mb / t["mean_us"] / 1e3}


class Practical:
    """Practical HBM ceilings of plain streams with a kernel's read/write mix and total bytes,
    cold: regions of a 4 GiB pool rotate so that no launch finds its bytes in a cache. The
    pattern is the one whose share of written bytes is nearest the kernel's: read-only (0; the
    read probe q8_hbm_read_probe), two reads per write (1/3) or a copy (1/2) (the stream probe
    q8_hbm_stream_probe). Timed as the kernels are: one pair of HIP events around a back-to-back
    batch. The best of a few launch shapes is kept."""
    READ_SHAPES = ((256, 1), (512, 1), (1024, 1), (2048, 1), (2048, 2), (4096, 2))
    GRID = (1024, 2048, 4096)

    def __init__(self, D):
        self.D = D
        self.pool = None
        self.out = None
        self.cache = {}

    @staticmethod
    def pattern(read_b, write_b):
        f = write_b / (read_b + write_b)
        return min((("read", 0.0), ("2read_1write", 1 / 3), ("copy", 0.5)), key=lambda p: abs(p[1] - f))[0]

    def ceiling(self, read_b, write_b, reps=10):
        torch, q8 = self.D.torch, self.D.q8
        pat = self.pattern(read_b, write_b)
        nstreams = {"read": 1, "2read_1write": 3, "copy": 2}[pat]
        stream_b = int((read_b + write_b) / nstreams) // 4096 * 4096
        key = (pat, stream_b >> 20)
        if key in self.cache:
            return self.cache[key]
        if self.pool is None:
            self.pool = torch.empty(4 << 30, dtype=torch.uint8, device=self.D.dev)
            self.out = torch.empty(65536, dtype=torch.int32, device=self.D.dev)
        set_b = stream_b * nstreams
        nsets = max(2, min(math.ceil(COLD_BYTES / set_b), (4 << 30) // set_b))
        bufs = [[self.pool[k * set_b + j * stream_b:k * set_b + (j + 1) * stream_b] for j in range(nstreams)]
                for k in range(nsets)]
        shapes = self.READ_SHAPES if pat == "read" else [(w, 1) for w in self.GRID]
        best = None
        for wgs, u in shapes:
            def one(i, wgs=wgs, u=u):
                b = bufs[i % nsets]
                if pat == "read":
                    q8.hbm_read_probe(b[0], wgs, u, self.out)
                elif pat == "copy":
                    q8.hbm_stream_probe(stream_b, wgs, src0=b[0], dst=b[1])
                else:
                    q8.hbm_stream_probe(stream_b, wgs, src0=b[0], src1=b[1], dst=b[2])
            us = time_batch(self.D, one, 4 * reps) * 1e3
            gbs = set_b / us / 1e3
            if best is None or gbs > best["GBps"]:
                best = {"pattern": pat, "bytes": set_b, "GBps": gbs, "mean_us": us, "sets": nsets,
                        "timing": "back-to-back batch", "workgroups": wgs, "loads_per_lane": u}
        self.cache[key] = best
        return best


PRACTICAL = None  # set in main()

# The (read, written) bytes per launch of the bandwidth-bound kernels above: the decode step
# (165 MB read), rmsnorm_quant and q8_quantize PLANE64, swiglu_quant PLANE64 with and without
# its f32 output, and the LM-head GEMV.
PRACTICAL_MIXES = [
    (165260032, 0),
    (3325 * 3584 * 4 + 3584 * 4, rms_bytes(3325, 3584, 1) - 3325 * 3584 * 4 - 3584 * 4),
    (3325 * 18944 * 4, quant_bytes(3325, 18944, 1) - 3325 * 18944 * 4),
    (3325 * 18944 * 8, swiglu_bytes(3325, 18944, 1) - 3325 * 18944 * 8),
    (3325 * 18944 * 8, swiglu_bytes(3325, 18944, 1) - 3325 * 18944 * 12),
    (gemv_bytes(152064, 3584) - 152064 * 4, 152064 * 4),
]


def hbm_entry(t, b, warm=None, read_b=None):
    """A bandwidth-bound kernel's rate; warm: the same kernel on one set of buffers. read_b: the
    bytes it reads (the rest are written), for the practical ceiling of that mix."""
    e = {**t, "bytes": b, "GBps": b / t["mean_us"] / 1e3, "frac_hbm": b / t["mean_us"] / 1e3 / HBM_PEAK_GBS}
    if read_b is not None and PRACTICAL is not None:
        c = PRACTICAL.ceiling(read_b, b - read_b)
        e["practical"] = c
        e["frac_of_practical"] = e["GBps"] / c["GBps"]
    if warm is not None:
        e["warm"] = {"mean_us": warm["mean_us"],
                     "GBps": b / warm["mean_us"] / 1e3, "frac_hbm": b / warm["mean_us"] / 1e3 / HBM_PEAK_GBS,
                     "note": "one set of buffers reused by every rep (may be served in part by the 256 MB "
                             "Infinity Cache); the headline figure above rotates distinct sets"}
    return e


def n_sets(set_bytes):
    """Distinct buffer sets to rotate so that a rep never finds its operands in the 256 MB
    Infinity Cache or the L2s: at least COLD_BYTES in all, and at least 2."""
    return max(2, math.ceil(COLD_BYTES / set_bytes))


def act_sets(D, src, n, layout, with_y=True):
    """n sets of (x, y, qs, sd): x a distinct copy of src, y [rows, K] f32, the quantized buffers."""
    torch, q8 = D.torch, D.q8
    rows, K = src.shape
    out = []
    for i in range(n):
        x = src if i == 0 else src.clone()
        q, sd = q8.alloc_act(rows, K, layout)
        out.append((x, torch.empty_like(src) if with_y else None, q, sd))
    return out


def bench_prefill_rms(D, reps):
    torch, q8 = D.torch, D.q8
    wl = "prefill_rms"
    T, K = 3325, 3584
    x = D.tensor(wl, "x")
    w = D.tensor(wl, "w_norm")
    Ws = {n: D.weights(wl, n) for n in ("Wq", "Wk", "Wv")}
    b = rms_bytes(T, K, 1)
    ns = n_sets(b)
    sets = act_sets(D, x, ns, q8.LAYOUT_PLANE64)
    log(f"[prefill_rms] {ns} input/output sets of {b / 1e6:.1f} MB")
    out = {}

    def rms(i):
        xs, ys, qs, sd = sets[i % ns]
        q8.rmsnorm_quant(xs, w, EPS, q8.LAYOUT_PLANE64, ys, qs, sd)

    t = timed(D, rms, reps)
    tw = timed(D, lambda i: rms(0), reps)
    out["rmsnorm_quant_plane64"] = hbm_entry(t, b, tw, read_b=T * K * 4 + K * 4)
    out["rmsnorm_quant_plane64"]["sets"] = ns
    prod_us = t["mean_us"]
    for i in range(ns):
        rms(i)
    # GEMM operands: distinct (weights, plane, output) sets over >= 1 GB, so no rep finds them
    # in the Infinity Cache
    gb = sum(gemm_min_bytes(T, W.n, K) for W in Ws.values())
    ng = n_sets(gb)
    wsets = [Ws] + [{n: q8.Q8Weights(W.qs.clone(), W.d.clone()) for n, W in Ws.items()} for _ in range(ng - 1)]
    csets = [{n: torch.empty((T, W.n), device=D.dev) for n, W in Ws.items()} for _ in range(ng)]
    log(f"[prefill_rms] {ng} GEMM operand sets of {gb / 1e6:.1f} MB")
    sep_us = 0.0
    for n in Ws:
        def one(i, n=n):
            _, _, qs, sd = sets[i % ns]
            q8.q8_gemm(wsets[i % ng][n], qs, sd, T, csets[i % ng][n])
        t = timed(D, one, reps)
        out[f"q8_gemm_{Ws[n].n}x{K}"] = gemm_entry(t, T, Ws[n].n, K)
        sep_us += t["mean_us"]
    # q, k and v over the one plane in one grouped launch (what the slice uses)
    names = list(Ws)

    def grouped(i):
        _, _, qs, sd = sets[i % ns]
        q8.q8_gemm_shared_multi([wsets[i % ng][n] for n in names], qs, sd, T, [csets[i % ng][n] for n in names])

    t = timed(D, grouped, reps)
    n_all = sum(W.n for W in Ws.values())
    out[f"q8_gemm_shared_multi_qkv_{n_all}x{K}"] = gemm_entry(t, T, n_all, K)
    out[f"q8_gemm_shared_multi_qkv_{n_all}x{K}"]["warm"] = {
        "mean_us": timed(D, lambda i: grouped(0), reps)["mean_us"], "note": "one operand set"}
    pq, ps = sets[0][2], sets[0][3]
    y = sets[0][1]
    C = csets[0]
    out["slice_launches"] = {"predicted": 2, "counted": counted_launches(q8, lambda: (
        q8.rmsnorm_quant(x, w, EPS, q8.LAYOUT_PLANE64, y, pq, ps),
        q8.q8_gemm_shared_multi([Ws[n] for n in names], pq, ps, T, [C[n] for n in names])))}
    out["slice_tok_per_s"] = T / ((prod_us + t["mean_us"]) * 1e-6)
    out["slice_tok_per_s_separate_gemms"] = T / ((prod_us + sep_us) * 1e-6)
    return out


def bench_prefill_swiglu(D, reps):
    torch, q8 = D.torch, D.q8
    wl = "prefill_swiglu"
    T, K, N = 3325, 18944, 3584
    g = D.tensor(wl, "gate")
    u = D.tensor(wl, "up")
    W = D.weights(wl, "Wd")
    out = {}
    # two distinct (gate, up, y, plane) sets of 827 MB: a rep never finds its inputs or the
    # previous rep's outputs in the 256 MB Infinity Cache
    b = swiglu_bytes(T, K, 1)
    gs = [(g, u)] + [(g.clone(), u.clone())]
    outs = [(torch.empty_like(g), *q8.alloc_act(T, K, q8.LAYOUT_PLANE64)) for _ in gs]

    def sw(i, f32=True):
        (gi, ui), (yi, qi, si) = gs[i % 2], outs[i % 2]
        q8.swiglu_quant(gi, ui, q8.LAYOUT_PLANE64, yi if f32 else None, qi, si, f32=f32)

    t = timed(D, sw, reps)
    out["swiglu_quant_plane64"] = hbm_entry(t, b, timed(D, lambda i: sw(0), reps), read_b=T * K * 8)
    # plane only (y = NULL): for a down projection that reads no f32 activation
    t3 = timed(D, lambda i: sw(i, False), reps)
    b3 = b - T * K * 4
    out["swiglu_quant_plane64_no_f32"] = hbm_entry(t3, b3, read_b=T * K * 8)
    # the unfused form's quantize pass: q8_quantize of the f32 y into the same plane (bit-identical
    # to the fused plane), the activation quantize at bandwidth scale; 323 MB per set, 4 sets
    sw(0)
    sw(1)
    b4 = quant_bytes(T, K, 1)
    nq = n_sets(b4)
    ysets = [outs[0][0], outs[1][0]] + [outs[0][0].clone() for _ in range(nq - 2)]
    qsets = [q8.alloc_act(T, K, q8.LAYOUT_PLANE64) for _ in range(nq)]

    def quant(i):
        q8.q8_quantize(ysets[i % nq], q8.LAYOUT_PLANE64, *qsets[i % nq])

    t4 = timed(D, quant, reps)
    out["q8_quantize_plane64"] = hbm_entry(t4, b4, timed(D, lambda i: quant(0), reps), read_b=T * K * 4)
    del ysets[2:], qsets[2:]
    # the down GEMM: distinct (weights, plane, output) sets over >= 1 GB
    gb = gemm_min_bytes(T, N, K)
    ng = n_sets(gb)
    Wset = [W] + [q8.Q8Weights(W.qs.clone(), W.d.clone()) for _ in range(ng - 1)]
    Pset = [outs[0][1:], outs[1][1:]] + [tuple(a.clone() for a in outs[0][1:]) for _ in range(ng - 2)]
    Cset = [torch.empty((T, N), device=D.dev) for _ in range(ng)]
    log(f"[prefill_swiglu] {ng} GEMM operand sets of {gb / 1e6:.1f} MB")

    def gemm(i):
        q8.q8_gemm(Wset[i % ng], *Pset[i % ng], T, Cset[i % ng])

    t2 = timed(D, gemm, reps)
    out[f"q8_gemm_{N}x{K}"] = gemm_entry(t2, T, N, K)
    out[f"q8_gemm_{N}x{K}"]["warm"] = {"mean_us": timed(D, lambda i: gemm(0), reps)["mean_us"],
                                       "note": "one operand set"}
    del Wset[1:], Pset[2:], Cset[1:]
    y, (pq, ps), C = outs[0][0], outs[0][1:], torch.empty((T, N), device=D.dev)
    out["slice_launches"] = {"predicted": 2, "counted": counted_launches(q8, lambda: (
        q8.swiglu_quant(g, u, q8.LAYOUT_PLANE64, y, pq, ps), q8.q8_gemm(W, pq, ps, T, C)))}
    out["slice_tok_per_s"] = T / ((t["mean_us"] + t2["mean_us"]) * 1e-6)
    out["slice_tok_per_s_no_f32"] = T / ((t3["mean_us"] + t2["mean_us"]) * 1e-6)
    return out


def bench_prefill_q4k(D, reps):
    """q4_K gate and up projections over the rms-class plane (T=3325, d=3584, N=18944 each)."""
    import synth
    torch, q8 = D.torch, D.q8
    T, K = 3325, 3584
    x = D.tensor("prefill_rms", "x")
    w = D.tensor("prefill_rms", "w_norm")
    pq, ps = q8.alloc_act(T, K, q8.LAYOUT_PLANE64)
    t = timed(D, lambda i: q8.rmsnorm_quant(x, w, EPS, q8.LAYOUT_PLANE64, None, pq, ps, f32=False), reps)
    out = {"rmsnorm_quant_plane64_no_f32": {**t, "bytes": rms_bytes(T, K, 1) - T * K * 4}}
    total_us = t["mean_us"]
    launches = counted_launches(q8, lambda: q8.rmsnorm_quant(x, w, EPS, q8.LAYOUT_PLANE64, None, pq, ps, f32=False))
    for name in ("Wg", "Wu"):
        blocks = D.upload(synth.q4k_tensor("prefill_q4k", name))
        W = q8.Q4KWeights(blocks, K)
        C = torch.empty((T, W.n), device=D.dev)
        tg = timed(D, lambda i: q8.q4k_gemm(W, pq, ps, T, C), reps)
        launches += counted_launches(q8, lambda: q8.q4k_gemm(W, pq, ps, T, C))
        e = gemm_entry(tg, T, W.n, K)
        e["min_bytes"] = T * K + (T // 64 + 1) * (K // 32) * 256 + blocks.numel() + T * W.n * 4
        e["GBps_min_bytes"] = e["min_bytes"] / tg["mean_us"] / 1e3
        out[f"q4k_gemm_{name}_{W.n}x{K}"] = e
        total_us += tg["mean_us"]
        del W, C, blocks
    out["slice_launches"] = {"predicted": 3, "counted": launches}
    out["slice_tok_per_s"] = T / (total_us * 1e-6)
    return out


def bench_lm_head(D, reps):
    torch, q8 = D.torch, D.q8
    wl = "lm_head"
    N, K = 152064, 3584
    W = D.weights(wl, "W")
    n = max(2, math.ceil(COLD_BYTES / (W.qs.numel() * 1.0625)))
    Ws = D.copies(W, n)
    w = D.tensor(wl, "w_norm")
    x1 = D.tensor(wl, "x1")
    x512 = D.tensor(wl, "x512")
    out = {}
    y1 = torch.empty_like(x1)
    aq, asd = q8.alloc_act(1, K, q8.LAYOUT_ROW)
    logits = torch.empty(N, device=D.dev)
    t = timed(D, lambda i: q8.rmsnorm_quant(x1, w, EPS, q8.LAYOUT_ROW, y1, aq, asd), reps)
    out["rmsnorm_quant_row_3584"] = {**t, "bytes": rms_bytes(1, K), "GBps": rms_bytes(1, K) / t["mean_us"] / 1e3}
    tg = timed(D, lambda i: q8.q8_gemv(Ws[i % n], aq, asd, logits), reps)
    gb = gemv_bytes(N, K)
    out[f"q8_gemv_{N}x{K}"] = hbm_entry(tg, gb, read_b=gb - N * 4)
    out["t1_slice_tok_per_s_two_launches"] = 1.0 / ((t["mean_us"] + tg["mean_us"]) * 1e-6)

    # the T=1 slice in one launch: the output norm and the LM-head GEMV
    def t1_step(i):
        q8.rmsnorm_quant_gemv_shared_multi_plus_f32(x1, w, EPS, [Ws[i % n]], None, None, y1, aq, asd, [logits])
    ts = timed(D, t1_step, reps)
    sb = rms_bytes(1, K) + gb - (K + (K // 32) * 4)  # the GEMV reads its activation from LDS
    out["rmsnorm_quant_gemv_1x3584_152064"] = {**ts, "bytes": sb, "GBps": sb / ts["mean_us"] / 1e3,
                                               "frac_hbm": sb / ts["mean_us"] / 1e3 / HBM_PEAK_GBS}
    out["t1_slice_launches"] = {"predicted": 1, "counted": counted_launches(q8, lambda: t1_step(0))}
    out["t1_slice_tok_per_s"] = 1.0 / (ts["mean_us"] * 1e-6)
    T = 512
    y512 = torch.empty_like(x512)
    pq, ps = q8.alloc_act(T, K, q8.LAYOUT_PLANE64)
    C = torch.empty((T, N), device=D.dev)
    t = timed(D, lambda i: q8.rmsnorm_quant(x512, w, EPS, q8.LAYOUT_PLANE64, y512, pq, ps), reps)
    out["rmsnorm_quant_plane64_512"] = {**t, "bytes": rms_bytes(T, K, 1),
                                        "GBps": rms_bytes(T, K, 1) / t["mean_us"] / 1e3}
    t2 = timed(D, lambda i: q8.q8_gemm(Ws[i % n], pq, ps, T, C), max(3, reps // 2))
    out[f"q8_gemm_{N}x{K}_T512"] = gemm_entry(t2, T, N, K)
    out["t512_slice_launches"] = {"predicted": 2, "counted": counted_launches(q8, lambda: (
        q8.rmsnorm_quant(x512, w, EPS, q8.LAYOUT_PLANE64, y512, pq, ps), q8.q8_gemm(Ws[0], pq, ps, T, C)))}
    out["t512_slice_tok_per_s"] = T / ((t["mean_us"] + t2["mean_us"]) * 1e-6)
    return out


# ---------------------------------------------------------------------------
# CPU baseline: the oracle computing the decode step on this host
# ---------------------------------------------------------------------------
def cpu_gemv2048(budget_s, max_steps):
    """The oracle on the single 2048x2048 GEMV at batch 1 (quantize of x, then the GEMV reference),
    on all cores and on one thread: the same work as the GPU's q8_gemv_f32 launch."""
    import oracle
    import synth

    wl = "gemv_2048"
    x = synth.tensor(wl, "x").reshape(1, -1)
    wq, wd, _ = oracle.quantize(synth.tensor(wl, "W"))  # untimed: weights are quantized once, at load

    def one():
        aq, ad, _ = oracle.quantize(x)
        oracle.gemv(wq, wd, aq[0], ad[0])

    def sample(budget):
        one()  # warm
        t0 = time.perf_counter()
        k = 0
        while k < max_steps and (time.perf_counter() - t0) < budget:
            one()
            k += 1
        return k, time.perf_counter() - t0

    b = gemv_f32_bytes(2048, 2048)
    cores = oracle.num_threads()
    k, dt = sample(budget_s)
    oracle.set_threads(1)
    k1, dt1 = sample(budget_s / 2)
    oracle.set_threads(cores)
    return {"value": b * k / dt / 1e9, "unit": "GB/s", "cores": cores, "us_per_gemv": dt / k * 1e6,
            "sample": f"{k} GEMVs (quantize of x, then the f64 reference) in {dt:.1f} s",
            "single_thread": {"value": b * k1 / dt1 / 1e9, "unit": "GB/s", "cores": 1,
                              "us_per_gemv": dt1 / k1 * 1e6, "gemvs": k1}}


def cpu_baseline(budget_s=10.0, max_steps=100000):
    import numpy as np

    import oracle
    import synth

    wl = "decode_h7168"
    x = synth.tensor(wl, "x").reshape(1, -1)
    w = synth.tensor(wl, "w_norm")
    x128 = synth.tensor(wl, "x128").reshape(1, -1)
    Wq = {}
    for n in DEC_N:  # untimed: weights are quantized once, at load
        q, d, _ = oracle.quantize(synth.tensor(wl, n))
        Wq[n] = (q, d)

    def step():
        y = oracle.rmsnorm_f64(x, w, EPS).astype(np.float32)
        aq, ad, _ = oracle.quantize(y)
        for n in DEC_GROUP:
            oracle.gemv(Wq[n][0], Wq[n][1], aq[0], ad[0])
        bq, bd, _ = oracle.quantize(x128)
        oracle.gemv(Wq["W128"][0], Wq["W128"][1], bq[0], bd[0])

    step()  # warm
    t0 = time.perf_counter()
    k = 0
    while k < max_steps and (time.perf_counter() - t0) < budget_s:
        step()
        k += 1
    dt = time.perf_counter() - t0
    step_bytes = sum(decode_step_bytes().values())
    cores = oracle.num_threads()
    # the same steps on one thread, a shorter sample (the results do not depend on the thread count)
    oracle.set_threads(1)
    t1 = time.perf_counter()
    k1 = 0
    while k1 < max_steps and (time.perf_counter() - t1) < budget_s / 4:
        step()
        k1 += 1
    dt1 = time.perf_counter() - t1
    oracle.set_threads(cores)
    return {"value": step_bytes * k / dt / 1e9, "unit": "GB/s", "cores": cores, "kind": "oracle",
            "per_core_GBps": step_bytes * k / dt / 1e9 / cores,
            "gemv2048": cpu_gemv2048(budget_s / 4, max_steps),
            "sample": f"{k} full decode steps (rmsnorm + quantize, the six K=7168 GEMVs, quantize + GEMV "
                      f"for K=128; oracle references, f64) in {dt:.1f} s; "
                      "weights quantized once beforehand, untimed",
            "ms_per_step": dt / k * 1e3,
            "single_thread": {"value": step_bytes * k1 / dt1 / 1e9, "unit": "GB/s", "cores": 1,
                              "ms_per_step": dt1 / k1 * 1e3, "steps": k1}}


PROBE_GRID = [(1024, 1), (2048, 1), (4096, 1), (8192, 1), (2048, 2), (4096, 2), (2048, 4)]


def hbm_reference(D, mib=2048, reps=5):
    """Practical HBM rates on this GPU, the ceilings the fractions can also be read against:
    the library's read probe (q8_hbm_read_probe: a 2 GiB buffer streamed once per launch, larger
    than every cache) over a few launch shapes, the best reported; and a plain device copy."""
    torch, q8 = D.torch, D.q8
    n = mib * (1 << 20) // 4
    src = torch.ones(n, device=D.dev)
    out_words = torch.empty(65536, dtype=torch.int32, device=D.dev)
    sweep = {}
    for wgs, u in PROBE_GRID:
        t = timed(D, lambda i, wgs=wgs, u=u: q8.hbm_read_probe(src, wgs, u, out_words), reps)
        sweep[f"{wgs}wg_x{u}"] = {"mean_us": t["mean_us"], "GBps": n * 4 / t["mean_us"] / 1e3}
    best = max(sweep, key=lambda k: sweep[k]["GBps"])
    dst = torch.empty_like(src)
    tc = timed(D, lambda i: dst.copy_(src), reps)
    # the stream probe (q8_hbm_stream_probe) on the same buffers: writes only, and one read per write
    nb = n * 4
    tw = min((timed(D, lambda i, w=w: q8.hbm_stream_probe(nb, w, dst=dst), reps) for w in Practical.GRID),
             key=lambda t: t["mean_us"])
    tp = min((timed(D, lambda i, w=w: q8.hbm_stream_probe(nb, w, src0=src, dst=dst), reps)
              for w in Practical.GRID), key=lambda t: t["mean_us"])
    out = {"read_GBps": sweep[best]["GBps"], "read_bytes": n * 4, "read_launch": best,
           "read_kernel": "q8_hbm_read_probe (k_read_probe): 16-byte grid-stride loads, one pass, "
                          "workgroups x loads per lane in flight",
           "read_sweep": sweep, "frac_of_peak": sweep[best]["GBps"] / HBM_PEAK_GBS,
           "copy_bytes": 2 * n * 4, "copy_GBps": 2 * n * 4 / tc["mean_us"] / 1e3,
           "copy_kernel": "torch copy_ of a %d MiB f32 buffer" % mib,
           "write_GBps": nb / tw["mean_us"] / 1e3, "copy_probe_GBps": 2 * nb / tp["mean_us"] / 1e3,
           "write_kernel": "q8_hbm_stream_probe (k_stream_probe) with a destination only / one source "
                           "and one destination, 16-byte grid-stride, the better of %s workgroups"
                           % "/".join(map(str, Practical.GRID))}
    del src, dst, out_words
    torch.cuda.empty_cache()
    return out


# The pages' own figures for this path, with the hardware each page names (context beside the
# measured numbers, not targets: other GPUs, other models, whole-model or multi-GPU timings).
PAGES_CONTEXT = {
    "decode_tok_per_s": {
        "value": "3.54 -> 9.94 tok/s at 128k context (2.77x, bit-identical outputs)",
        "what": "end-to-end decode of a 93-layer MoE after the Q8_0 projection-path rewrite (five GEMV defects)",
        "hardware": "8x H200 SXM (sm_90), tensor parallel 8; the page calls each a 4.8 TB/s part",
        "source": "Part 4 - Lecture 05 - Fusion and the Activation-Quantization Discipline, s2.6"},
    "swiglu_quant_ms_per_call": {
        "value": "4.09 ms per call (the unfused swiglu + quantize pair: 5.46 ms)",
        "what": "fused SwiGLU + q8_0 plane producer at T=3325, nf=18944 (7B-class prefill), 27 calls per prefill",
        "hardware": "not named on the page",
        "source": "54 - r51 - producer-fused A-quantize mode 1, s5 (and s2.4)"},
    "int8_mmq_TMACps": {
        "value": "~6.1 TMAC/s (about 12 TOPS), 23 ms per ffn gate/up call",
        "what": "the int8 MMQ prefill GEMM with q4_K weights before its structural rewrite",
        "hardware": "not named on the page",
        "source": "12 - r5-r6 re-ranking + structural rewrite spec, s1"},
}


def traffic_for(kernel_key: str):
    """Measured HBM traffic of a kernel from profiles/traffic.json, if the kernel's sources have
    not changed since the counters were taken; else None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path)).get(kernel_key)
    except Exception:
        return None
    if not rec:
        return None
    h = hashlib.sha256()
    for f in rec["sources"]:
        h.update(open(os.path.join(ROOT, f), "rb").read())
    if h.hexdigest() != rec["sources_sha256"]:
        return None
    return rec["bytes_per_launch"]


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--reps", type=int, default=20, help="timed launches per kernel in the per-config section")
    ap.add_argument("--configs", default="all",
                    help="comma list of: decode,gemv2048,prefill_rms,prefill_swiglu,lm_head,prefill_q4k; "
                         "or ceilings (the practical HBM ceilings only)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="wall-clock budget of the oracle CPU baseline")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: the library has no multi-GPU path (asked for --gpus {args.gpus}).",
              file=sys.stderr)
        sys.exit(2)
    ensure_built()
    D = Dev()
    torch = D.torch
    torch.cuda.set_device(0)
    which = set(["decode", "gemv2048", "prefill_rms", "prefill_swiglu", "lm_head", "prefill_q4k"]) \
        if args.configs == "all" \
        else set(args.configs.split(","))
    global PRACTICAL
    PRACTICAL = Practical(D)
    if "ceilings" in which:  # the practical ceilings alone (for a trace of the probes)
        hbm = hbm_reference(D)
        for read_b, write_b in PRACTICAL_MIXES:
            PRACTICAL.ceiling(read_b, write_b)
        hbm["practical_ceilings"] = sorted(PRACTICAL.cache.values(), key=lambda c: (c["pattern"], c["bytes"]))
        print(json.dumps({"hbm_reference": hbm}), flush=True)
        return
    if "decode" not in which:  # profiling a subset: no headline line
        for name, fn in (("gemv2048", bench_gemv2048), ("prefill_rms", bench_prefill_rms),
                         ("prefill_swiglu", bench_prefill_swiglu), ("lm_head", bench_lm_head),
                         ("prefill_q4k", bench_prefill_q4k)):
            if name in which:
                log(f"[{name}] running")
                print(json.dumps({name: fn(D, args.reps)}), flush=True)
        return

    hbm = hbm_reference(D)
    log(f"[hbm] copy {hbm['copy_GBps']:.0f} GB/s, read {hbm['read_GBps']:.0f} GB/s ({hbm['read_launch']})")
    dec = bench_decode(D, args.steps, args.warmup, args.reps)
    log(f"[decode] {dec['value_GBps']:.1f} GB/s, {dec['ms_per_step'] * 1e3:.2f} us/step")
    per = {}
    for name, fn in (("gemv2048", bench_gemv2048), ("prefill_rms", bench_prefill_rms),
                     ("prefill_swiglu", bench_prefill_swiglu), ("lm_head", bench_lm_head),
                     ("prefill_q4k", bench_prefill_q4k)):
        if name in which:
            log(f"[{name}] running")
            per[name] = fn(D, args.reps)
            torch.cuda.empty_cache()
    dom_name = "rmsnorm_quant_gemv_shared_multi_plus_f32"
    dom = dec["components"][dom_name]
    # average launch duration: HIP events around a batch of back-to-back launches on the
    # launch stream (weights rotate over cold copies); per-launch event pairs are in components
    achieved = dom["bytes"] / (dom["batch_mean_us"] * 1e-6) / 1e9
    practical = PRACTICAL.ceiling(dom["bytes"], 0)
    roofline = {"bound": "hbm", "kernel": dom_name, "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": achieved / HBM_PEAK_GBS, "traffic": traffic_for(dom_name),
                "algorithmic_bytes": dom["bytes"], "mean_launch_us": dom["batch_mean_us"],
                "launches_timed": 4 * args.reps,
                "practical": practical, "frac_of_practical": achieved / practical["GBps"]}
    hbm["practical_ceilings"] = sorted(PRACTICAL.cache.values(), key=lambda c: (c["pattern"], c["bytes"]))
    PRACTICAL.pool = None
    torch.cuda.empty_cache()
    cpu = None
    if not args.no_cpu:
        log("[cpu] timing the oracle")
        cpu = cpu_baseline(budget_s=args.cpu_seconds)
    line = {
        "metric": METRIC, "value": dec["value_GBps"], "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": dec["ms_per_step"], "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "i8", "data": "synthetic",
        "config": {"workload": "decode_h7168", "batch": 1, "hidden": 7168,
                   "gemvs": "one launch (rmsnorm_quant_gemv_shared_multi_plus_f32): rmsnorm_quant ROW of the "
                            "row, the grouped GEMV over N=4096/512/512/4096/12288/96 (K=7168) on it, and the "
                            "N=4096 K=128 GEMV, whose f32 activation is quantized in the launch",
                   "launches_per_step": dec["launches_per_step"],
                   "launches_per_step_predicted": dec["launches_per_step_predicted"],
                   "launch_counts_per_step": dec["launch_counts_per_step"], "weight_copies": dec["copies"],
                   "timing": "HIP graph of all timed steps, HIP events around the replay",
                   "slice_tok_per_s": dec["slice_tok_per_s"],
                   "slice_tok_per_s_note": "one decode projection set (one layer's q/k/v/g, N=12288, N=96 and "
                                           "K=128 GEMVs with their producer) per token: a slice, not a model"},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "hbm_reference": hbm,
        "frac_of_measured_read": achieved / hbm["read_GBps"],
        "pages_context": PAGES_CONTEXT,
        "device": device_info(torch),
        "decode_warm": dec["warm"],
        "components": dec["components"],
        "per_config": per,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
