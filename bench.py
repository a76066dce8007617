#!/usr/bin/env python3
"""Decode-attention benchmark on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--chunk C]

A step is one decode step of the whole path: the chunk kernel
(gqa_decode_attn_*) and the merge kernel (gqa_decode_merge) over one batch of
seeded synthetic inputs already resident in HBM.  The default workload is the
int8 decode at context 32768 (8 sequences, 24 query / 2 KV heads, head_dim
256), the configuration the >= 70 % HBM-roofline goal is set on.

Reported (one JSON line on stdout):
  value        effective KV GB/s of the whole step = algorithmic KV bytes per
               step / wall-clock seconds per step (K steps back to back,
               bracketed by device synchronisation)
  ms_per_step  wall-clock milliseconds per step
  step_us_p10_p50_p90  percentiles of single steps (attention + merge), each
               between its own pair of HIP events
  cold_step_us_p10_p50_p90  the same for 20 steps each preceded (outside its
               events) by a 1 GiB streaming read that evicts every cache
  roofline     the chunk kernel alone: algorithmic bytes per launch / its
               mean duration from HIP events on its stream (bursts of
               back-to-back launches), against the 8 TB/s HBM peak; `traffic` is HBM bytes per launch measured
               with rocprofv3 counters (from profiles/, null when the kernel
               source changed since they were taken); `stream_read` is the
               rate of a plain streaming read of the same number of bytes
               (gqa_bench_stream_read, best of a few launch shapes), the
               machine's practical read ceiling, and the kernel's fraction
               of it
  cpu_baseline the fp64 oracle on the host cores over a bounded sample
  workloads    every other configuration (tiny f16, f16 batch, budgeted
               int8, f16 multi-query causal, or int8 32K when another one is
               named), measured the same way with at most 100 steps and no
               CPU baseline: step and chunk-kernel us, their fractions of
               8 TB/s and of the streaming read, HBM traffic over the
               algorithmic bytes (from profiles/)
To keep back-to-back steps from hitting the 256 MB last-level cache, the
inputs are replicated and the steps rotate through the copies, so every step
reads K/V that were last touched several hundred MB earlier.
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

HBM_PEAK_GBS = 8000.0
# G wave64 VALU instructions per second: 256 CUs x 4 SIMDs x 2.4 GHz, one
# instruction per SIMD every 4 cycles (16 lanes per cycle)
VALU_ISSUE_PEAK_G = 256 * 4 * 2.4 / 4
LLC_BYTES = 256 << 20
SETTLE_S = 0.05
PROFILES = os.path.join(ROOT, "profiles")


# the sources each measured kernel is built from: counters taken on one
# version of a kernel do not describe another
KERNEL_SOURCES = {
    "attn": ["attn_mfma.h", "mfma_util.h", "common.h", "gqa_decode.hip", "plan.h", "plan.cpp"],
    "merge": ["merge.hip", "common.h", "plan.h"],
    "append": ["append.hip"],
    "select": ["select.hip"],
    "tq": ["attn_tq.h", "mfma_util.h", "common.h", "tq.hip", "plan.h", "plan.cpp"],
}


def kernel_source_hash(kernel: str = "attn") -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "decode_attention_kv_gqa_amd", "csrc")
    for fn in KERNEL_SOURCES[kernel]:
        with open(os.path.join(csrc, fn), "rb") as f:
            h.update(fn.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def load_traffic_record(workload: str, kernel: str = "attn"):
    """The rocprofv3 counter record of the workload's measured kernel
    (profiles/traffic_<workload>.json), if it was taken on the current kernel
    source; else None."""
    path = os.path.join(PROFILES, f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_source_hash") != kernel_source_hash(kernel):
        return None
    return rec


def load_traffic(workload: str, kernel: str = "attn"):
    """HBM bytes per launch of the workload's measured kernel from rocprofv3
    counters, if they were taken on the current kernel source."""
    rec = load_traffic_record(workload, kernel)
    return None if rec is None else rec.get("hbm_bytes_per_launch")


def cpu_baseline(inp, budget_s: float = 12.0):
    """The fp64 oracle, as it stands, on the host cores: whole decode steps of
    the workload, or the first sequences of one when a step would take too
    long, repeated until about `budget_s` seconds of work."""
    import numpy as np
    from oracle.decode_ref import gqa_decode_ref
    from workloads import Inputs, kv_bytes
    threads = os.cpu_count()
    try:
        from threadpoolctl import threadpool_info
        info = [x for x in threadpool_info() if x.get("user_api") == "blas"]
        if info:
            threads = int(info[0]["num_threads"])
    except Exception:
        pass

    def sub(nseq):
        sl = slice(0, nseq)
        f = lambda x: None if x is None else x[sl]
        return Inputs(q=inp.q[sl], k=inp.k[sl], v=inp.v[sl], seq_lens=inp.seq_lens[sl],
                      scale=inp.scale, k_scales=f(inp.k_scales), v_scales=f(inp.v_scales),
                      ids=f(inp.ids))

    def run(x):
        t0 = time.perf_counter()
        gqa_decode_ref(x.q, x.k, x.v, x.seq_lens, x.scale, x.k_scales, x.v_scales, x.ids)
        return time.perf_counter() - t0

    S = inp.q.shape[0]
    one = sub(1)
    t1 = run(one)
    nseq = max(1, min(S, int(budget_s / max(t1, 1e-6))))
    x = sub(nseq)
    total_t, total_b, reps = 0.0, 0, 0
    while total_t < budget_s or reps == 0:
        total_t += run(x)
        total_b += kv_bytes(x)
        reps += 1
        if total_t > 3 * budget_s:
            break
    host = {"cpu_count": os.cpu_count(), "numpy": np.__version__}
    try:
        with open("/proc/cpuinfo") as f:
            host["cpu_model"] = next((ln.split(":", 1)[1].strip() for ln in f
                                      if ln.startswith("model name")), None)
    except OSError:
        pass
    try:
        blas = np.__config__.show(mode="dicts")["Build Dependencies"]["blas"]
        host["blas"] = f"{blas.get('name')} {blas.get('version')}"
    except Exception:
        pass
    return {"value": round(total_b / total_t / 1e9, 4), "unit": "GB/s", "cores": threads,
            "kind": "oracle", "host": host,
            "sample": f"{reps} run(s) of the fp64 oracle over the first {nseq} of {S} sequences "
                      f"({total_b} KV bytes, {total_t:.1f} s); numpy + OpenBLAS"}


def copy_calibration(nbytes: int = 1 << 30, reps: int = 5):
    """A plain device-to-device copy of known size: what rocprofv3's
    FETCH_SIZE / WRITE_SIZE read for it converts their units to bytes."""
    import torch
    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / reps
    print(json.dumps({"copy_bytes_read": nbytes, "copy_bytes_written": nbytes, "reps": reps,
                      "copy_GBps": round(2 * nbytes / dt / 1e9, 1)}), flush=True)


def stream_read_rate(nbytes: int, dev, shapes=(256, 512, 1024, 2048), reps: int = 20):
    """The machine's practical HBM read rate over nbytes: gqa_bench_stream_read
    (a plain 16-byte streaming read, include/gqa_bench.h) over buffers of that
    size rotated like the inputs, best of a few launch shapes, each timed with
    HIP events around `reps` back-to-back launches.  Checks that the XOR of
    the sink words equals the XOR of the buffer, i.e. that every byte was
    read.  Returns (GB/s, workgroups, bytes read)."""
    import torch
    import decode_attention_kv_gqa_amd as gq
    n = nbytes // 16 * 16
    copies = max(2, min(8, math.ceil(3 * LLC_BYTES / n) + 1))
    g = torch.Generator(device=dev).manual_seed(7)
    bufs = [torch.randint(-2 ** 31, 2 ** 31 - 1, (n // 4,), dtype=torch.int32, device=dev,
                          generator=g) for _ in range(copies)]
    sink = torch.zeros(max(shapes), dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream()

    def launch(i, wg):
        rc = gq.gqa_bench_stream_read(bufs[i % copies].data_ptr(), n, sink.data_ptr(), wg,
                                      stream.cuda_stream)
        if rc != 0:
            raise RuntimeError(f"gqa_bench_stream_read: {gq.strerror(rc)}")

    def xor_all(t):
        t = t.view(torch.int64) if t.numel() % 2 == 0 else t
        while t.numel() > 1:
            if t.numel() % 2:
                t = torch.cat([t, torch.zeros(1, dtype=t.dtype, device=t.device)])
            t = torch.bitwise_xor(t[0::2], t[1::2])
        return int(t.item())

    best = (float("inf"), 0)
    for wg in shapes:
        launch(0, wg)
        torch.cuda.synchronize()
        want = xor_all(bufs[0].clone())
        got = xor_all(sink[:wg].clone())
        if (want ^ (want >> 32)) & 0xffffffff != (got ^ (got >> 32)) & 0xffffffff:
            raise RuntimeError("gqa_bench_stream_read: sink XOR does not match the buffer")
        for i in range(5):
            launch(i, wg)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(reps):
            launch(i, wg)
        e1.record(stream)
        e1.synchronize()
        sec = e0.elapsed_time(e1) / reps / 1e3
        best = min(best, (sec, wg))
    del bufs
    return n / best[0] / 1e9, best[1], n


def bench_select(args):
    """Budget-selection kernel alone: one JSON line."""
    print(json.dumps(measure_select(args.workload, args.steps, args.warmup)), flush=True)


def measure_select(workload, steps, warmup):
    """Budget-selection kernel alone (gqa_decode_select_ids) on a selection
    workload: block scores resident in HBM, K launches timed with HIP events
    after W warm-up launches.  Returns the result dict."""
    import torch
    import decode_attention_kv_gqa_amd as gq
    from workloads import SELECT_WORKLOADS, make_block_scores
    w = SELECT_WORKLOADS[workload]
    S, T, Lmax, B = w["S"], w["T"], w["Lmax"], w["B"]
    dev = torch.device("cuda:0")
    bs = torch.from_numpy(make_block_scores(S, T, Lmax, seed=1000 + w["index"])).to(dev)
    lens = torch.full((S,), Lmax, dtype=torch.int32, device=dev)
    out = torch.full((S, T, B), -1, dtype=torch.int32, device=dev)
    for _ in range(warmup):
        gq.select_ids(bs, lens, B, out=out, Lmax=Lmax)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    stream = torch.cuda.current_stream()
    a.record(stream)
    for _ in range(steps):
        gq.select_ids(bs, lens, B, out=out, Lmax=Lmax)
    b.record(stream)
    torch.cuda.synchronize()
    us = a.elapsed_time(b) / steps * 1e3
    nbytes = S * T * ((Lmax // 4 + 1) * 4 + B * 4)    # scores read once + ids written
    return {
        "metric": "budget selection us per call", "value": round(us, 3), "unit": "us",
        "higher_is_better": False, "n_gpus": 1, "steps": steps, "warmup": warmup,
        "dtype": "f32 keys", "data": "synthetic (seeded numpy: block scores N(0,1) fp32)",
        "config": {"workload": workload, "S": S, "T": T, "Lmax": Lmax, "budget": B,
                   "algorithmic_bytes": nbytes},
        "roofline": {"bound": "hbm", "achieved": round(nbytes / us / 1e3, 2),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(nbytes / us / 1e3 / HBM_PEAK_GBS, 5), "traffic": None,
                     "note": "one workgroup per token; latency-bound at this size"}}


def bench_append(args):
    """Quantize-on-append kernel alone: one JSON line."""
    print(json.dumps(measure_append(args.workload, args.steps, args.warmup)), flush=True)


def measure_append(workload, steps, warmup):
    """Quantize-on-append kernel alone (gqa_decode_append_i8): new fp32 rows
    and the int8 cache resident in HBM, K launches timed with HIP events
    after W warm-up launches.  Returns the result dict."""
    import torch
    import decode_attention_kv_gqa_amd as gq
    from workloads import APPEND_WORKLOADS, make_append_rows
    w = APPEND_WORKLOADS[workload]
    S, Tn, Hk, D, Lmax = w["S"], w["Tn"], w["Hk"], w["D"], w["Lmax"]
    dev = torch.device("cuda:0")
    rows = make_append_rows(S, Tn, Hk, D, seed=1000 + w["index"])
    # several copies of the new rows, rotated, so a launch never finds its
    # input in the 256 MB last-level cache
    copies = max(2, math.ceil(2 * LLC_BYTES / (2 * rows[0].nbytes)) + 1)
    sets = [[torch.from_numpy(x).to(dev) for x in rows] for _ in range(copies)]
    pos = torch.full((S,), w["pos"], dtype=torch.int32, device=dev)
    k = torch.zeros((S, Lmax, Hk, D), dtype=torch.int8, device=dev)
    v = torch.zeros_like(k)
    ks = torch.zeros((S, Lmax, Hk, D // 64), dtype=torch.float16, device=dev)
    vs = torch.zeros_like(ks)
    for i in range(warmup):
        gq.append_i8(*sets[i % copies], pos, k, v, ks, vs)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    stream = torch.cuda.current_stream()
    a.record(stream)
    for i in range(steps):
        gq.append_i8(*sets[i % copies], pos, k, v, ks, vs)
    b.record(stream)
    torch.cuda.synchronize()
    us = a.elapsed_time(b) / steps * 1e3
    elems = 2 * S * Tn * Hk * D
    nbytes = elems * 4 + elems + elems // 64 * 2           # fp32 read, codes + scales written
    achieved = nbytes / us / 1e3
    return {
        "metric": "quantize-on-append GB/s", "value": round(achieved, 2), "unit": "GB/s",
        "higher_is_better": True, "n_gpus": 1, "steps": steps, "warmup": warmup,
        "us_per_call": round(us, 3), "dtype": "f32 -> i8",
        "data": "synthetic (seeded numpy: new rows N(0,1) fp32)",
        "config": {"workload": workload, "S": S, "Tn": Tn, "Hk": Hk, "D": D, "Lmax": Lmax,
                   "algorithmic_bytes": nbytes, "input_copies_rotated": copies},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": load_traffic(workload, "append")}}


def bench_tq(args):
    """Decode step over a TurboQuant-compressed cache: one JSON line."""
    import torch
    chunk = -1 if args.chunk is None else args.chunk
    print(json.dumps(measure_tq(args.workload, chunk, args.steps, args.warmup,
                                torch.device("cuda:0"), args.copies)), flush=True)


def measure_tq(workload, chunk, steps, warmup, dev, copies_arg=0):
    """Decode step over a TurboQuant-compressed cache (gqa_decode_attn_tq +
    gqa_decode_merge_tq): compressed cache resident in HBM, copies rotated so
    no step finds its cache in the last-level cache; K steps timed by wall
    clock, the chunk kernel alone by HIP events over bursts.  Returns the
    result dict."""
    import numpy as np
    import torch
    import decode_attention_kv_gqa_amd as gq
    from workloads import make_tq_inputs, tq_bytes
    inp = make_tq_inputs(workload)
    sh = inp.shape
    nbytes = tq_bytes(inp)
    d = lambda x: torch.from_numpy(np.ascontiguousarray(x.view(np.int32) if x.dtype == np.uint32
                                                        else x)).to(dev)
    foot = sum(x.nbytes for x in (inp.k_polar, inp.k_jl, inp.k_norms, inp.v_polar, inp.v_norms))
    copies = copies_arg or max(2, min(8, math.ceil(3 * LLC_BYTES / foot) + 1))
    sets = [dict(q_rot=d(inp.q_rot), q_jl=d(inp.q_jl), k_polar=d(inp.k_polar), k_jl=d(inp.k_jl),
                 k_norms=d(inp.k_norms), v_polar=d(inp.v_polar), v_norms=d(inp.v_norms))
            for _ in range(copies)]
    lens, signs = d(inp.seq_lens), d(inp.signs)
    step = gq.TqDecodeAttention(sh["S"], sh["T"], sh["H"], sh["Hk"], sh["D"], sh["Lmax"],
                                chunk=max(0, chunk), device=dev)

    def attn(i):
        x = sets[i % copies]
        step.attn(x["q_rot"], x["q_jl"], x["k_polar"], x["k_jl"], x["k_norms"], x["v_polar"],
                  x["v_norms"], lens, inp.centroids, inp.qjl_scale, inp.scale)

    def one(i):
        attn(i)
        step.merge(lens, signs)

    for i in range(warmup):
        one(i)
    torch.cuda.synchronize()
    t_w, extra = time.perf_counter(), 0
    while time.perf_counter() - t_w < SETTLE_S:
        for i in range(10):
            one(i)
        extra += 10
        torch.cuda.synchronize()
    K = steps
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        one(i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    stream = torch.cuda.current_stream()
    bursts, per = 5, max(1, K // 5)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(bursts)]
    for b in range(bursts):
        evs[b][0].record(stream)
        for i in range(per):
            attn(b * per + i)
        evs[b][1].record(stream)
    torch.cuda.synchronize()
    attn_ms = np.array([a.elapsed_time(b) / per for a, b in evs])
    kern_s = float(attn_ms.mean()) / 1e3
    achieved = nbytes / kern_s / 1e9
    # The kernel is bound by vector-ALU issue (unpacking the codes), so its
    # roofline is the issue rate of wave64 VALU instructions: 256 CUs x 4 SIMDs
    # x 2.4 GHz / 4 cycles per instruction = 614.4 G/s.  The instruction count
    # per launch comes from the rocprofv3 SQ_INSTS_VALU run kept in profiles/
    # (null once the kernel source changes); the HBM view is reported beside it.
    rec = load_traffic_record(workload, "tq")
    valu = rec.get("valu_wave_instructions_per_launch") if rec else None
    hbm = {"achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
           "frac": round(achieved / HBM_PEAK_GBS, 4),
           "traffic": rec.get("hbm_bytes_per_launch") if rec else None}
    roof = {"bound": "alu", "achieved": None, "peak": VALU_ISSUE_PEAK_G, "unit": "G VALU instr/s",
            "frac": None, "traffic": hbm["traffic"], "kernel": "attn_tq",
            "kernel_us_mean": round(kern_s * 1e6, 3),
            "kernel_us_burst_min_max": [round(float(attn_ms.min()) * 1e3, 3),
                                        round(float(attn_ms.max()) * 1e3, 3)],
            "hbm_view": hbm}
    if valu:
        roof["achieved"] = round(valu / kern_s / 1e9, 2)
        roof["frac"] = round(valu / kern_s / 1e9 / VALU_ISSUE_PEAK_G, 4)
    return {
        "metric": "TurboQuant-cache decode effective cache GB/s and us/step, 1 MI355X",
        "value": round(nbytes / (wall / K) / 1e9, 2), "unit": "GB/s", "n_gpus": 1, "steps": K,
        "warmup": warmup, "extra_warmup_steps": extra, "us_per_step": round(wall / K * 1e6, 2),
        "higher_is_better": True, "dtype": "2-bit polar + 1-bit QJL codes, f16 norms",
        "data": "synthetic (seeded numpy: uniform codes, f16 norms, N(0,1) rotated queries)",
        "config": {"workload": workload, **sh, "chunk": step.chunk,
                   "cache_bytes_per_step": nbytes, "input_copies_rotated": copies},
        "roofline": roof}


def measure_attention(name, chunk, steps, warmup, dev, gate=False, copies=0, cold=20,
                      with_stream_read=True, sort_ids=True):
    """One attention workload on the GPU: seeded inputs resident in HBM (as
    many copies as keep successive steps out of the last-level cache), K
    steps of attention + merge back to back (wall clock bracketed by device
    synchronisation), the chunk kernel alone from HIP events around bursts of
    back-to-back launches on its stream, single steps between their own
    events, cold steps, and a plain streaming read of the same bytes.  With
    sort_ids False a gathered workload's ids keep the order they were drawn
    in (no counter record applies then: traffic is None).
    Returns (result dict, inputs)."""
    import numpy as np
    import torch
    import decode_attention_kv_gqa_amd as gq
    from workloads import WORKLOADS, make_inputs, kv_bytes

    w = WORKLOADS[name]
    chunk = w.chunk if chunk is None else chunk
    t_gen = time.perf_counter()
    inp = make_inputs(name, sort_ids=sort_ids)
    step_bytes = kv_bytes(inp)
    sh = inp.shape
    print(f"[bench] {name}: inputs drawn in {time.perf_counter() - t_gen:.1f} s, "
          f"{step_bytes} KV bytes/step", file=sys.stderr, flush=True)

    # resident footprint of one copy of the inputs
    foot = sum(x.nbytes for x in (inp.q, inp.k, inp.v, inp.k_scales, inp.v_scales, inp.ids)
               if x is not None)
    copies = copies or max(2, min(8, math.ceil(3 * LLC_BYTES / foot) + 1))
    d = lambda x: None if x is None else torch.from_numpy(x).to(dev)
    sets = []
    gate_np = None
    if gate:
        # the output gate as the second half of [query | gate] rows
        gate_np = np.random.default_rng(2000 + w.index).standard_normal(inp.q.shape).astype(np.float32)
    for _ in range(copies):
        x = dict(q=d(inp.q), k=d(inp.k), v=d(inp.v), seq_lens=d(inp.seq_lens),
                 k_scales=d(inp.k_scales), v_scales=d(inp.v_scales), ids=d(inp.ids), gate=None)
        if gate:
            full = d(np.concatenate([inp.q, gate_np], axis=-1))
            x["q"] = full[..., :sh["D"]].contiguous()
            x["gate"] = full[..., sh["D"]:]
        sets.append(x)
    step = gq.DecodeAttention(sh["S"], sh["T"], sh["H"], sh["Hk"], sh["D"], sh["Lmax"], inp.kv,
                              B=sh["B"], chunk=chunk, device=dev)
    stream = torch.cuda.current_stream()

    def attn(i):
        x = sets[i % copies]
        step.attn(x["q"], x["k"], x["v"], x["seq_lens"], inp.scale, x["k_scales"], x["v_scales"],
                  x["ids"])

    def one(i):
        x = sets[i % copies]
        attn(i)
        step.merge(x["seq_lens"], x["ids"], gate=x["gate"],
                   gate_stride=None if x["gate"] is None else 2 * sh["D"])

    for i in range(warmup):
        one(i)
    torch.cuda.synchronize()
    # The GPU's clocks take a few milliseconds of sustained load to settle; a
    # short warm-up leaves the first timed steps ~10 % slow.  Keep stepping
    # (untimed) until at least SETTLE_S of warm-up has run.
    extra = 0
    t_w = time.perf_counter()
    while time.perf_counter() - t_w < SETTLE_S:
        for i in range(10):
            one(warmup + extra + i)
        extra += 10
        torch.cuda.synchronize()

    # timed region: K steps back to back, wall clock bracketed by synchronisation
    K = steps
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        one(i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    # chunk-kernel duration from HIP events on the launch stream, in a pass of
    # its own after the timed steps: bursts of back-to-back chunk-kernel
    # launches (rotating input copies) between two events, so the figure is
    # the kernel's launch-to-launch time and carries no per-event overhead.
    bursts, per = 5, max(1, K // 5)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(bursts)]
    torch.cuda.synchronize()
    for b in range(bursts):
        evs[b][0].record(stream)
        for i in range(per):
            attn(b * per + i)
        evs[b][1].record(stream)
    torch.cuda.synchronize()
    attn_ms = np.array([a.elapsed_time(b) / per for a, b in evs])
    attn_mean_s = float(attn_ms.mean()) / 1e3

    # spread of single steps: each step (attention + merge) between its own
    # pair of events, input copies still rotating
    nst = min(K, 100)
    sev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(nst)]
    torch.cuda.synchronize()
    for i in range(nst):
        sev[i][0].record(stream)
        one(i)
        sev[i][1].record(stream)
    torch.cuda.synchronize()
    step_us = np.array([a.elapsed_time(b) * 1e3 for a, b in sev])

    # cold steps: a 1 GiB scratch buffer is read between steps (outside the
    # events), so neither the L2s nor the 256 MB last-level cache hold
    # anything of the step's inputs or partials.  A read, not a write: a
    # written buffer would leave up to 256 MB of dirty lines whose write-back
    # then competes with the step's reads.
    cold_us = None
    if cold:
        scratch = torch.zeros(1 << 30, dtype=torch.uint8, device=dev)
        sink = torch.empty(512, dtype=torch.int32, device=dev)
        flush = lambda: gq.gqa_bench_stream_read(scratch.data_ptr(), scratch.numel(),
                                                 sink.data_ptr(), 512, stream.cuda_stream)
        for _ in range(2):
            flush()
        cev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(cold)]
        torch.cuda.synchronize()
        for i in range(cold):
            flush()
            cev[i][0].record(stream)
            one(i)
            cev[i][1].record(stream)
        torch.cuda.synchronize()
        cold_us = np.array([a.elapsed_time(b) * 1e3 for a, b in cev])
        del scratch

    achieved = step_bytes / attn_mean_s / 1e9
    traffic = load_traffic(name) if sort_ids or inp.ids is None else None
    res = {
        "value": round(step_bytes / (wall / K) / 1e9, 2),
        "ms_per_step": round(wall / K * 1e3, 5),
        "us_per_step": round(wall / K * 1e6, 2),
        "step_us_p10_p50_p90": [round(float(np.percentile(step_us, q)), 2) for q in (10, 50, 90)],
        "pct_of_hbm_peak": round(100 * step_bytes / (wall / K) / 1e9 / HBM_PEAK_GBS, 2),
        "extra_warmup_steps": extra,
        "chunk": step.chunk,
        "kv_bytes_per_step": step_bytes,
        "input_copies_rotated": copies,
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic,
                     "traffic_over_algorithmic": (round(traffic / step_bytes, 4)
                                                  if traffic else None),
                     "kernel": "attn_chunk",
                     "kernel_us_mean": round(attn_mean_s * 1e6, 3),
                     "kernel_us_burst_min_max": [round(float(attn_ms.min()) * 1e3, 3),
                                                 round(float(attn_ms.max()) * 1e3, 3)]},
    }
    if cold_us is not None:
        res["cold_step_us_p10_p50_p90"] = [round(float(np.percentile(cold_us, q)), 2)
                                           for q in (10, 50, 90)]
    if with_stream_read:
        sr_gbs, sr_wg, sr_bytes = stream_read_rate(step_bytes, dev)
        res["roofline"]["stream_read"] = {"gbs": round(sr_gbs, 2), "bytes": sr_bytes,
                                          "workgroups": sr_wg,
                                          "kernel_frac_of_stream_read": round(achieved / sr_gbs, 4)}
    del sets, step
    torch.cuda.empty_cache()
    return res, inp


def launch_floor():
    """How long a launch takes that does the int8 32K merge's memory work and
    no arithmetic: gqa_bench_stream_read over 3 MiB with 192 workgroups (the
    merge reads 192 rows x 16 partials of 1 KB), and over 16 KiB with one
    workgroup.  Each shape is timed one launch at a time (HIP events around a
    single launch, synchronised between launches; median of 200) and back to
    back (mean over 200).  Then runs the int8 32K merge alone and attention +
    merge steps, for a kernel trace to compare."""
    import statistics
    import torch
    import decode_attention_kv_gqa_amd as gq
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    res = {}
    for name, nbytes, wg in (("merge_shape", 3 << 20, 192), ("one_workgroup", 16 << 10, 1)):
        buf = torch.ones(nbytes // 4, dtype=torch.int32, device=dev)
        sink = torch.zeros(wg, dtype=torch.int32, device=dev)

        def launch():
            rc = gq.gqa_bench_stream_read(buf.data_ptr(), nbytes, sink.data_ptr(), wg,
                                          stream.cuda_stream)
            if rc != 0:
                raise RuntimeError(f"gqa_bench_stream_read: {gq.strerror(rc)}")
        for _ in range(50):
            launch()
        torch.cuda.synchronize()
        single = []
        for _ in range(200):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            launch()
            e1.record(stream)
            e1.synchronize()
            single.append(e0.elapsed_time(e1) * 1e3)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(200):
            launch()
        e1.record(stream)
        e1.synchronize()
        res[name] = {"bytes": nbytes, "workgroups": wg,
                     "us_single_p50": round(statistics.median(single), 3),
                     "us_back_to_back": round(e0.elapsed_time(e1) * 1e3 / 200, 3)}
    # the int8 32K merge on its own, 300 times over one set of partials, then
    # 100 attention + merge steps: a kernel trace of this run gives the
    # merge's duration on partials it has read before and right after the
    # attention launch that wrote them
    from workloads import make_inputs
    inp = make_inputs("i8_32k")
    dd = lambda x: None if x is None else torch.from_numpy(x).to(dev)
    q, k, v, ks, vs, sl = (dd(inp.q), dd(inp.k), dd(inp.v), dd(inp.k_scales), dd(inp.v_scales),
                           dd(inp.seq_lens))
    S, T, H, D = inp.q.shape
    step = gq.DecodeAttention(S, T, H, inp.k.shape[2], D, inp.k.shape[1], "i8")
    for _ in range(20):
        step(q, k, v, sl, inp.scale, ks, vs)
    torch.cuda.synchronize()
    for _ in range(300):
        step.merge(sl)
    for _ in range(100):
        step(q, k, v, sl, inp.scale, ks, vs)
    torch.cuda.synchronize()
    print(json.dumps({"launch_floor": res}))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="i8_32k")
    ap.add_argument("--chunk", type=int, default=None,
                    help="cells per split (default: the workload's); 0: the library's choice")
    ap.add_argument("--pieces", type=int, default=0,
                    help="balanced partition: the batch's windows cut into P pieces per KV head "
                         "(dense workloads; overrides --chunk)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-other-workloads", action="store_true",
                    help="measure only the named workload (by default the int8 32K headline "
                         "run also measures every other configuration, with fewer steps)")
    ap.add_argument("--gate", action="store_true",
                    help="merge with the output gate (gate rows interleaved with the query)")
    ap.add_argument("--copies", type=int, default=0, help="input replicas to rotate through")
    ap.add_argument("--unsorted-ids", action="store_true",
                    help="gathered workloads: ids in the order drawn instead of ascending")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy 5 times (HBM counter calibration)")
    ap.add_argument("--launch-floor", action="store_true",
                    help="only time a streaming read doing the int8 32K merge's memory work "
                         "(and a one-workgroup read): the cost of a launch that reads memory")
    args = ap.parse_args()
    if args.copy_calibration:
        copy_calibration()
        return
    if args.launch_floor:
        launch_floor()
        return

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the decode-attention path here is a single-GPU "
              "kernel pair (multi-GPU sharding is a design note, not built); run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from workloads import WORKLOADS, WORKLOAD_ORDER, SELECT_WORKLOADS, APPEND_WORKLOADS, TQ_WORKLOADS

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.workload in SELECT_WORKLOADS:
        bench_select(args)
        return
    if args.workload in APPEND_WORKLOADS:
        bench_append(args)
        return
    if args.workload in TQ_WORKLOADS:
        bench_tq(args)
        return
    dev = torch.device("cuda:0")
    w = WORKLOADS[args.workload]
    chunk = -args.pieces if args.pieces > 0 else args.chunk
    m, inp = measure_attention(args.workload, chunk, args.steps, args.warmup, dev,
                               gate=args.gate, copies=args.copies,
                               sort_ids=not args.unsorted_ids)
    sh = inp.shape
    res = {
        "metric": "decode-attention effective KV HBM GB/s (% of peak) and us/step, 1 MI355X",
        "value": m["value"],
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "extra_warmup_steps": m["extra_warmup_steps"],
        "ms_per_step": m["ms_per_step"],
        "us_per_step": m["us_per_step"],
        "step_us_p10_p50_p90": m["step_us_p10_p50_p90"],
        "cold_step_us_p10_p50_p90": m["cold_step_us_p10_p50_p90"],
        "pct_of_hbm_peak": m["pct_of_hbm_peak"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "i8" if inp.kv == "i8" else "f16",
        "data": "synthetic (seeded numpy: q N(0,1) fp32; " +
                ("K/V int8 U[-127,127], f16 scales U[0.005,0.02])" if inp.kv == "i8"
                 else "K/V f16 N(0,1))"),
        "config": {"workload": args.workload, "S": sh["S"], "T": sh["T"], "H": sh["H"],
                   "Hk": sh["Hk"], "D": sh["D"], "Lmax": sh["Lmax"], "budget": sh["B"],
                   "kv": inp.kv, "chunk": m["chunk"], "kv_bytes_per_step": m["kv_bytes_per_step"],
                   "input_copies_rotated": m["input_copies_rotated"],
                   "output_gate": bool(args.gate), "ids_sorted": not args.unsorted_ids,
                   "description": w.description},
        "roofline": m["roofline"],
    }
    if not args.no_cpu_baseline:
        print("[bench] timing the fp64 oracle on the host", file=sys.stderr, flush=True)
        res["cpu_baseline"] = cpu_baseline(inp)
    del inp
    if not args.no_other_workloads and not args.gate and chunk is None:
        # every other configuration, measured the same way with fewer steps
        # (no CPU baseline); the line's value stays the named workload's
        res["workloads"] = {}
        # gathered workloads once more with their ids in the order drawn
        # (the selection emits them ascending, which the named line uses)
        runs = [(n, True) for n in WORKLOAD_ORDER]
        runs += [(n, False) for n in WORKLOAD_ORDER if WORKLOADS[n].budget > 0]
        for name, sort_ids in runs:
            if name == args.workload and sort_ids != args.unsorted_ids:
                continue
            o, _ = measure_attention(name, None, min(args.steps, 100), min(args.warmup, 10), dev,
                                     cold=10, sort_ids=sort_ids)
            r = o["roofline"]
            key = name if sort_ids else name + "_unsorted_ids"
            res["workloads"][key] = {
                "description": WORKLOADS[name].description +
                               ("" if sort_ids else "; ids in the order drawn"),
                "chunk": o["chunk"],
                "kv_bytes_per_step": o["kv_bytes_per_step"], "us_per_step": o["us_per_step"],
                "step_us_p10_p50_p90": o["step_us_p10_p50_p90"],
                "cold_step_us_p10_p50_p90": o["cold_step_us_p10_p50_p90"],
                "step_GBps": o["value"], "step_frac_of_peak": round(o["value"] / HBM_PEAK_GBS, 4),
                "kernel_us_mean": r["kernel_us_mean"], "kernel_GBps": r["achieved"],
                "kernel_frac_of_peak": r["frac"],
                "kernel_frac_of_stream_read": r["stream_read"]["kernel_frac_of_stream_read"],
                "stream_read_GBps": r["stream_read"]["gbs"],
                "traffic": r["traffic"], "traffic_over_algorithmic": r["traffic_over_algorithmic"]}
        # the decode over a TurboQuant-compressed cache (its own metric: GB/s
        # of codes; bound by instruction issue, so the VALU fraction beside)
        for name in TQ_WORKLOADS:
            o = measure_tq(name, -1, min(args.steps, 100), min(args.warmup, 10), dev)
            r = o["roofline"]
            res["workloads"][name] = {
                "description": "TurboQuant-compressed cache: 4 seqs at context 131072, 32/8 heads, "
                               "hd 128, 2-bit polar keys/values + 1-bit QJL signs",
                "chunk": o["config"]["chunk"],
                "cache_bytes_per_step": o["config"]["cache_bytes_per_step"],
                "us_per_step": o["us_per_step"], "step_GBps": o["value"],
                "step_frac_of_peak": round(o["value"] / HBM_PEAK_GBS, 4),
                "kernel_us_mean": r["kernel_us_mean"], "kernel_GBps": r["hbm_view"]["achieved"],
                "kernel_frac_of_peak": r["hbm_view"]["frac"],
                "kernel_valu_frac_of_issue_peak": r["frac"], "traffic": r["traffic"]}
        # the two kernels beside the decode: budget selection and
        # quantize-on-append (each alone, HIP events around 200 launches)
        for name in SELECT_WORKLOADS:
            o = measure_select(name, 200, 20)
            res["workloads"][name] = {"kernel": "select_ids", "us_per_call": o["value"],
                                      "config": o["config"], "GBps": o["roofline"]["achieved"]}
        for name in APPEND_WORKLOADS:
            o = measure_append(name, 200, 20)
            res["workloads"][name] = {"kernel": "append_i8", "us_per_call": o["us_per_call"],
                                      "config": o["config"], "GBps": o["value"],
                                      "frac_of_peak": o["roofline"]["frac"],
                                      "traffic": o["roofline"]["traffic"]}
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
