"""Benchmark of the SWA(w,s) hot path on one MI355X.

    python bench.py [--steps K] [--warmup W] [--w 512] [--no-cpu]

Prints ONE JSON line.  The headline workload is the Llama-3.1-8B-shaped
prefill (B=1, 32 query / 8 kv heads, d=128, L=4096, bf16, SWA(w,4), sink-key
outliers): one step is one swa_prefill call over that batch, and `value` is
its algorithmic TFLOP/s, 4*d*Hq*sum_t min(t,w) flops per step.  The streaming
decode of the same model shape (batch 64, SWA(w,4), full window) is measured
in the same run and reported under "decode": one step appends one position
and decodes it in each of 4 layer caches (4 x 128 MiB at w=512, more than the
256 MB Infinity Cache, so the KV reads come from HBM), and its headline is KV
GB/s.  Every roofline figure uses the average duration of the named kernel's
launches, timed with HIP events on the stream it runs on.  The oracle's CPU
time on the same prefill is reported as cpu_baseline.

Also in the line: the prefill at every window (w = 128, 256, 512) with its
fraction of the attainable roofline min(MFMA peak, AI x HBM peak), warm (one
80 MiB input set, resident in the 256 MB Infinity Cache) and cold (8 sets,
640 MiB, read from HBM); a cold w=64 decode (>= 512 MiB of caches rotated);
the achievable HBM read and bf16 MFMA rates measured on this GPU
(libswa_peaks.so) beside the vendor peaks; n = 2^7, 2^12, 2^18 of the
long-context sweep, on the 32/8-head model and on the decode-speed figure's own
4-layer model (16 heads of 64, multi-head, batch 1); the small fp32 parity
configuration, timed for information; and oracle timings of the other workloads.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0      # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, TFLOP/s
RIDGE = BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)  # flop per byte

METRIC = "SWA(w,4) decode KV GB/s (% HBM peak) + prefill TFLOP/s (% MFMA peak)"
# The decode-speed figure's own model: 4 layers of width 1024 as 16 heads of 64,
# multi-head (one kv-head per query head), batch 1.
PAGES_MODEL = {"layers": 4, "q_heads": 16, "kv_heads": 16, "head_dim": 64, "batch": 1}


def pairs(L, w):
    """Attended (query, key) pairs of one head over a prompt of L tokens."""
    return sum(min(t, w) for t in range(1, L + 1))


def prefill_work(B, L, Hq, Hkv, d, w, es=2):
    flops = 4.0 * d * Hq * B * pairs(L, w)
    nbytes = es * (2 * B * L * Hq * d + 2 * B * L * Hkv * d)  # Q, O, K, V once
    return flops, nbytes


class Pacer:
    """Keeps the GPU queue ahead of the host in a timed region.

    The host needs tens of microseconds to enqueue one library call (Python,
    ctypes), more than a short decode kernel runs.  A spin kernel enqueued
    first keeps the GPU busy while the host enqueues the whole timed region, so
    the HIP events around each launch bracket the kernel itself, and the
    region's total is GPU time for back-to-back steps.
    """

    def __init__(self, torch):
        self.torch = torch
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record()
        torch.cuda._sleep(1_000_000)
        b.record()
        torch.cuda.synchronize()
        self.ms_per_mcycle = max(a.elapsed_time(b), 1e-3)

    def lead(self, host_ms):
        """Enqueue a spin of about 1.5 x host_ms + 2 ms."""
        cycles = int((1.5 * host_ms + 2.0) / self.ms_per_mcycle * 1e6)
        self.torch.cuda._sleep(max(cycles, 1000))


WARM_MS = 500.0  # untimed GPU work before each timed region: the clocks settle after a few hundred ms of load


def timed_region(torch, pacer, step, steps, warmup, warm=None):
    """warmup untimed calls of warm() (more if they ran for less than WARM_MS),
    then `steps` timed calls of step() back to back between two HIP events on
    the current stream.  Returns the region's ms.  warm defaults to step; a
    step that changes state the measurement depends on (an append into a cache
    that is still growing) passes one that does not."""
    warm = warm or step
    w0 = torch.cuda.Event(enable_timing=True)
    w1 = torch.cuda.Event(enable_timing=True)
    w0.record()
    for _ in range(max(warmup, 1)):
        warm()
    w1.record()
    torch.cuda.synchronize()
    warm_ms = w0.elapsed_time(w1)
    if warm_ms < WARM_MS:
        for _ in range(int((WARM_MS - warm_ms) / max(warm_ms / max(warmup, 1), 1e-3)) + 1):
            warm()
        torch.cuda.synchronize()
    t = time.perf_counter()  # host time to enqueue a region (sizes the lead spin)
    for _ in range(steps):
        warm()
    host_ms = (time.perf_counter() - t) * 1e3
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    pacer.lead(host_ms)
    t0.record()
    for _ in range(steps):
        step()
    t1.record()
    torch.cuda.synchronize()
    return t0.elapsed_time(t1)


# HBM traffic per launch from rocprofv3 FETCH_SIZE / WRITE_SIZE passes, scaled by
# what the same counters read for a plain 256 MiB copy (FETCH_SIZE x2.0,
# WRITE_SIZE x1.0 on this GPU).  Keyed by the SHA-256 of the kernel sources
# the counters were taken on; reported as null once those sources change.
TRAFFIC = {
    "prefill_w512": {"sources": ["prefill.hip", "device_common.h"],
                    "sha256": "e929a7ddd2a4e5309b260e623b6f425ab7102b9d832a7264c772f6d2f8d2281b",
                    "bytes": (2 * 24696 + 32768) * 1024},
    "decode_w512": {"sources": ["decode.hip", "device_common.h"],
                   "sha256": "21060d6cb8112bdd0ec60345eb50386e2c98761a9033f26daf3a9624584fd459",
                   "bytes": (2 * 65857 + 512) * 1024},
    "decode_w64": {"sources": ["decode.hip", "device_common.h"],
                  "sha256": "21060d6cb8112bdd0ec60345eb50386e2c98761a9033f26daf3a9624584fd459",
                  "bytes": (2 * 8500 + 512) * 1024},
    "fp8_decode_w512": {"sources": ["decode.hip", "device_common.h"],
                       "sha256": "21060d6cb8112bdd0ec60345eb50386e2c98761a9033f26daf3a9624584fd459",
                       "bytes": (2 * 33079 + 512) * 1024},
    "fp8_decode_w64": {"sources": ["decode.hip", "device_common.h"],
                      "sha256": "21060d6cb8112bdd0ec60345eb50386e2c98761a9033f26daf3a9624584fd459",
                      "bytes": (2 * 4411 + 512) * 1024},
}


def kernel_sha(sources):
    import hashlib
    h = hashlib.sha256()
    for name in sources:
        with open(os.path.join(ROOT, "sliding_window_sink_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def traffic(key):
    entry = TRAFFIC.get(key)
    if not entry or entry["bytes"] is None or entry["sha256"] != kernel_sha(entry["sources"]):
        return None
    return entry["bytes"]


def attainable(ai, mfma_tflops, hbm_gbs):
    """Roofline ceiling in TFLOP/s for arithmetic intensity ai (flop/B)."""
    return min(mfma_tflops, ai * hbm_gbs / 1e3)


def bench_prefill(swa, torch, pacer, args, w, cold=False, peaks=None):
    """The Llama-3.1-8B-shaped prefill at SWA(w,4).  Warm: one input set
    re-read every step (its 80 MiB stay in the 256 MB Infinity Cache).  Cold:
    8 distinct input sets (640 MiB) taken in turn, so each step's Q, K, V
    come from HBM and its O goes there."""
    import synth
    B, L, Hq, Hkv, d, s = 1, 4096, 32, 8, 128, 4
    Q, K, V = synth.prefill_inputs(B, L, Hq, Hkv, d, seed=0, workload=2, bf16=True, sink_outliers=4)
    q, k, v = (torch.from_numpy(a).to("cuda", torch.bfloat16) for a in (Q, K, V))
    sets = [(q, k, v, torch.empty_like(q))]
    if cold:
        # distinct memory with the same statistics: the sequence rolled by
        # a different offset per set (sink rows move with it; timing only)
        for j in range(1, 8):
            sets.append((q.roll(37 * j, 1).contiguous(), k.roll(37 * j, 1).contiguous(),
                         v.roll(37 * j, 1).contiguous(), torch.empty_like(q)))
    flops, nbytes = prefill_work(B, L, Hq, Hkv, d, w)
    state = {"i": 0}

    def step():
        qq, kk, vv, oo = sets[state["i"] % len(sets)]
        state["i"] += 1
        swa.prefill(qq, kk, vv, w, s, out=oo)

    # One step = one launch, so the region's mean step is the kernel's mean
    # launch duration (plus the gap between back-to-back launches).
    total_ms = timed_region(torch, pacer, step, args.steps, args.warmup)
    ms_step = avg_ms = total_ms / args.steps
    ai = flops / nbytes
    bound = "mfma" if ai >= RIDGE else "hbm"
    tflops = flops / (avg_ms * 1e-3) / 1e12
    if bound == "mfma":
        achieved, peak, unit = tflops, BF16_PEAK_TFLOPS, "TFLOP/s"
    else:
        achieved, peak, unit = nbytes / (avg_ms * 1e-3) / 1e9, HBM_PEAK_GBS, "GB/s"
    ceil_vendor = attainable(ai, BF16_PEAK_TFLOPS, HBM_PEAK_GBS)
    res = {
        "w": w, "inputs": "cold (8 sets, 640 MiB)" if cold else "warm (one 80 MiB set)",
        "tflops": tflops,
        "ms_per_step": ms_step,
        "kernel_ms": avg_ms,
        "flops_per_step": flops,
        "bytes_per_step": nbytes,
        "arith_intensity": ai,
        "mfma_frac": tflops / BF16_PEAK_TFLOPS,
        "attainable_tflops": ceil_vendor,
        "attainable_frac": tflops / ceil_vendor,
        "hbm_gbs": nbytes / (avg_ms * 1e-3) / 1e9,
        "roofline": {"kernel": "swa_prefill_kernel<bf16,bf16,128,4>", "bound": bound,
                     "achieved": achieved, "peak": peak, "unit": unit,
                     "frac": achieved / peak,
                     "traffic": None if cold else traffic("prefill_w%d" % w),
                     "mfma_frac": tflops / BF16_PEAK_TFLOPS,
                     "hbm_gbs": nbytes / (avg_ms * 1e-3) / 1e9},
    }
    if peaks:
        ceil_meas = attainable(ai, peaks["mfma_tflops"], peaks["hbm_read_gbs"])
        res["attainable_tflops_measured_peaks"] = ceil_meas
        res["attainable_frac_measured_peaks"] = tflops / ceil_meas
    return res, (Q, K, V, w, s, flops)


def bench_decode(swa, torch, pacer, args, w, layers=4, fp8=False):
    """Batch-64 decode step over `layers` layers of 32/8 heads, d=128, at a
    full SWA(w,4) window; fp8=True keeps the caches as E4M3 codes with
    per-kv-head scales (new rows and queries stay bf16)."""
    import synth
    B, Hq, Hkv, d, s = 64, 32, 8, 128, 4
    es = 1 if fp8 else 2  # cache bytes per element
    caches = []
    for layer in range(layers):
        if fp8:
            sc = torch.full((2, Hkv), 4.0 / 448.0, dtype=torch.float32, device="cuda")
            c = swa.Cache(B, Hkv, d, w, s, dtype=torch.float8_e4m3fn, kv_scale=sc)
        else:
            c = swa.Cache(B, Hkv, d, w, s, dtype=torch.bfloat16)
        Kp, Vp = synth.prompt_rows(B, Hkv, d, 1, w, seed=0, workload=3, layer=layer, bf16=True)
        c.append(torch.from_numpy(Kp).to("cuda", torch.bfloat16),
                 torch.from_numpy(Vp).to("cuda", torch.bfloat16))
        caches.append(c)
    bank = 4  # per-step inputs kept resident and cycled
    qs, ks, vs = [], [], []
    for j in range(bank):
        pos = w + 1 + j
        qs.append(torch.from_numpy(synth.query_rows(B, Hq, d, pos)).to("cuda", torch.bfloat16))
        Kn, Vn = synth.position_rows(B, Hkv, d, [pos], seed=0, workload=3, bf16=True)
        ks.append(torch.from_numpy(Kn).to("cuda", torch.bfloat16))
        vs.append(torch.from_numpy(Vn).to("cuda", torch.bfloat16))
    outs = [torch.empty((B, Hq, d), dtype=torch.bfloat16, device="cuda") for _ in range(layers)]
    state = {"i": 0}

    def step():
        # bf16: one fused launch per layer (swa_decode_step); fp8: append, then decode
        j = state["i"] % bank
        state["i"] += 1
        for layer, c in enumerate(caches):
            if fp8:
                c.append(ks[j], vs[j])
                c.decode(qs[j], out=outs[layer])
            else:
                c.step(ks[j], vs[j], qs[j], out=outs[layer])

    def step_two_calls():
        j = state["i"] % bank
        state["i"] += 1
        for layer, c in enumerate(caches):
            c.append(ks[j], vs[j])
            c.decode(qs[j], out=outs[layer])

    def decodes():
        j = state["i"] % bank
        state["i"] += 1
        for layer, c in enumerate(caches):
            c.decode(qs[j], out=outs[layer])

    # the step as served (append + decode per layer), then the decode kernel
    # alone, back to back, for its mean launch duration
    total_ms = timed_region(torch, pacer, step, args.steps, args.warmup)
    ms_step = total_ms / args.steps
    ms_two = None if fp8 else timed_region(torch, pacer, step_two_calls, args.steps, args.warmup) / args.steps
    avg_ms = timed_region(torch, pacer, decodes, args.steps, args.warmup) / (args.steps * layers)
    kv_bytes = 2.0 * B * Hkv * w * d * es           # one layer, full window
    launch_bytes = kv_bytes + 2.0 * B * Hq * d * 2  # + Q read, O written (bf16)
    achieved = launch_bytes / (avg_ms * 1e-3) / 1e9
    kname = "swa_decode_mfma_kernel<128,4,%s>" % ("fp8" if fp8 else "bf16")
    return {
        "w": w, "batch": B, "layers": layers,
        "kv_gbs": kv_bytes * layers * args.steps / (total_ms * 1e-3) / 1e9,
        "kernel_kv_gbs": kv_bytes / (avg_ms * 1e-3) / 1e9,
        "tok_per_s": B / (ms_step * 1e-3),
        "ms_per_step": ms_step,
        "ms_per_step_append_then_decode": ms_two,
        "kernel_ms": avg_ms,
        "cache_bytes_per_layer": 2 * B * Hkv * w * d * es,
        "roofline": {"kernel": kname, "bound": "hbm",
                     "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS,
                     "traffic": traffic(("fp8_decode_w%d" if fp8 else "decode_w%d") % w)},
    }


def bench_decode_cold(swa, torch, pacer, args, w, total_mib=512):
    """Decode launches at batch 64, 32/8 heads, d=128, a full SWA(w,4) window,
    rotating over enough layer caches that their K/V (>= total_mib MiB) exceed
    the 256 MB Infinity Cache: every launch reads its cache from HBM."""
    B, Hq, Hkv, d, s = 64, 32, 8, 128, 4
    per = 2 * B * Hkv * w * d * 2
    n = max(4, -(-total_mib * 2 ** 20 // per))
    caches = []
    for _ in range(n):
        c = swa.Cache(B, Hkv, d, w, s, dtype=torch.bfloat16)
        _fill(c, 2 * w, torch)
        caches.append(c)
    q = torch.randn((B, Hq, d), device="cuda").to(torch.bfloat16)
    o = torch.empty_like(q)
    state = {"i": 0}

    def dec():
        state["i"] += 1
        caches[state["i"] % n].decode(q, out=o)

    ms = timed_region(torch, pacer, dec, max(args.steps, 2 * n), args.warmup) / max(args.steps, 2 * n)
    launch_bytes = per + 2.0 * B * Hq * d * 2
    return {"w": w, "batch": B, "caches": n, "rotated_mib": n * per / 2 ** 20, "kernel_ms": ms,
            "kernel_kv_gbs": per / (ms * 1e-3) / 1e9,
            "hbm_frac": launch_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS}


def measure_peaks(torch):
    """Achievable HBM read bandwidth and bf16 MFMA rate on this GPU (the
    probes of libswa_peaks.so), best over a few launch shapes."""
    import ctypes
    path = os.path.join(ROOT, "sliding_window_sink_amd", "libswa_peaks.so")
    lib = ctypes.CDLL(path)
    vp, i, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    lib.swa_peak_stream_read.argtypes = [vp, sz, vp, i, i, i, vp]
    lib.swa_peak_stream_read.restype = i
    lib.swa_peak_mfma.argtypes = [vp, vp, i, i, vp]
    lib.swa_peak_mfma.restype = i
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    nbytes = 2 << 30
    buf = torch.zeros(nbytes // 4, dtype=torch.int32, device="cuda")
    sink = torch.zeros(1 << 16, dtype=torch.int32, device="cuda")

    def best_ms(launch, reps):
        for _ in range(3):
            launch()
        torch.cuda.synchronize()
        times = []
        for _ in range(3):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(reps):
                launch()
            e1.record()
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1) / reps)
        return min(times)

    hbm = {}
    for blocks in (2048, 4096, 8192):
        for unroll in (4, 8):
            for nt in (0, 1):
                def run(b=blocks, u=unroll, n=nt):
                    assert lib.swa_peak_stream_read(buf.data_ptr(), nbytes, sink.data_ptr(), b, u, n, st) == 0
                ms = best_ms(run, 5)
                hbm["b%d_u%d_nt%d" % (blocks, unroll, nt)] = nbytes / (ms * 1e-3) / 1e9
    operands = torch.zeros(1024, dtype=torch.int32, device="cuda")
    mfma = {}
    iters = 4000
    for blocks in (512, 1024, 2048):
        def runm(b=blocks):
            assert lib.swa_peak_mfma(operands.data_ptr(), sink.data_ptr(), b, iters, st) == 0
        ms = best_ms(runm, 3)
        mfma["b%d" % blocks] = blocks * 16.0 * iters * 32768 / (ms * 1e-3) / 1e12
    del buf
    torch.cuda.empty_cache()
    return {"hbm_read_gbs": max(hbm.values()), "mfma_tflops": max(mfma.values()),
            "hbm_read_frac_of_vendor": max(hbm.values()) / HBM_PEAK_GBS,
            "mfma_frac_of_vendor": max(mfma.values()) / BF16_PEAK_TFLOPS,
            "hbm_read_by_shape": hbm, "mfma_by_blocks": mfma,
            "probe": "2 GiB streaming read (16-B loads, grid-stride); four independent "
                     "v_mfma_f32_32x32x16_bf16 chains per wave"}


def _fill(cache, n, torch, chunk=4096):
    """Advance a cache to n positions with device-side rows (timing only: the
    kernels' work does not depend on the values)."""
    c = cache.c
    blk = torch.randn((c.B, min(chunk, max(n, 1)), c.Hkv, c.d), device="cuda").to(cache.compute_dtype)
    while cache.n < n:
        k = min(blk.shape[1], n - cache.n)
        cache.append(blk[:, :k].contiguous(), blk[:, :k].contiguous())


def bench_qwen(swa, torch, pacer, args, layers=36):
    """Qwen3-4B-shaped generation: 36 layers of 32/8 heads, d=128, bf16, batch
    32, SWA(576,4).  The 512-token prompt's prefill (one layer; full causal,
    512 <= 576), and one decode step at a full window: every layer appends one
    position and decodes it (72 MiB of K/V per layer, 2.5 GiB per step)."""
    import synth
    B, L, Hq, Hkv, d, w, s = 32, 512, 32, 8, 128, 576, 4
    Q, K, V = synth.prefill_inputs(B, L, Hq, Hkv, d, seed=0, workload=5, bf16=True, sink_outliers=4)
    q, k, v = (torch.from_numpy(a).to("cuda", torch.bfloat16) for a in (Q, K, V))
    out = torch.empty_like(q)
    flops, nbytes = prefill_work(B, L, Hq, Hkv, d, w)
    pre_ms = timed_region(torch, pacer, lambda: swa.prefill(q, k, v, w, s, out=out), args.steps,
                          args.warmup) / args.steps
    caches = []
    for _ in range(layers):
        c = swa.Cache(B, Hkv, d, w, s, dtype=torch.bfloat16)
        c.append(k, v)  # the prompt's rows
        _fill(c, 1024, torch)
        caches.append(c)
    qd = torch.randn((B, Hq, d), device="cuda").to(torch.bfloat16)
    kn = torch.randn((B, 1, Hkv, d), device="cuda").to(torch.bfloat16)
    outs = [torch.empty((B, Hq, d), dtype=torch.bfloat16, device="cuda") for _ in range(layers)]

    def step():  # one fused append + decode launch per layer
        for i, c in enumerate(caches):
            c.step(kn, kn, qd, out=outs[i])

    def step_two_calls():
        for i, c in enumerate(caches):
            c.append(kn, kn)
            c.decode(qd, out=outs[i])

    steps = max(4, args.steps // 5)
    step_ms = timed_region(torch, pacer, step, steps, max(2, args.warmup // 5)) / steps
    two_ms = timed_region(torch, pacer, step_two_calls, steps, max(2, args.warmup // 5)) / steps
    kv_bytes = 2.0 * B * Hkv * w * d * 2 * layers
    return {"batch": B, "layers": layers, "window": w, "sinks": s, "prompt": L,
            "prefill_layer_ms": pre_ms, "prefill_tflops": flops / (pre_ms * 1e-3) / 1e12,
            "prefill_mfma_frac": flops / (pre_ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS,
            "decode_step_ms": step_ms, "decode_tok_per_s": B / (step_ms * 1e-3),
            "decode_step_ms_append_then_decode": two_ms,
            "decode_kv_gbs": kv_bytes / (step_ms * 1e-3) / 1e9,
            "decode_hbm_frac": kv_bytes / (step_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "cache_bytes": kv_bytes}


def bench_sweep(swa, torch, pacer, args, exps=range(7, 19), Hq=32, Hkv=8, d=128, batches=(1, 16)):
    """Long-context sweep: 4 layers of Hq/Hkv heads of dimension d (default
    32/8, d=128), bf16, at each batch in `batches`, context n = 2^k for k in
    exps (default 7..18) for SWA(64,4), SWA(512,4) and full causal (capacity
    2^18 + the timed steps).  At each n: fill untimed, then time 128 steps
    (append + decode in every layer)."""
    s, layers, steps = 4, 4, 128
    rows = []
    for B in batches:
        for name, w in (("swa64", 64), ("swa512", 512), ("full", 2 ** 18 + steps + 16)):
            caches = [swa.Cache(B, Hkv, d, w, s, dtype=torch.bfloat16) for _ in range(layers)]
            qd = torch.randn((B, Hq, d), device="cuda").to(torch.bfloat16)
            kn = torch.randn((B, 1, Hkv, d), device="cuda").to(torch.bfloat16)
            outs = [torch.empty((B, Hq, d), dtype=torch.bfloat16, device="cuda") for _ in range(layers)]

            def step():  # one fused append + decode launch per layer
                for i, c in enumerate(caches):
                    c.step(kn, kn, qd, out=outs[i])

            def warm():  # the decode alone: the untimed calls leave n where _fill put it
                for i, c in enumerate(caches):
                    c.decode(qd, out=outs[i])

            for k in exps:
                n = 2 ** k
                for c in caches:
                    _fill(c, n, torch)
                ms = timed_region(torch, pacer, step, steps, 0, warm=warm)
                held = min(n + steps // 2, w)
                kv = 2.0 * B * Hkv * held * d * 2 * layers
                rows.append({"batch": B, "attention": name, "n": n, "tok_per_s": B * steps / (ms * 1e-3),
                             "ms_per_step": ms / steps, "kv_gbs": kv / (ms / steps * 1e-3) / 1e9,
                             "cache_bytes": 2 * B * Hkv * min(w, n + steps) * d * 2 * layers})
                print("sweep %d/%d d=%d B=%d %s n=%d: %.0f tok/s, %.0f GB/s" % (
                    Hq, Hkv, d, B, name, n, rows[-1]["tok_per_s"], rows[-1]["kv_gbs"]), file=sys.stderr, flush=True)
            del caches
            torch.cuda.empty_cache()
    return rows


def bench_graph_steps(swa, torch, pacer, args, exps=(7, 12, 18), Hq=32, Hkv=8, d=128, B=1):
    """The batch-1 generation step of bench_sweep (4 layers, one fused append +
    decode launch per layer) captured once in a HIP graph at context n and
    replayed 128 times.  Each replay appends position n+1 again and decodes at
    it: the per-step work of a serving loop that captures its step.  At batch 1
    the launches are short enough that the per-launch overhead of a stream
    launch is a large part of the step; the graph removes most of it."""
    s, layers, reps = 4, 4, 128
    rows = []
    for name, w in (("swa64", 64), ("swa512", 512), ("full", 2 ** 18 + 16)):
        caches = [swa.Cache(B, Hkv, d, w, s, dtype=torch.bfloat16) for _ in range(layers)]
        qd = torch.randn((B, Hq, d), device="cuda").to(torch.bfloat16)
        kn = torch.randn((B, 1, Hkv, d), device="cuda").to(torch.bfloat16)
        outs = [torch.empty((B, Hq, d), dtype=torch.bfloat16, device="cuda") for _ in range(layers)]
        for k in exps:
            n = 2 ** k
            for c in caches:
                _fill(c, n, torch)
            for i, c in enumerate(caches):  # one eager step sizes any workspace; then rewind
                c.step(kn, kn, qd, out=outs[i])
                c.n = n
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            side = torch.cuda.Stream()
            with torch.cuda.stream(side):
                with torch.cuda.graph(g, stream=side):
                    for i, c in enumerate(caches):
                        c.step(kn, kn, qd, out=outs[i])
            for c in caches:
                c.n = n
            torch.cuda.synchronize()
            ms = timed_region(torch, pacer, g.replay, reps, 0)
            rows.append({"batch": B, "attention": name, "n": n, "tok_per_s": B * reps / (ms * 1e-3),
                         "ms_per_step": ms / reps})
            print("graph step %d/%d d=%d B=%d %s n=%d: %.0f tok/s" % (Hq, Hkv, d, B, name, n, rows[-1]["tok_per_s"]),
                  file=sys.stderr, flush=True)
            del g
        del caches
        torch.cuda.empty_cache()
    return rows


def bench_chunk(swa, torch, pacer, args):
    """Chunked prefill and multi-query decode against a full cache (32/8 heads,
    d=128, bf16, SWA(512,4)): a 512-position chunk at batch 1 and 16 behind
    n = 4096 cached positions (every row attends 512 keys: the cache ring and
    the chunk), and 4 draft positions verified at once at batch 64 and at
    batch 1 behind n = 32768.  One step = one swa_prefill_chunk call on a copy of the cache state (the cache is
    reset to n before each call, outside the timed kernel's work)."""
    Hq, Hkv, d, w, s = 32, 8, 128, 512, 4
    out = {}
    for B, C, n in ((1, 512, 4096), (16, 512, 4096), (64, 4, 32768), (1, 4, 32768)):
        c = swa.Cache(B, Hkv, d, w, s, dtype=torch.bfloat16)
        _fill(c, n, torch)
        q = torch.randn((B, C, Hq, d), device="cuda").to(torch.bfloat16)
        kv = torch.randn((B, C, Hkv, d), device="cuda").to(torch.bfloat16)
        o = torch.empty_like(q)

        def step():
            c.n = n  # the call appends; rewind so every step sees the same state
            c.prefill_chunk(q, kv, kv, out=o)

        ms = timed_region(torch, pacer, step, args.steps, args.warmup) / args.steps
        pairs = sum(min(n + i, w) for i in range(1, C + 1))
        flops = 4.0 * d * Hq * B * pairs
        kv_bytes = 2.0 * B * Hkv * (min(n, w) + C) * d * 2
        out["B%d_C%d" % (B, C)] = {"batch": B, "chunk": C, "cached": n, "window": w, "ms_per_call": ms,
                                   "tflops": flops / (ms * 1e-3) / 1e12,
                                   "kv_gbs": kv_bytes / (ms * 1e-3) / 1e9,
                                   "note": "call = attention over cache + chunk and the chunk's append (one "
                                           "launch for short chunks, the multi-query decode; two otherwise)"}
        print("chunk B=%d C=%d: %.3f ms, %.1f TFLOP/s, %.0f GB/s of K/V" % (
            B, C, ms, out["B%d_C%d" % (B, C)]["tflops"], out["B%d_C%d" % (B, C)]["kv_gbs"]),
            file=sys.stderr, flush=True)
    return out


def bench_tiny(swa, torch, pacer, args):
    """The small fp32 parity configuration, timed for information: B=1, one
    head (G=1), d=64, L=256, SWA(64,4), fp32 in and out.  A launch this small
    is bound by the launch and one workgroup's latency, not by a roofline."""
    import synth
    B, L, Hq, Hkv, d, w, s = 1, 256, 1, 1, 64, 64, 4
    Q, K, V = synth.prefill_inputs(B, L, Hq, Hkv, d, seed=0, workload=1, bf16=False)
    q, k, v = (torch.from_numpy(a).to("cuda") for a in (Q, K, V))
    out = torch.empty_like(q)
    flops, nbytes = prefill_work(B, L, Hq, Hkv, d, w, es=4)
    ms = timed_region(torch, pacer, lambda: swa.prefill(q, k, v, w, s, out=out), args.steps, args.warmup) / args.steps
    return {"shape": {"batch": B, "seq_len": L, "q_heads": Hq, "kv_heads": Hkv, "head_dim": d, "window": w,
                      "sinks": s, "dtype": "f32"},
            "ms_per_call": ms, "mflop_per_call": flops / 1e6, "kib_per_call": nbytes / 1024,
            "note": "launch- and latency-bound; for information"}


def bench_lsink(swa, torch, pacer, args):
    """The learned-sink variant on the headline shapes: the 8B-shaped prefill
    at SWA(512,4) and one batch-64 decode at a full SWA(512,4) window, each
    with one synthetic logit per query head."""
    import synth
    B, L, Hq, Hkv, d, w, s = 1, 4096, 32, 8, 128, 512, 4
    Q, K, V = synth.prefill_inputs(B, L, Hq, Hkv, d, seed=0, workload=2, bf16=True, sink_outliers=4)
    q, k, v = (torch.from_numpy(a).to("cuda", torch.bfloat16) for a in (Q, K, V))
    out = torch.empty_like(q)
    logit = torch.linspace(-2.0, 12.0, Hq, device="cuda", dtype=torch.float32)
    flops, _ = prefill_work(B, L, Hq, Hkv, d, w)
    pre_ms = timed_region(torch, pacer, lambda: swa.prefill(q, k, v, w, s, out=out, sink_logit=logit),
                          args.steps, args.warmup) / args.steps
    Bd = 64
    caches = []
    for _ in range(4):
        c = swa.Cache(Bd, Hkv, d, w, s, dtype=torch.bfloat16)
        _fill(c, 2 * w, torch)
        caches.append(c)
    qd = torch.randn((Bd, Hq, d), device="cuda").to(torch.bfloat16)
    od = torch.empty_like(qd)
    state = {"i": 0}

    def dec():
        state["i"] += 1
        caches[state["i"] % 4].decode(qd, out=od, sink_logit=logit)

    dec_ms = timed_region(torch, pacer, dec, args.steps, args.warmup) / args.steps
    kv = 2.0 * Bd * Hkv * w * d * 2
    return {"prefill_tflops": flops / (pre_ms * 1e-3) / 1e12, "prefill_ms": pre_ms,
            "decode_ms": dec_ms, "decode_kv_gbs": kv / (dec_ms * 1e-3) / 1e9}


def bench_serving(swa, torch, pacer, args, layers=4):
    """Ragged and paged batches on the 8B shapes (32/8 heads, d=128, bf16,
    SWA(512,4)): batch-64 decode from paged caches (pages of 64 slots,
    shuffled block tables), first with every sequence at a full window (the
    dense decode's workload, for the paging overhead), then with ragged
    positions n_b uniform in [1, 1024]; a varlen prefill of 8 prompts
    with lengths uniform in [256, 1024]; and a chunked prefill over paged
    caches (8 sequences at ragged positions, chunks of 128 .. 512 rows)."""
    B, Hq, Hkv, d, w, s, page = 64, 32, 8, 128, 512, 4, 64
    pps = w // page
    gen = torch.Generator(device="cpu").manual_seed(7)
    out = {"batch": B, "window": w, "page": page, "layers": layers}
    for mode in ("full", "ragged"):
        if mode == "full":
            n_b = torch.full((B,), 2 * w, dtype=torch.int64)
        else:
            n_b = torch.randint(1, 2 * w + 1, (B,), generator=gen, dtype=torch.int64)
        caches = []
        for _ in range(layers):
            table = torch.randperm(B * pps, generator=gen).to(torch.int32).reshape(B, pps).cuda()
            c = swa.PagedCache(B, Hkv, d, w, s, page, B * pps, block_table=table)
            cu = torch.cat([torch.zeros(1, dtype=torch.int64), torch.cumsum(n_b, 0)]).to(torch.int32).cuda()
            rows = torch.randn((int(n_b.sum()), Hkv, d), device="cuda").to(torch.bfloat16)
            c.append(rows, rows, cu)
            caches.append(c)
        q = torch.randn((B, Hq, d), device="cuda").to(torch.bfloat16)
        o = torch.empty_like(q)
        state = {"i": 0}

        def dec():
            state["i"] += 1
            caches[state["i"] % layers].decode(q, out=o)

        ms = timed_region(torch, pacer, dec, args.steps, args.warmup) / args.steps
        attended = int(torch.clamp(n_b, max=w).sum())
        kv = 2.0 * attended * Hkv * d * 2
        out["decode_" + mode] = {"kernel_ms": ms, "kv_gbs": kv / (ms * 1e-3) / 1e9,
                                 "mean_attended": attended / B}
        del caches
    lens = torch.randint(256, 1025, (8,), generator=gen, dtype=torch.int64)
    total = int(lens.sum())
    cu = torch.cat([torch.zeros(1, dtype=torch.int64), torch.cumsum(lens, 0)]).to(torch.int32).cuda()
    qv = torch.randn((total, Hq, d), device="cuda").to(torch.bfloat16)
    kv_ = torch.randn((total, Hkv, d), device="cuda").to(torch.bfloat16)
    ov = torch.empty_like(qv)
    mx = int(lens.max())
    ms = timed_region(torch, pacer, lambda: swa.prefill_varlen(qv, kv_, kv_, cu, mx, w, s, out=ov),
                      args.steps, args.warmup) / args.steps
    flops = sum(prefill_work(1, int(n), Hq, Hkv, d, w)[0] for n in lens)
    out["prefill_varlen"] = {"prompts": [int(n) for n in lens], "kernel_ms": ms,
                             "tflops": flops / (ms * 1e-3) / 1e12}
    # chunked prefill over paged caches: 8 sequences at ragged positions
    # (0 .. 2048 cached), each with a chunk of 128 .. 512 new rows
    Bc = 8
    hist = torch.randint(0, 2049, (Bc,), generator=gen, dtype=torch.int64)
    chunks = torch.randint(128, 513, (Bc,), generator=gen, dtype=torch.int64)
    table = torch.randperm(Bc * pps, generator=gen).to(torch.int32).reshape(Bc, pps).cuda()
    pc = swa.PagedCache(Bc, Hkv, d, w, s, page, Bc * pps, block_table=table)
    cu_h = torch.cat([torch.zeros(1, dtype=torch.int64), torch.cumsum(hist, 0)]).to(torch.int32).cuda()
    rows = torch.randn((max(int(hist.sum()), 1), Hkv, d), device="cuda").to(torch.bfloat16)
    pc.append(rows[:int(hist.sum())], rows[:int(hist.sum())], cu_h)
    n0 = pc.n.clone()
    total_c = int(chunks.sum())
    cu_c = torch.cat([torch.zeros(1, dtype=torch.int64), torch.cumsum(chunks, 0)]).to(torch.int32).cuda()
    qc = torch.randn((total_c, Hq, d), device="cuda").to(torch.bfloat16)
    kc = torch.randn((total_c, Hkv, d), device="cuda").to(torch.bfloat16)
    oc = torch.empty_like(qc)
    mxc = int(chunks.max())

    def chunk_step():
        pc.n.copy_(n0)  # every call sees the same positions
        pc.prefill_chunk(qc, kc, kc, cu_c, mxc, out=oc)

    ms = timed_region(torch, pacer, chunk_step, args.steps, args.warmup) / args.steps
    flops = sum(4.0 * d * Hq * sum(min(int(h) + i, w) for i in range(1, int(c) + 1)) for h, c in zip(hist, chunks))
    out["prefill_chunk_paged"] = {"cached": [int(h) for h in hist], "chunks": [int(c) for c in chunks],
                                  "ms_per_call": ms, "tflops": flops / (ms * 1e-3) / 1e12,
                                  "note": "call = position reset (one device copy), attention over pages + "
                                          "chunk, then the chunks' paged append"}
    return out


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(prefill_inputs, min_seconds=8.0):
    """The fp64 oracle on the host cores: the headline prefill repeated for
    about min_seconds (the line's value), then one call each of a streaming
    decode step (batch 64, full SWA(64,4) and SWA(512,4) windows), a
    long-context decode (batch 1, full causal at n = 2^12 and 2^18, one layer
    timed, x4 for the 4-layer step) and the Qwen3-4B-shaped layer (batch-32
    512-token prompt, one decode step at a full SWA(576,4) window; x36 for
    the model, labelled extrapolated)."""
    import oracle
    import synth
    Q, K, V, w, s, flops = prefill_inputs
    threads = oracle.default_threads()
    reps, t_total = 0, 0.0
    while t_total < min_seconds and reps < 200:
        t = time.perf_counter()
        oracle.prefill(Q, K, V, w, s, threads=threads)
        t_total += time.perf_counter() - t
        reps += 1
    out = {"value": flops * reps / t_total / 1e12, "unit": "TFLOP/s", "cores": threads,
           "kind": "oracle", "cpu_model": cpu_model(),
           "sample": "the full prefill step (B=1, L=4096, 32/8 heads, d=128, SWA(%d,4)) in fp64, "
                     "%d repetition(s), %.1f s" % (w, reps, t_total)}
    others = {}

    def timed(fn):
        t = time.perf_counter()
        fn()
        return time.perf_counter() - t

    Hq, Hkv, d = 32, 8, 128
    for ww in (64, 512):  # streaming decode, batch 64, one full-window step
        B = 64
        Kh, Vh = synth.history_rows(B, Hkv, d, ww, workload=3)
        q = synth.query_rows(B, Hq, d, ww)
        sec = timed(lambda: oracle.decode(q, np.arange(1, ww + 1), Kh, Vh, ww, ww, 4, threads=threads))
        kv = 2.0 * B * Hkv * ww * d * 2
        others["decode_b64_w%d" % ww] = {"seconds": sec, "kv_gbs": kv / sec / 1e9,
                                         "sample": "one decode step, batch 64, full SWA(%d,4) window" % ww}
    for k in (12, 18):  # long-context decode, batch 1, full causal
        n = 2 ** k
        Kh, Vh = synth.history_rows(1, Hkv, d, n, workload=4)
        q = synth.query_rows(1, Hq, d, n, workload=4)
        sec = timed(lambda: oracle.decode(q, np.arange(1, n + 1), Kh, Vh, n, 2 ** 18 + 272, 4, threads=threads))
        others["sweep_b1_full_n%d" % n] = {"seconds_per_layer": sec, "tok_per_s_4_layers": 1.0 / (4 * sec),
                                           "sample": "one full-causal decode step at n = 2^%d, batch 1; "
                                                     "4-layer figure = 4 x the one layer timed" % k}
        del Kh, Vh
    Bq, Lq, wq = 32, 512, 576  # Qwen3-4B-shaped layer
    Qq, Kq, Vq = synth.prefill_inputs(Bq, Lq, Hq, Hkv, d, seed=0, workload=5, bf16=True, sink_outliers=4)
    sec_p = timed(lambda: oracle.prefill(Qq, Kq, Vq, wq, 4, threads=threads))
    pflops = 4.0 * d * Hq * Bq * pairs(Lq, wq)
    Kh, Vh = synth.history_rows(Bq, Hkv, d, wq, workload=5)
    q = synth.query_rows(Bq, Hq, d, wq, workload=5)
    sec_d = timed(lambda: oracle.decode(q, np.arange(1, wq + 1), Kh, Vh, wq, wq, 4, threads=threads))
    others["qwen3_4b"] = {"prefill_layer_seconds": sec_p, "prefill_tflops": pflops / sec_p / 1e12,
                          "decode_layer_seconds": sec_d,
                          "decode_step_36_layers_seconds_extrapolated": 36 * sec_d,
                          "prefill_36_layers_seconds_extrapolated": 36 * sec_p,
                          "sample": "one layer timed (batch 32: 512-token prompt; one decode step at a full "
                                    "SWA(576,4) window), x36 labelled extrapolated"}
    out["others"] = others
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--w", type=int, default=512, choices=[128, 256, 512])
    ap.add_argument("--decode-windows", default="512,64")
    ap.add_argument("--windows", default="128,256,512",
                    help="prefill windows measured (the headline --w is always among them)")
    ap.add_argument("--no-cold", action="store_true",
                    help="profile helper: skip the cold (rotated-input) prefill and decode runs")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle timing")
    ap.add_argument("--only-8b", action="store_true",
                    help="profile helper: the 8B-shaped prefill and decode legs without the Qwen3-4B leg")
    ap.add_argument("--sweep", action="store_true",
                    help="run only the long-context decode sweep and print its JSON line")
    ap.add_argument("--only", choices=["peaks", "prefill", "decode", "qwen", "chunk", "tiny", "lsink", "fp8", "serving",
                                       "context"],
                    default=None,
                    help="profile helper: run one leg only")
    ap.add_argument("--copy-probe", action="store_true",
                    help="also run a plain 256 MiB device-to-device copy 5 times (a kernel of known "
                         "traffic against which the FETCH_SIZE / WRITE_SIZE counters are scaled)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: libswa has no multi-GPU path (its kernels work on one GPU's "
              "share of heads or sequences); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    import sliding_window_sink_amd as swa
    if not torch.cuda.is_available():
        print("bench.py needs a ROCm GPU", file=sys.stderr)
        sys.exit(2)
    torch.cuda.set_device(0)

    if args.copy_probe:
        src = torch.empty(128 << 20, dtype=torch.bfloat16, device="cuda").fill_(1.0)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print("copy probe: 5 x 256 MiB read + 256 MiB written", file=sys.stderr, flush=True)
        del src, dst
    pacer = Pacer(torch)
    if args.sweep:
        print(json.dumps({"metric": "long-context decode tok/s (4 layers, bf16)",
                          "unit": "tok/s", "n_gpus": 1, "data": "synthetic",
                          "sweep": bench_sweep(swa, torch, pacer, args),
                          "sweep_pages_model": bench_sweep(swa, torch, pacer, args, Hq=16, Hkv=16, d=64,
                                                           batches=(1,)),
                          "pages_model": PAGES_MODEL}), flush=True)
        return
    peaks = None
    if args.only in (None, "peaks"):
        peaks = measure_peaks(torch)
        print("peaks: HBM read %.0f GB/s, bf16 MFMA %.0f TFLOP/s" % (peaks["hbm_read_gbs"], peaks["mfma_tflops"]),
              file=sys.stderr, flush=True)
    pre, pre_inputs = (None, None)
    prefill_windows, prefill_cold = {}, {}
    if args.only in (None, "prefill"):
        # every window of the 8B-shaped prefill, warm; the headline window last
        # (its inputs feed the oracle timing); then cold runs of w = 512 and 128
        wins = [int(x) for x in args.windows.split(",") if x]
        for w in [x for x in wins if x != args.w] + [args.w]:
            r, inputs = bench_prefill(swa, torch, pacer, args, w, peaks=peaks)
            prefill_windows["w%d" % w] = {k: v for k, v in r.items() if k != "roofline"}
            print("prefill w=%d: %.1f TFLOP/s, kernel %.4f ms, %.0f%% of attainable" % (
                w, r["tflops"], r["kernel_ms"], 100 * r["attainable_frac"]), file=sys.stderr, flush=True)
            if w == args.w:
                pre, pre_inputs = r, inputs
        if args.only is None and not args.no_cold:
            for w in (512, 128):
                r, _ = bench_prefill(swa, torch, pacer, args, w, cold=True, peaks=peaks)
                prefill_cold["w%d" % w] = {k: v for k, v in r.items() if k != "roofline"}
                print("prefill cold w=%d: %.1f TFLOP/s, kernel %.4f ms" % (w, r["tflops"], r["kernel_ms"]),
                      file=sys.stderr, flush=True)
    dec = {}
    if args.only in (None, "decode"):
        for w in (int(x) for x in args.decode_windows.split(",") if x):
            dec["w%d" % w] = bench_decode(swa, torch, pacer, args, w)
            print("decode w=%d: %.0f GB/s, kernel %.4f ms" % (w, dec["w%d" % w]["kernel_kv_gbs"],
                                                              dec["w%d" % w]["kernel_ms"]),
                  file=sys.stderr, flush=True)
        if not args.no_cold:
            dec["w64_cold"] = bench_decode_cold(swa, torch, pacer, args, 64)
        if "w64_cold" in dec:
            print("decode cold w=64: %.0f GB/s, kernel %.4f ms over %d caches" % (
                dec["w64_cold"]["kernel_kv_gbs"], dec["w64_cold"]["kernel_ms"], dec["w64_cold"]["caches"]),
                file=sys.stderr, flush=True)
    qwen = None
    if args.only in (None, "qwen") and not args.only_8b:
        qwen = bench_qwen(swa, torch, pacer, args)
        print("qwen3-4b shape: prefill %.1f TFLOP/s; decode step %.3f ms, %.0f tok/s, %.0f GB/s" % (
            qwen["prefill_tflops"], qwen["decode_step_ms"], qwen["decode_tok_per_s"], qwen["decode_kv_gbs"]),
            file=sys.stderr, flush=True)
    chunk = None
    if args.only in (None, "chunk") and not args.only_8b:
        chunk = bench_chunk(swa, torch, pacer, args)
    tiny = None
    if args.only in (None, "tiny") and not args.only_8b:
        tiny = bench_tiny(swa, torch, pacer, args)
        print("tiny fp32 prefill (B=1, 1 head, d=64, L=256, SWA(64,4)): %.4f ms per call" % tiny["ms_per_call"],
              file=sys.stderr, flush=True)
    lsink = None
    if args.only in (None, "lsink") and not args.only_8b:
        lsink = bench_lsink(swa, torch, pacer, args)
        print("learned sink: prefill %.1f TFLOP/s; decode w=512 %.0f GB/s" % (
            lsink["prefill_tflops"], lsink["decode_kv_gbs"]), file=sys.stderr, flush=True)
    fp8 = {}
    if args.only in (None, "fp8") and not args.only_8b:
        for w in (int(x) for x in args.decode_windows.split(",") if x):
            # 8 layers: 512 MiB of codes at w = 512, past the 256 MB Infinity Cache
            fp8["w%d" % w] = bench_decode(swa, torch, pacer, args, w, layers=8, fp8=True)
            print("fp8 decode w=%d: %.0f GB/s, kernel %.4f ms" % (w, fp8["w%d" % w]["kernel_kv_gbs"],
                                                                  fp8["w%d" % w]["kernel_ms"]),
                  file=sys.stderr, flush=True)
    serving = None
    if args.only in (None, "serving") and not args.only_8b:
        serving = bench_serving(swa, torch, pacer, args)
        print("serving: paged decode full %.4f ms (%.0f GB/s), ragged %.4f ms (%.0f GB/s); varlen prefill "
              "%.1f TFLOP/s" % (serving["decode_full"]["kernel_ms"], serving["decode_full"]["kv_gbs"],
                                serving["decode_ragged"]["kernel_ms"], serving["decode_ragged"]["kv_gbs"],
                                serving["prefill_varlen"]["tflops"]), file=sys.stderr, flush=True)
        print("serving: paged chunked prefill %.4f ms, %.1f TFLOP/s" % (
            serving["prefill_chunk_paged"]["ms_per_call"], serving["prefill_chunk_paged"]["tflops"]),
            file=sys.stderr, flush=True)
    context = None
    if args.only in (None, "context") and not args.only_8b:
        rows = bench_sweep(swa, torch, pacer, args, exps=(7, 12, 18))
        pages_rows = bench_sweep(swa, torch, pacer, args, exps=(7, 12, 18), Hq=16, Hkv=16, d=64, batches=(1,))
        graph_rows = bench_graph_steps(swa, torch, pacer, args)
        context = {"layers": 4, "q_heads": 32, "kv_heads": 8, "head_dim": 128, "steps_timed": 128,
                   "rows": rows,
                   "pages_model": {"shape": PAGES_MODEL, "rows": pages_rows},
                   "graph_b1": {"rows": graph_rows,
                                "note": "the same 4-layer batch-1 step captured in a HIP graph at position n+1 "
                                        "and replayed (rows above: stream launches)"},
                   "note": "n = 2^7, 2^12, 2^18 of the full sweep (bench.py --sweep runs every power of two)"}
    if args.only is not None:
        return

    line = {
        "metric": METRIC,
        "value": pre["tflops"],
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": pre["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "Llama-3.1-8B-shaped SWA prefill", "batch": 1, "seq_len": 4096,
                   "q_heads": 32, "kv_heads": 8, "head_dim": 128, "window": args.w, "sinks": 4,
                   "sink_outliers": True},
        "roofline": pre["roofline"],
        "prefill": {k: v for k, v in pre.items() if k != "roofline"},
        "prefill_windows": prefill_windows,
        "prefill_cold": prefill_cold,
        "measured_peaks": peaks,
        "decode": dec,
        "context_sweep": context,
        "qwen3_4b": qwen,
        "chunk": chunk,
        "learned_sink": lsink,
        "tiny_prefill": tiny,
        "fp8_kv_decode": fp8,
        "serving": serving,
    }
    if not args.no_cpu:
        line["cpu_baseline"] = cpu_baseline(pre_inputs)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
