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


def pairs(L, w):
    """Attended (query, key) pairs of one head over a prompt of L tokens."""
    return sum(min(t, w) for t in range(1, L + 1))


def prefill_work(B, L, Hq, Hkv, d, w, es=2):
    flops = 4.0 * d * Hq * B * pairs(L, w)
    nbytes = es * (2 * B * L * Hq * d + 2 * B * L * Hkv * d)  # Q, O, K, V once
    return flops, nbytes


def timed_launches(fn, steps, warmup, torch):
    """Run fn() warmup+steps times; returns (avg launch ms from per-launch HIP
    events, total ms of the timed region)."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)]
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for a, b in evs:
        a.record()
        fn()
        b.record()
    t1.record()
    torch.cuda.synchronize()
    per = [a.elapsed_time(b) for a, b in evs]
    return float(np.mean(per)), t0.elapsed_time(t1), per


def bench_prefill(swa, torch, args):
    import synth
    B, L, Hq, Hkv, d, w, s = 1, 4096, 32, 8, 128, args.w, 4
    Q, K, V = synth.prefill_inputs(B, L, Hq, Hkv, d, seed=0, workload=2, bf16=True, sink_outliers=4)
    q, k, v = (torch.from_numpy(a).to("cuda", torch.bfloat16) for a in (Q, K, V))
    out = torch.empty_like(q)
    flops, nbytes = prefill_work(B, L, Hq, Hkv, d, w)
    avg_ms, total_ms, _ = timed_launches(lambda: swa.prefill(q, k, v, w, s, out=out), args.steps,
                                         args.warmup, torch)
    ms_step = total_ms / args.steps
    ai = flops / nbytes
    bound = "mfma" if ai >= RIDGE else "hbm"
    if bound == "mfma":
        achieved, peak, unit = flops / (avg_ms * 1e-3) / 1e12, BF16_PEAK_TFLOPS, "TFLOP/s"
    else:
        achieved, peak, unit = nbytes / (avg_ms * 1e-3) / 1e9, HBM_PEAK_GBS, "GB/s"
    res = {
        "tflops": flops / (ms_step * 1e-3) / 1e12,
        "ms_per_step": ms_step,
        "kernel_ms": avg_ms,
        "flops_per_step": flops,
        "bytes_per_step": nbytes,
        "arith_intensity": ai,
        "roofline": {"kernel": "swa_prefill_kernel<bf16,128,4>", "bound": bound,
                     "achieved": achieved, "peak": peak, "unit": unit,
                     "frac": achieved / peak, "traffic": None,
                     "mfma_frac": flops / (avg_ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS},
    }
    return res, (Q, K, V, w, s, flops)


def bench_decode(swa, torch, args, w, layers=4):
    import synth
    B, Hq, Hkv, d, s = 64, 32, 8, 128, 4
    caches = []
    for layer in range(layers):
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
    dec_events = []

    def step(record=False):
        j = state["i"] % bank
        state["i"] += 1
        for layer, c in enumerate(caches):
            c.append(ks[j], vs[j])
            if record:
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record()
                c.decode(qs[j], out=outs[layer])
                b.record()
                dec_events.append((a, b))
            else:
                c.decode(qs[j], out=outs[layer])

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(args.steps):
        step(record=True)
    t1.record()
    torch.cuda.synchronize()
    per = [a.elapsed_time(b) for a, b in dec_events]
    avg_ms = float(np.mean(per))
    ms_step = t0.elapsed_time(t1) / args.steps
    kv_bytes = 2.0 * B * Hkv * w * d * 2            # one layer, full window
    launch_bytes = kv_bytes + 2.0 * B * Hq * d * 2  # + Q read, O written
    achieved = launch_bytes / (avg_ms * 1e-3) / 1e9
    return {
        "w": w, "batch": B, "layers": layers,
        "kv_gbs": kv_bytes * layers * args.steps / (t0.elapsed_time(t1) * 1e-3) / 1e9,
        "kernel_kv_gbs": kv_bytes / (avg_ms * 1e-3) / 1e9,
        "tok_per_s": B / (ms_step * 1e-3),
        "ms_per_step": ms_step,
        "kernel_ms": avg_ms,
        "cache_bytes_per_layer": 2 * B * Hkv * w * d * 2,
        "roofline": {"kernel": "swa_decode_kernel<bf16,128,4>", "bound": "hbm",
                     "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": None},
    }


def cpu_baseline(prefill_inputs, min_seconds=10.0):
    import oracle
    Q, K, V, w, s, flops = prefill_inputs
    threads = oracle.default_threads()
    reps, t_total = 0, 0.0
    while t_total < min_seconds and reps < 20:
        t = time.perf_counter()
        oracle.prefill(Q, K, V, w, s, threads=threads)
        t_total += time.perf_counter() - t
        reps += 1
    return {"value": flops * reps / t_total / 1e12, "unit": "TFLOP/s", "cores": threads,
            "kind": "oracle",
            "sample": "the full prefill step (B=1, L=4096, 32/8 heads, d=128, SWA(%d,4)) in fp64, "
                      "%d repetition(s), %.1f s" % (w, reps, t_total)}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--w", type=int, default=512, choices=[128, 256, 512])
    ap.add_argument("--decode-windows", default="512,64")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle timing")
    ap.add_argument("--only", choices=["prefill", "decode"], default=None,
                    help="profile helper: run one leg only")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (see DESIGN.md, "
              "'How it would shard'); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    import sliding_window_sink_amd as swa
    if not torch.cuda.is_available():
        print("bench.py needs a ROCm GPU", file=sys.stderr)
        sys.exit(2)
    torch.cuda.set_device(0)

    pre, pre_inputs = (None, None)
    if args.only != "decode":
        pre, pre_inputs = bench_prefill(swa, torch, args)
        print("prefill: %.1f TFLOP/s, kernel %.3f ms" % (pre["tflops"], pre["kernel_ms"]),
              file=sys.stderr, flush=True)
    dec = {}
    if args.only != "prefill":
        for w in (int(x) for x in args.decode_windows.split(",") if x):
            dec["w%d" % w] = bench_decode(swa, torch, args, w)
            print("decode w=%d: %.0f GB/s, kernel %.4f ms" % (w, dec["w%d" % w]["kernel_kv_gbs"],
                                                              dec["w%d" % w]["kernel_ms"]),
                  file=sys.stderr, flush=True)
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
        "decode": dec,
    }
    if not args.no_cpu:
        line["cpu_baseline"] = cpu_baseline(pre_inputs)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
