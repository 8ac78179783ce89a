"""GPU parity: the HIP path through the C ABI against the fp64 oracle.

Tolerances (written here, applied per output tensor):
  fp32 path : max|gpu - oracle| / max|oracle| <= 1e-5
  bf16 path : max|gpu - oracle| <= 2e-2 (gpu output is bf16, oracle fp64)
Attended sets and cache slot maps are compared bit-exactly (one-hot probe,
cache read-back against the oracle's ring simulation).
"""
import numpy as np
import pytest
import torch

import oracle
from oracle import brute
import synth

pytestmark = pytest.mark.gpu

F32_REL = 1e-5
BF16_ABS = 2e-2


@pytest.fixture(scope="module")
def swa():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    import sliding_window_sink_amd as swa
    return swa


def dev(x, dtype):
    return torch.from_numpy(np.ascontiguousarray(x)).to(device="cuda", dtype=dtype)


def host(t):
    return t.float().cpu().numpy().astype(np.float64)


def check(got, ref, dtype, what=""):
    err = np.max(np.abs(got - ref)) if got.size else 0.0
    if dtype == torch.float32:
        scale = max(np.max(np.abs(ref)), 1e-30) if ref.size else 1.0
        assert err / scale <= F32_REL, "%s: rel err %.3g" % (what, err / scale)
    else:
        assert err <= BF16_ABS, "%s: abs err %.3g" % (what, err)
    return err


# --- prefill -----------------------------------------------------------------

def test_prefill_tiny_fp32(swa):
    """B=1, one head, d=64, L=256, SWA(64,4), fp32 N(0,1)."""
    Q, K, V = synth.prefill_inputs(1, 256, 1, 1, 64, seed=0, workload=1, bf16=False)
    O = host(swa.prefill(dev(Q, torch.float32), dev(K, torch.float32), dev(V, torch.float32), 64, 4))
    check(O, oracle.prefill(Q, K, V, 64, 4), torch.float32, "oracle")
    check(O, brute.prefill(Q, K, V, 64, 4), torch.float32, "brute force")


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("w,s", [(64, 4), (16, 0), (40, 33)])
def test_prefill_attended_sets_exact(swa, dtype, w, s):
    """Zero queries + one-hot values: O[t, c] = 1/|S_t| exactly when position
    block+c+1 is in S_t, else exactly 0.  Four blocks cover L = 256 at d = 64."""
    L, d = 256, 64
    for block in range(0, L, d):
        Q, K, V = synth.one_hot_probe(1, L, 4, 1, d, block)
        O = host(swa.prefill(dev(Q, dtype), dev(K, dtype), dev(V, dtype), w, s))
        want = np.zeros((L, d))
        for t in range(1, L + 1):
            S = oracle.attended(w, s, t)
            val = float(torch.tensor(1.0 / len(S), dtype=torch.float64).to(dtype).double())
            for i in S:
                if block < i <= block + d:
                    want[t - 1, i - 1 - block] = val
        for h in range(4):
            np.testing.assert_array_equal(O[0, :, h, :], want)


@pytest.mark.parametrize("w", [128, 256, 512])
def test_prefill_8b_shape(swa, w):
    """B=1, 32/8 heads, d=128, L=4096, bf16, SWA(w,4), first 4 keys with the
    shared outlier direction."""
    Q, K, V = synth.prefill_inputs(1, 4096, 32, 8, 128, seed=0, workload=2, bf16=True,
                                   sink_outliers=4)
    O = host(swa.prefill(dev(Q, torch.bfloat16), dev(K, torch.bfloat16), dev(V, torch.bfloat16), w, 4))
    check(O, oracle.prefill(Q, K, V, w, 4), torch.bfloat16, "w=%d" % w)


EDGE = [  # B, L, Hq, Hkv, d, w, s, dtype
    (1, 1, 4, 1, 128, 64, 4, torch.bfloat16),
    (2, 17, 4, 1, 128, 8, 4, torch.bfloat16),
    (1, 1000, 32, 8, 128, 128, 4, torch.bfloat16),
    (2, 300, 8, 8, 64, 64, 4, torch.bfloat16),
    (1, 333, 16, 8, 128, 100, 0, torch.bfloat16),
    (1, 257, 8, 1, 64, 1000, 4, torch.bfloat16),    # w >= L: full causal
    (1, 400, 8, 2, 128, 90, 40, torch.bfloat16),    # sinks span two key tiles
    (1, 200, 4, 2, 64, 5, 4, torch.bfloat16),       # a one-slot ring
    (3, 130, 2, 1, 64, 33, 1, torch.float32),
    (1, 500, 8, 8, 128, 64, 4, torch.float32),
    (1, 96, 16, 2, 128, 48, 4, torch.float32),
]


@pytest.mark.parametrize("case", EDGE, ids=lambda c: "B%d_L%d_H%d-%d_d%d_w%d_s%d_%s" % (
    c[0], c[1], c[2], c[3], c[4], c[5], c[6], str(c[7]).split(".")[-1]))
def test_prefill_edge_cases(swa, case):
    B, L, Hq, Hkv, d, w, s, dtype = case
    bf = dtype == torch.bfloat16
    Q, K, V = synth.prefill_inputs(B, L, Hq, Hkv, d, seed=L + w, workload=11, bf16=bf)
    O = host(swa.prefill(dev(Q, dtype), dev(K, dtype), dev(V, dtype), w, s))
    check(O, oracle.prefill(Q, K, V, w, s), dtype, str(case))


@pytest.mark.parametrize("w", [64, 512])
def test_prefill_bf16_in_fp32_out(swa, w):
    """bf16 inputs, fp32 output (out_dt = F32): within the bf16 bound of the
    oracle, and rounding it to bf16 gives the bf16-output path bit for bit
    (both store the same fp32 quotient; only the final rounding differs)."""
    Q, K, V = synth.prefill_inputs(1, 1000, 32, 8, 128, seed=w, workload=2, bf16=True, sink_outliers=4)
    q, k, v = (dev(x, torch.bfloat16) for x in (Q, K, V))
    O32 = swa.prefill(q, k, v, w, 4, out_dtype=torch.float32)
    assert O32.dtype == torch.float32
    O16 = swa.prefill(q, k, v, w, 4)
    assert torch.equal(O32.to(torch.bfloat16), O16)
    check(host(O32), oracle.prefill(Q, K, V, w, 4), torch.bfloat16, "fp32 out")


def test_prefill_lse(swa):
    Q, K, V = synth.prefill_inputs(2, 300, 8, 2, 64, seed=5, workload=12, bf16=False)
    O, lse = swa.prefill(dev(Q, torch.float32), dev(K, torch.float32), dev(V, torch.float32), 50, 4,
                         lse=True)
    Or, lr = oracle.prefill(Q, K, V, 50, 4, want_lse=True)
    check(host(O), Or, torch.float32)
    assert np.max(np.abs(host(lse) - lr)) < 1e-4


def test_prefill_deterministic_and_poison_invariant(swa):
    """Two runs are bit-identical; overwriting K/V of a position with +-1e4
    leaves bit-identical every row that does not attend it."""
    B, L, Hq, Hkv, d, w, s = 1, 700, 8, 2, 128, 64, 4
    Q, K, V = synth.prefill_inputs(B, L, Hq, Hkv, d, seed=3, workload=13, bf16=True)
    q, k, v = (dev(a, torch.bfloat16) for a in (Q, K, V))
    O1 = swa.prefill(q, k, v, w, s)
    O2 = swa.prefill(q, k, v, w, s)
    assert torch.equal(O1, O2)
    p = 100  # 1-based position, not a sink
    k2, v2 = k.clone(), v.clone()
    k2[:, p - 1] = 1e4
    v2[:, p - 1] = -1e4
    O3 = swa.prefill(q, k2, v2, w, s)
    untouched = [t for t in range(1, L + 1) if not brute.member(w, s, t, p)]
    assert len(untouched) > 500
    idx = torch.tensor([t - 1 for t in untouched], device="cuda")
    assert torch.equal(O1[:, idx], O3[:, idx])


# --- cache and decode -----------------------------------------------------------

def _rows(B, Hkv, d, positions, bf16, workload=3, sinks=0):
    return synth.position_rows(B, Hkv, d, positions, seed=0, workload=workload, bf16=bf16,
                               sink_outliers=sinks)


def _check_cache_slots(cache, rows_by_pos, w, s, n, dtype):
    """Read the cache back: slot j must hold exactly the row of the position the
    oracle's ring simulation put there."""
    rc = oracle.RingCache(w, s)
    for _ in range(n):
        rc.append()
    kc = cache.k.float().cpu().numpy()
    vc = cache.v.float().cpu().numpy()
    for j in range(min(n, w)):
        p = rc.held[j]
        kr, vr = rows_by_pos[p]
        np.testing.assert_array_equal(kc[:, :, j, :], kr)
        np.testing.assert_array_equal(vc[:, :, j, :], vr)


@pytest.mark.parametrize("dtype,d,G,w,s,prompt,last", [
    (torch.bfloat16, 128, 4, 64, 4, 100, 260),
    (torch.float32, 64, 2, 32, 4, 1, 120),
    (torch.bfloat16, 64, 1, 20, 0, 5, 90),
    (torch.bfloat16, 128, 8, 512, 4, 500, 1100),
])
def test_streaming_decode(swa, dtype, d, G, w, s, prompt, last):
    """Bulk-append a prompt, then append one position and decode at a time;
    every step matches the oracle over the full history, and the cache holds
    exactly the positions of S_n in the oracle's slots."""
    B, Hkv = 2, 4 if G < 8 else 2
    Hq = Hkv * G
    bf = dtype == torch.bfloat16
    cache = swa.Cache(B, Hkv, d, w, s, dtype=dtype)
    Kp, Vp = _rows(B, Hkv, d, range(1, prompt + 1), bf)
    cache.append(dev(Kp, dtype), dev(Vp, dtype))
    rows = {p: (Kp[:, p - 1], Vp[:, p - 1]) for p in range(1, prompt + 1)}
    checkpoints = {prompt + 1, w - 1, w, w + 1, 2 * w - s, 2 * w - s + 1, last}
    for n in range(prompt + 1, last + 1):
        Kn, Vn = _rows(B, Hkv, d, [n], bf)
        rows[n] = (Kn[:, 0], Vn[:, 0])
        cache.append(dev(Kn, dtype), dev(Vn, dtype))
        q = synth.query_rows(B, Hq, d, n, bf16=bf)
        o = host(cache.decode(dev(q, dtype)))
        S = oracle.attended(w, s, n)
        Kh = np.stack([rows[p][0] for p in S], axis=1)
        Vh = np.stack([rows[p][1] for p in S], axis=1)
        check(o, oracle.decode(q, S, Kh, Vh, n, w, s), dtype, "n=%d" % n)
        if n in checkpoints:
            _check_cache_slots(cache, rows, w, s, n, dtype)


@pytest.mark.parametrize("d,G,w,n", [(128, 4, 256, 600), (128, 8, 200, 180), (64, 8, 256, 257),
                                     (128, 4, 576, 1100), (128, 4, 576, 300), (64, 8, 576, 1100)])
def test_decode_eight_wave_workgroups(swa, d, G, w, n):
    """32 x 8 (batch, kv-head) pairs with 5..18 chunks of 32 rows each: the
    decode plan gives each pair a whole 8-wave workgroup (the Qwen3-4B-shaped
    batch-32 layer takes this path); plain and fused-step decode match the
    oracle, including a window not yet full (n = 180 < w = 200).  At SWA(576,4)
    the 18 chunks leave waves 0 and 1 one chunk more, which they request
    together with their first: the fused step's new row lands in that early
    chunk at n = 1100 (slot 527) and at n = 300 (slot 299, the last rows of a
    window still filling, 10 chunks)."""
    B, Hkv, s = 32, 8, 4
    Hq = G * Hkv
    cache = swa.Cache(B, Hkv, d, w, s, dtype=torch.bfloat16)
    K, V = _rows(B, Hkv, d, range(1, n + 1), True, workload=29)
    cache.append(dev(K[:, :n - 1], torch.bfloat16), dev(V[:, :n - 1], torch.bfloat16))
    q = synth.query_rows(B, Hq, d, n)
    # fused step: append position n and decode at it in one call
    o_step = host(cache.step(dev(K[:, n - 1], torch.bfloat16), dev(V[:, n - 1], torch.bfloat16),
                             dev(q, torch.bfloat16)))
    o = host(cache.decode(dev(q, torch.bfloat16)))
    S = np.asarray(oracle.attended(w, s, n))
    ref = oracle.decode(q, S, K[:, S - 1], V[:, S - 1], n, w, s)
    check(o, ref, torch.bfloat16, "decode B=32 d=%d G=%d w=%d n=%d" % (d, G, w, n))
    check(o_step, ref, torch.bfloat16, "fused step B=32 d=%d G=%d w=%d n=%d" % (d, G, w, n))


@pytest.mark.parametrize("B,Hkv,G,w,n", [(40, 3, 4, 64, 200),     # 120 pairs of 2 chunks: two tasks per workgroup
                                         (51, 6, 4, 256, 300),    # 306 pairs of 8 chunks: 8-wave workgroups
                                         (3, 5, 2, 512, 700),     # 15 pairs of 16 chunks: 16-wave workgroups
                                         (1, 3, 8, 4096, 5000)])  # 3 pairs of 128 chunks: splits and the merge
def test_decode_kv_heads_not_power_of_two(swa, B, Hkv, G, w, n):
    """Kv-head counts that are not powers of two, on each decode plan: the
    kernel takes a task's (batch, kv-head) pair by division there (by shifts
    for powers of two), and a split's index by division whenever the window
    is split.  Plain decode and the fused step against the oracle."""
    d, s = 128, 4
    Hq = G * Hkv
    cache = swa.Cache(B, Hkv, d, w, s, dtype=torch.bfloat16)
    K, V = _rows(B, Hkv, d, range(1, n + 1), True, workload=41, sinks=4)
    cache.append(dev(K[:, :n - 1], torch.bfloat16), dev(V[:, :n - 1], torch.bfloat16))
    q = synth.query_rows(B, Hq, d, n, workload=41)
    ws = torch.empty(max(cache.workspace_bytes(Hq), 16), dtype=torch.uint8, device="cuda")
    o_step = host(cache.step(dev(K[:, n - 1], torch.bfloat16), dev(V[:, n - 1], torch.bfloat16),
                             dev(q, torch.bfloat16), workspace=ws))
    o = host(cache.decode(dev(q, torch.bfloat16), workspace=ws))
    S = np.asarray(oracle.attended(w, s, n))
    ref = oracle.decode(q, S, K[:, S - 1], V[:, S - 1], n, w, s)
    what = "B=%d Hkv=%d G=%d SWA(%d,4) n=%d" % (B, Hkv, G, w, n)
    check(o, ref, torch.bfloat16, "decode " + what)
    check(o_step, ref, torch.bfloat16, "fused step " + what)


@pytest.mark.parametrize("B,d,G,w,n", [(1, 128, 4, 512, 900), (3, 64, 8, 300, 301), (7, 128, 1, 512, 512),
                                       (2, 128, 4, 400, 390)])
def test_decode_sixteen_wave_workgroups(swa, B, d, G, w, n):
    """Fewer than 64 (batch, kv-head) pairs with 9..16 chunks of 32 rows each:
    the decode plan gives each pair one 16-wave workgroup (a chunk per wave,
    accumulators left in each wave's V tile) instead of splitting the window
    over workgroups and merging in a second launch.  Plain decode, the fused
    step and the learned sink against the oracle."""
    Hkv, s = 8, 4
    Hq = G * Hkv
    cache = swa.Cache(B, Hkv, d, w, s, dtype=torch.bfloat16)
    assert cache.workspace_bytes(Hq) == 0  # no split anywhere up to a full window
    K, V = _rows(B, Hkv, d, range(1, n + 1), True, workload=31)
    cache.append(dev(K[:, :n - 1], torch.bfloat16), dev(V[:, :n - 1], torch.bfloat16))
    q = synth.query_rows(B, Hq, d, n)
    o_step = host(cache.step(dev(K[:, n - 1], torch.bfloat16), dev(V[:, n - 1], torch.bfloat16),
                             dev(q, torch.bfloat16)))
    o = host(cache.decode(dev(q, torch.bfloat16)))
    sink = np.random.default_rng(n).uniform(-2.0, 12.0, Hq).astype(np.float32)
    o_sink = host(cache.decode(dev(q, torch.bfloat16), sink_logit=torch.from_numpy(sink).cuda()))
    S = np.asarray(oracle.attended(w, s, n))
    ref = oracle.decode(q, S, K[:, S - 1], V[:, S - 1], n, w, s)
    ref_sink = oracle.decode(q, S, K[:, S - 1], V[:, S - 1], n, w, s, sink=sink.astype(np.float64))
    check(o, ref, torch.bfloat16, "decode B=%d d=%d G=%d w=%d n=%d" % (B, d, G, w, n))
    check(o_step, ref, torch.bfloat16, "fused step B=%d d=%d G=%d w=%d n=%d" % (B, d, G, w, n))
    check(o_sink, ref_sink, torch.bfloat16, "learned sink B=%d d=%d G=%d w=%d n=%d" % (B, d, G, w, n))


def test_decode_batch16_w512_eight_wave_two_chunks(swa):
    """Batch 16 x 8 kv-heads at SWA(512,4), n = 700: 128 (batch, kv-head)
    pairs with 16 chunks each, which the decode plan gives one 8-wave
    workgroup per pair, two chunks per wave, with no split; plain decode and
    the fused step against the oracle."""
    B, Hkv, d, w, s, G, n = 16, 8, 128, 512, 4, 4, 700
    Hq = G * Hkv
    cache = swa.Cache(B, Hkv, d, w, s, dtype=torch.bfloat16)
    K, V = _rows(B, Hkv, d, range(1, n + 1), True, workload=30)
    cache.append(dev(K[:, :n - 1], torch.bfloat16), dev(V[:, :n - 1], torch.bfloat16))
    q = synth.query_rows(B, Hq, d, n)
    o_step = host(cache.step(dev(K[:, n - 1], torch.bfloat16), dev(V[:, n - 1], torch.bfloat16),
                             dev(q, torch.bfloat16)))
    o = host(cache.decode(dev(q, torch.bfloat16)))
    S = np.asarray(oracle.attended(w, s, n))
    ref = oracle.decode(q, S, K[:, S - 1], V[:, S - 1], n, w, s)
    check(o, ref, torch.bfloat16, "decode B=16 w=512 n=%d" % n)
    check(o_step, ref, torch.bfloat16, "fused step B=16 w=512 n=%d" % n)


def test_bulk_append_equals_sequential(swa):
    B, Hkv, d, w, s = 2, 8, 128, 64, 4
    dtype = torch.bfloat16
    K, V = _rows(B, Hkv, d, range(1, 301), True, workload=21)
    a = swa.Cache(B, Hkv, d, w, s, dtype=dtype)
    b = swa.Cache(B, Hkv, d, w, s, dtype=dtype)
    a.k.zero_(); a.v.zero_(); b.k.zero_(); b.v.zero_()
    a.append(dev(K, dtype), dev(V, dtype))
    kd, vd = dev(K, dtype), dev(V, dtype)
    for p in range(300):
        b.append(kd[:, p:p + 1].contiguous(), vd[:, p:p + 1].contiguous())
    assert a.n == b.n == 300
    assert torch.equal(a.k, b.k) and torch.equal(a.v, b.v)
    # chunks of odd sizes, some longer than the ring
    c = swa.Cache(B, Hkv, d, w, s, dtype=dtype)
    c.k.zero_(); c.v.zero_()
    for lo, hi in [(0, 3), (3, 150), (150, 151), (151, 230), (230, 300)]:
        c.append(kd[:, lo:hi].contiguous(), vd[:, lo:hi].contiguous())
    assert torch.equal(a.k, c.k) and torch.equal(a.v, c.v)


@pytest.mark.parametrize("w", [64, 512])
def test_decode_streaming_shape_full_size(swa, w):
    """Batch 64, 32/8 heads, d=128, bf16, SWA(w,4) at positions 32766..32768:
    a 128-token prompt, then positions up to 32765 fast-forwarded in bulk.
    Positions that S_32768 no longer holds carry finite poison (+-1e4), so any
    read of an evicted row shows up."""
    B, Hq, Hkv, d, s, N = 64, 32, 8, 128, 4, 32768
    dtype = torch.bfloat16
    cache = swa.Cache(B, Hkv, d, w, s, dtype=dtype)
    Kp, Vp = _rows(B, Hkv, d, range(1, 129), True)
    cache.append(dev(Kp, dtype), dev(Vp, dtype))
    rows = {p: (Kp[:, p - 1], Vp[:, p - 1]) for p in range(1, 5)}  # sinks
    tail0 = N - 3 - w  # real rows from here on
    chunk = 4096
    pk = torch.full((B, chunk, Hkv, d), 1e4, dtype=dtype, device="cuda")
    pv = torch.full((B, chunk, Hkv, d), -1e4, dtype=dtype, device="cuda")
    p = 129
    while p < tail0:
        k = min(chunk, tail0 - p)
        cache.append(pk[:, :k].contiguous(), pv[:, :k].contiguous())
        p += k
    Kt, Vt = _rows(B, Hkv, d, range(tail0, N - 2), True)
    cache.append(dev(Kt, dtype), dev(Vt, dtype))
    for j, pos in enumerate(range(tail0, N - 2)):
        rows[pos] = (Kt[:, j], Vt[:, j])
    assert cache.n == N - 3
    for n in (N - 2, N - 1, N):
        Kn, Vn = _rows(B, Hkv, d, [n], True)
        rows[n] = (Kn[:, 0], Vn[:, 0])
        cache.append(dev(Kn, dtype), dev(Vn, dtype))
        q = synth.query_rows(B, Hq, d, n)
        o = host(cache.decode(dev(q, dtype)))
        S = oracle.attended(w, s, n)
        Kh = np.stack([rows[i][0] for i in S], axis=1)
        Vh = np.stack([rows[i][1] for i in S], axis=1)
        check(o, oracle.decode(q, S, Kh, Vh, n, w, s), dtype, "n=%d" % n)


@pytest.mark.parametrize("n", [1100, 16384])
def test_full_history_decode_split(swa, n):
    """Full causal attention as SWA with a window as long as the context
    (w = capacity): a long cache at batch 1 is split over workgroups and merged."""
    B, Hq, Hkv, d, w, s = 1, 32, 8, 128, 16384, 4
    dtype = torch.bfloat16
    cache = swa.Cache(B, Hkv, d, w, s, dtype=dtype)
    K, V = _rows(B, Hkv, d, range(1, n + 1), True, workload=4)
    cache.append(dev(K, dtype), dev(V, dtype))
    q = synth.query_rows(B, Hq, d, n, workload=4)
    o = host(cache.decode(dev(q, dtype)))
    pos = np.arange(1, n + 1)
    check(o, oracle.decode(q, pos, K, V, n, w, s), dtype, "n=%d" % n)


def test_decode_equals_prefill_rows(swa):
    """Decode at position t over a cache filled with positions 1..t gives the
    prefill row t (both within tolerance of the same oracle row)."""
    B, L, Hq, Hkv, d, w, s = 2, 200, 8, 2, 128, 48, 4
    dtype = torch.bfloat16
    Q, K, V = synth.prefill_inputs(B, L, Hq, Hkv, d, seed=9, workload=14, bf16=True)
    q, k, v = (dev(a, dtype) for a in (Q, K, V))
    O = host(swa.prefill(q, k, v, w, s))
    cache = swa.Cache(B, Hkv, d, w, s, dtype=dtype)
    for t in range(1, L + 1):
        cache.append(k[:, t - 1:t].contiguous(), v[:, t - 1:t].contiguous())
        if t in (1, 2, 47, 48, 49, 100, 200):
            o = host(cache.decode(q[:, t - 1].contiguous()))
            assert np.max(np.abs(o - O[:, t - 1])) <= 2 * BF16_ABS


def test_decode_snapshot_restore(swa):
    B, Hq, Hkv, d, w, s = 2, 16, 4, 128, 64, 4
    dtype = torch.bfloat16
    a = swa.Cache(B, Hkv, d, w, s, dtype=dtype)
    K, V = _rows(B, Hkv, d, range(1, 151), True, workload=22)
    a.append(dev(K, dtype), dev(V, dtype))
    b = swa.Cache(B, Hkv, d, w, s, dtype=dtype, k=a.k.clone(), v=a.v.clone())
    b.n = a.n
    for n in range(151, 170):
        Kn, Vn = _rows(B, Hkv, d, [n], True, workload=22)
        q = dev(synth.query_rows(B, Hq, d, n, workload=22), dtype)
        for c in (a, b):
            c.append(dev(Kn, dtype), dev(Vn, dtype))
        assert torch.equal(a.decode(q), b.decode(q))


def test_decode_errors_on_device(swa):
    cache = swa.Cache(1, 8, 128, 64, 4, dtype=torch.bfloat16)
    q = torch.zeros((1, 32, 128), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(swa.SwaError) as e:
        cache.decode(q)
    assert e.value.status == swa.SWA_ERR_STATE
