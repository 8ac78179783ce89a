"""GPU parity of chunked prefill / multi-query decode against the cache
(swa_prefill_chunk): positions n+1..n+C attend the cached ring plus the chunk,
then the chunk is appended.  The oracle is the plain definition: rows
n+1..n+C of an fp64 prefill over all n + C positions.  Tolerances as in
test_gpu_parity: fp32 max|d|/max|ref| <= 1e-5, bf16 max|d| <= 2e-2.
"""
import numpy as np
import pytest
import torch

import oracle
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
    err = float(np.max(np.abs(got - ref)))
    if dtype == torch.float32:
        scale = max(float(np.max(np.abs(ref))), 1e-30)
        assert err / scale <= F32_REL, "%s: rel err %.3g" % (what, err / scale)
    else:
        assert err <= BF16_ABS, "%s: abs err %.3g" % (what, err)


CASES = [  # dtype, d, G, Hkv, w, s, chunk sizes
    (torch.bfloat16, 128, 4, 2, 64, 4, [100, 37, 1, 200, 262]),     # chunks shorter and longer than w
    (torch.bfloat16, 128, 4, 2, 512, 4, [256] * 6),                  # ring wraps inside chunks
    (torch.float32, 64, 2, 2, 40, 33, [5, 30, 3, 100, 162]),         # n < s: sinks split cache/chunk
    (torch.bfloat16, 64, 1, 4, 20, 0, [7, 1, 33, 64, 45]),           # no sinks
    (torch.float32, 128, 8, 1, 100, 4, [1] * 40 + [60, 150]),        # C = 1 steps (decode)
    (torch.bfloat16, 128, 4, 2, 1000, 4, [300, 300, 300]),           # w beyond the prompt: full causal
]


def _random_case(seed):
    """A seeded draw: head dim, group size, kv-heads, window (one slot past the
    sinks up to past the prompt), 0..40 sinks and 2..7 chunks of 1..300 rows."""
    r = np.random.default_rng(8100 + seed)
    s = int(r.choice([0, 1, 4, 4, 17, 40]))
    w = int(r.integers(s + 1, s + 600))
    chunks = [int(c) for c in r.integers(1, 301, size=int(r.integers(2, 8)))]
    dtype = torch.float32 if seed % 4 == 3 else torch.bfloat16
    return (dtype, int(r.choice([64, 128])), int(r.choice([1, 2, 4, 8])), int(r.integers(1, 4)), w, s, chunks)


CASES += [_random_case(k) for k in range(16)]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "%s_d%d_G%d_w%d_s%d" % (
    str(c[0]).split(".")[-1], c[1], c[2], c[4], c[5]))
def test_chunked_prefill_equals_full_prefill(swa, case):
    dtype, d, G, Hkv, w, s, chunks = case
    B, Hq, L = 2, G * Hkv, sum(chunks)
    bf = dtype == torch.bfloat16
    Q, K, V = synth.prefill_inputs(B, L, Hq, Hkv, d, seed=w + s, workload=31, bf16=bf,
                                   sink_outliers=4 if bf else 0)
    ref = oracle.prefill(Q, K, V, w, s)
    q, k, v = (dev(x, dtype) for x in (Q, K, V))
    cache = swa.Cache(B, Hkv, d, w, s, dtype=dtype)
    bulk = swa.Cache(B, Hkv, d, w, s, dtype=dtype)
    n = 0
    for C in chunks:
        o = cache.prefill_chunk(q[:, n:n + C].contiguous(), k[:, n:n + C].contiguous(), v[:, n:n + C].contiguous())
        check(host(o), ref[:, n:n + C], dtype, "rows %d..%d" % (n + 1, n + C))
        n += C
        assert cache.n == n
    # the chunks left the cache a bulk append of all rows leaves
    bulk.append(k, v)
    held = min(n, w)
    assert torch.equal(cache.k[:, :, :held], bulk.k[:, :, :held])
    assert torch.equal(cache.v[:, :, :held], bulk.v[:, :, :held])


def test_chunk_lse_and_fp32_out(swa):
    B, Hq, Hkv, d, w, s = 1, 8, 2, 128, 64, 4
    Q, K, V = synth.prefill_inputs(B, 300, Hq, Hkv, d, seed=3, workload=32, bf16=True)
    ref, lref = oracle.prefill(Q, K, V, w, s, want_lse=True)
    q, k, v = (dev(x, torch.bfloat16) for x in (Q, K, V))
    cache = swa.Cache(B, Hkv, d, w, s, dtype=torch.bfloat16)
    cache.append(k[:, :200].contiguous(), v[:, :200].contiguous())
    o, lse = cache.prefill_chunk(q[:, 200:].contiguous(), k[:, 200:].contiguous(), v[:, 200:].contiguous(),
                                 lse=True, out_dtype=torch.float32)
    assert o.dtype == torch.float32
    check(host(o), ref[:, 200:], torch.bfloat16, "fp32 out")
    assert np.max(np.abs(host(lse) - lref[:, :, 200:])) < 2e-2


@pytest.mark.parametrize("w", [64, 512])
def test_multi_query_decode_after_long_stream(swa, w):
    """Batch 64, 32/8 heads, d = 128, bf16: the cache is driven to n = 32764
    (rows S_n no longer holds carry finite poison), then 4 draft positions are
    verified at once (C = 4) against the oracle over the full history."""
    B, Hq, Hkv, d, s, N, C = 64, 32, 8, 128, 4, 32764, 4
    dtype = torch.bfloat16
    cache = swa.Cache(B, Hkv, d, w, s, dtype=dtype)
    rows = lambda ps: synth.position_rows(B, Hkv, d, ps, seed=0, workload=33, bf16=True)
    Ks, Vs = rows(range(1, s + 1))
    cache.append(dev(Ks, dtype), dev(Vs, dtype))
    real_from = N + 1 - (w - s) + 1  # the first draft's window starts here; later drafts start later
    chunk = 4096
    pk = torch.full((B, chunk, Hkv, d), 1e4, dtype=dtype, device="cuda")
    pv = torch.full((B, chunk, Hkv, d), -1e4, dtype=dtype, device="cuda")
    while cache.n < real_from - 1:
        kk = min(chunk, real_from - 1 - cache.n)
        cache.append(pk[:, :kk].contiguous(), pv[:, :kk].contiguous())
    Kt, Vt = rows(range(real_from, N + 1))
    cache.append(dev(Kt, dtype), dev(Vt, dtype))
    assert cache.n == N
    Kd, Vd = rows(range(N + 1, N + C + 1))
    Qd = np.stack([synth.query_rows(B, Hq, d, N + 1 + i, workload=33) for i in range(C)], axis=1)
    o = host(cache.prefill_chunk(dev(Qd, dtype), dev(Kd, dtype), dev(Vd, dtype)))
    assert cache.n == N + C
    for i in range(C):
        t = N + 1 + i
        S = oracle.attended(w, s, t)
        Kh, Vh = rows(S)
        check(o[:, i], oracle.decode(Qd[:, i], S, Kh, Vh, t, w, s), dtype, "draft %d" % (i + 1))


@pytest.mark.parametrize("B,N", [(1, 4096), (2, 4133)])
def test_long_chunk_behind_full_ring(swa, B, N):
    """A 512-position chunk behind a full SWA(512,4) ring (32/8 heads,
    d = 128, bf16), the bench's chunked-prefill shape: every row of the chunk
    attends the sinks, the part of the ring its window still reaches, and
    the chunk up to itself, so each query block visits a different subset of
    the cache tiles.  Positions outside every S_t carry finite poison;
    sampled rows (block edges, the window's reach into the ring running out)
    against the oracle over the full history."""
    Hq, Hkv, d, w, s, C = 32, 8, 128, 512, 4, 512
    dtype = torch.bfloat16
    cache = swa.Cache(B, Hkv, d, w, s, dtype=dtype)
    rows = lambda ps: synth.position_rows(B, Hkv, d, ps, seed=1, workload=34, bf16=True)
    Ks, Vs = rows(range(1, s + 1))
    cache.append(dev(Ks, dtype), dev(Vs, dtype))
    real_from = N + 2 - (w - s)  # the first chunk row's window starts here
    pk = torch.full((B, real_from - 1 - s, Hkv, d), 1e4, dtype=dtype, device="cuda")
    pv = torch.full((B, real_from - 1 - s, Hkv, d), -1e4, dtype=dtype, device="cuda")
    cache.append(pk, pv)
    Kt, Vt = rows(range(real_from, N + 1))
    cache.append(dev(Kt, dtype), dev(Vt, dtype))
    assert cache.n == N
    Kd, Vd = rows(range(N + 1, N + C + 1))
    Qd = np.stack([synth.query_rows(B, Hq, d, N + 1 + i, workload=34) for i in range(C)], axis=1)
    o = host(cache.prefill_chunk(dev(Qd, dtype), dev(Kd, dtype), dev(Vd, dtype)))
    assert cache.n == N + C
    for i in (0, 1, 31, 32, 33, 95, 255, 256, 479, 480, 505, 506, 507, 508, 509, 511):
        t = N + 1 + i
        S = oracle.attended(w, s, t)
        Kh, Vh = rows(S)
        check(o[:, i], oracle.decode(Qd[:, i], S, Kh, Vh, t, w, s), dtype, "chunk row %d" % (i + 1))
