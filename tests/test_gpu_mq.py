"""GPU parity of the multi-query decode: a bf16 chunk of C rows with C * G <= 16
(several draft positions verified at once) after a cache that needs no split
goes through the decode kernel, whose MFMA columns then hold chunk rows x
heads, and the same launch writes the chunk's rows into their slots.  Each
chunk's rows must match the oracle's full prefill, and the cache must end up
holding what one bulk append of every row leaves -- across an empty cache,
sinks filled by the chunk, a ring that wraps inside a chunk, a one-slot ring
whose chunk rows evict each other, every (C, G) pairing and both workgroup
sizes of the kernel (4, 8 and 16 waves)."""
import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu

BF16_ABS = 2e-2


@pytest.fixture(scope="module")
def swa():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    import sliding_window_sink_amd as swa
    return swa


def dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).to(device="cuda", dtype=torch.bfloat16)


def host(t):
    return t.float().cpu().numpy().astype(np.float64)


CASES = [  # d, G, Hkv, w, s, chunk sizes (C * G <= 16)
    (128, 4, 2, 64, 4, [4] * 40),             # empty cache, sinks, ring fill and wraps
    (64, 1, 4, 5, 4, [16] * 5 + [3, 1]),      # one-slot ring: chunk rows evict each other
    (128, 8, 1, 40, 33, [2] * 30),            # the cache still inside the sinks for 16 chunks
    (64, 2, 4, 300, 0, [8] * 20 + [5, 7]),    # no sinks
    (128, 4, 3, 100, 17, [1, 2, 3, 4] * 12),  # every C at G = 4
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "d%d_G%d_w%d_s%d" % (c[0], c[1], c[3], c[4]))
def test_multi_query_chunks_equal_full_prefill(swa, case):
    d, G, Hkv, w, s, chunks = case
    B, Hq, L = 2, G * Hkv, sum(chunks)
    assert max(chunks) * G <= 16
    Q, K, V = synth.prefill_inputs(B, L, Hq, Hkv, d, seed=w + s, workload=37, bf16=True, sink_outliers=4)
    ref = oracle.prefill(Q, K, V, w, s)
    q, k, v = (dev(x) for x in (Q, K, V))
    cache = swa.Cache(B, Hkv, d, w, s)
    bulk = swa.Cache(B, Hkv, d, w, s)
    n = 0
    for C in chunks:
        o = cache.prefill_chunk(q[:, n:n + C].contiguous(), k[:, n:n + C].contiguous(), v[:, n:n + C].contiguous())
        err = np.max(np.abs(host(o) - ref[:, n:n + C]))
        assert err <= BF16_ABS, "rows %d..%d: abs err %.3g" % (n + 1, n + C, err)
        n += C
        assert cache.n == n
    bulk.append(k, v)
    held = min(n, w)
    assert torch.equal(cache.k[:, :, :held], bulk.k[:, :, :held])
    assert torch.equal(cache.v[:, :, :held], bulk.v[:, :, :held])


@pytest.mark.parametrize("B,w,C,G", [(32, 576, 4, 4), (32, 576, 2, 8), (32, 576, 16, 1),
                                     (1, 512, 4, 4), (1, 512, 16, 1), (3, 300, 8, 2)])
def test_multi_query_large_workgroups(swa, B, w, C, G):
    """Full windows whose plan gives each (batch, kv-head) pair one 8-wave
    workgroup (batch 32, SWA(576,4): the Qwen3-4B-shaped layer) or one 16-wave
    workgroup (batch 1 and 3, windows of up to 16 chunks): C draft rows after
    4000 positions, checked row by row against the oracle over the attended
    history, and the ring left as a bulk append leaves it."""
    Hkv, d, s, N = 8, 128, 4, 4000
    Hq = G * Hkv
    rows = lambda ps: synth.position_rows(B, Hkv, d, ps, seed=2, workload=38, bf16=True)
    cache = swa.Cache(B, Hkv, d, w, s)
    bulk = swa.Cache(B, Hkv, d, w, s)
    # the first chunk row (position N + 1) reaches back to position N + 2 - (w - s);
    # the positions between the sinks and that one are appended as constants
    first = N + 2 - (w - s)
    Kp, Vp = rows(range(1, s + 1))
    for c_ in (cache, bulk):
        c_.append(dev(Kp), dev(Vp))
    fill = torch.full((B, first - 1 - s, Hkv, d), 3.0, dtype=torch.bfloat16, device="cuda")
    for c_ in (cache, bulk):
        c_.append(fill, fill)
    Kt, Vt = rows(range(first, N + 1))
    for c_ in (cache, bulk):
        c_.append(dev(Kt), dev(Vt))
    assert cache.n == N
    Kd, Vd = rows(range(N + 1, N + C + 1))
    Qd = np.stack([synth.query_rows(B, Hq, d, N + 1 + i, workload=38) for i in range(C)], axis=1)
    o = host(cache.prefill_chunk(dev(Qd), dev(Kd), dev(Vd)))
    assert cache.n == N + C
    for i in range(C):
        t = N + 1 + i
        S = oracle.attended(w, s, t)
        Kh, Vh = rows(S)
        err = np.max(np.abs(o[:, i] - oracle.decode(Qd[:, i], S, Kh, Vh, t, w, s)))
        assert err <= BF16_ABS, "chunk row %d: abs err %.3g" % (i + 1, err)
    bulk.append(dev(Kd), dev(Vd))
    assert torch.equal(cache.k, bulk.k)
    assert torch.equal(cache.v, bulk.v)
