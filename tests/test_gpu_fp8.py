"""GPU parity of the fp8 (OCP E4M3) KV cache: swa_cache_append_fp8 and
swa_decode_fp8 against the oracle's E4M3 codec and fp64 decode.

- Cache bytes are compared bit-exactly: every occupied slot must hold the
  code oracle.fp8.quantize gives for the row of the position the oracle's
  slot map puts there (bulk appends that wrap the ring, single appends).
- Decode output is compared with the oracle's decode over the dequantised
  rows (code value * scale) within the bf16 tolerance of the other decode
  tests (2e-2 absolute).

Scales are synthetic: amax / 448 of each kv-head's rows (a per-head
calibration), with one head at a quarter of that so its largest values
saturate at +-448."""
import numpy as np
import pytest
import torch

import oracle
import oracle.fp8 as fp8
import synth

pytestmark = pytest.mark.gpu

BF16_ABS = 2e-2


@pytest.fixture(scope="module")
def swa():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    import sliding_window_sink_amd as swa
    return swa


def dev(x, dtype=torch.bfloat16):
    return torch.from_numpy(np.ascontiguousarray(x)).to(device="cuda", dtype=dtype)


def scales(K, V):
    """[2, Hkv] float32: amax/448 per kv-head, the last head's at a quarter."""
    out = np.empty((2, K.shape[2]), dtype=np.float32)
    for i, X in enumerate((K, V)):
        amax = np.max(np.abs(X), axis=(0, 1, 3))
        out[i] = np.maximum(amax, 1e-3) / 448.0
    out[:, -1] *= 0.25
    return out


def codes(X, sc):
    """E4M3 codes of rows X [B, n, Hkv, d] with per-head scales sc [Hkv]."""
    return np.stack([fp8.quantize(X[:, :, h], sc[h]) for h in range(X.shape[2])], axis=2)


def dequant(C, sc):
    return np.stack([fp8.dequantize(C[:, :, h], sc[h]) for h in range(C.shape[2])], axis=2)


def check_slots(cache, Kc, Vc, w, s, n):
    """Slot j of every (b, kv-head) holds the codes of the position the
    oracle's slot map assigns to it; unoccupied slots are not compared."""
    kb = cache.k.view(torch.uint8).cpu().numpy()
    vb = cache.v.view(torch.uint8).cpu().numpy()
    for p in oracle.attended(w, s, n):
        j = oracle.slot(w, s, int(p))
        np.testing.assert_array_equal(kb[:, :, j], Kc[:, p - 1], err_msg="K slot %d (position %d)" % (j, p))
        np.testing.assert_array_equal(vb[:, :, j], Vc[:, p - 1], err_msg="V slot %d (position %d)" % (j, p))


@pytest.mark.parametrize("d", [64, 128])
def test_append_codes_exact(swa, d):
    B, Hkv, w, s = 2, 4, 64, 4
    steps = [300, 1, 1, 1, 1, 1, 100, 37]  # bulk wraps, single appends, bulk again
    n = sum(steps)
    K, V = synth.history_rows(B, Hkv, d, n, workload=51)
    sc = scales(K, V)
    Kc, Vc = codes(K, sc[0]), codes(V, sc[1])
    assert np.any((Kc & 0x7F) == 0x7E), "the quarter-scale head should saturate"
    cache = swa.Cache(B, Hkv, d, w, s, dtype=torch.float8_e4m3fn, kv_scale=dev(sc, torch.float32))
    done = 0
    for k in steps:
        cache.append(dev(K[:, done:done + k]), dev(V[:, done:done + k]))
        done += k
        if k > 1 or done == n:
            torch.cuda.synchronize()
            check_slots(cache, Kc, Vc, w, s, done)
    assert cache.n == n


def test_append_sinks_before_ring(swa):
    """A cache still filling its sinks (n < s), then one bulk step past them."""
    B, Hkv, d, w, s = 1, 2, 128, 40, 8
    K, V = synth.history_rows(B, Hkv, d, 50, workload=52)
    sc = scales(K, V)
    Kc, Vc = codes(K, sc[0]), codes(V, sc[1])
    cache = swa.Cache(B, Hkv, d, w, s, dtype=torch.float8_e4m3fn, kv_scale=dev(sc, torch.float32))
    cache.append(dev(K[:, :5]), dev(V[:, :5]))
    torch.cuda.synchronize()
    check_slots(cache, Kc, Vc, w, s, 5)
    cache.append(dev(K[:, 5:]), dev(V[:, 5:]))
    torch.cuda.synchronize()
    check_slots(cache, Kc, Vc, w, s, 50)


@pytest.mark.parametrize("B,Hq,Hkv,d,w,s,n,sink", [
    (8, 32, 8, 128, 64, 4, 300, False),
    (4, 8, 8, 64, 512, 4, 2000, False),       # G = 1, d = 64
    (2, 64, 8, 128, 100, 0, 777, True),       # G = 8, s = 0, learned sink
    (3, 16, 4, 64, 48, 6, 20, False),         # window not yet full
    (1, 32, 8, 128, 16384, 4, 16384, False),  # rows split over workgroups + merge
    (1, 32, 8, 128, 16384, 4, 16384, True),   # ... with the sink in the merge
    (64, 32, 8, 128, 512, 4, 600, False),     # batch-64 decode, window 512
    (64, 32, 8, 128, 64, 4, 300, False),      # batch-64 decode, window 64
    (16, 32, 8, 128, 512, 4, 700, False),     # 128 pairs x 16 chunks: one 8-wave workgroup per pair
])
def test_decode_fp8(swa, B, Hq, Hkv, d, w, s, n, sink):
    K, V = synth.history_rows(B, Hkv, d, n, workload=53)
    sc = scales(K, V)
    cache = swa.Cache(B, Hkv, d, w, s, dtype=torch.float8_e4m3fn, kv_scale=dev(sc, torch.float32))
    cache.append(dev(K), dev(V))
    q = synth.query_rows(B, Hq, d, n, workload=53)
    b = None
    if sink:
        b = np.random.default_rng(n).uniform(-2.0, 12.0, Hq).astype(np.float32)
        b[0] = -np.inf
    o = cache.decode(dev(q), sink_logit=None if b is None else torch.from_numpy(b).cuda())
    got = o.float().cpu().numpy().astype(np.float64)
    S = np.asarray(oracle.attended(w, s, n))
    Kd = dequant(codes(K[:, S - 1], sc[0]), sc[0])
    Vd = dequant(codes(V[:, S - 1], sc[1]), sc[1])
    ref = oracle.decode(q, S, Kd, Vd, n, w, s, sink=None if b is None else b.astype(np.float64))
    err = float(np.max(np.abs(got - ref)))
    assert err <= BF16_ABS, "B=%d w=%d n=%d: abs err %.3g" % (B, w, n, err)


def test_decode_fp8_streaming(swa):
    """Append and decode one position at a time across the ring wrap."""
    B, Hq, Hkv, d, w, s = 4, 16, 4, 128, 32, 4
    n_end = 80
    K, V = synth.history_rows(B, Hkv, d, n_end, workload=54)
    sc = scales(K, V)
    Kd = dequant(codes(K, sc[0]), sc[0])
    Vd = dequant(codes(V, sc[1]), sc[1])
    cache = swa.Cache(B, Hkv, d, w, s, dtype=torch.float8_e4m3fn, kv_scale=dev(sc, torch.float32))
    pos = np.arange(1, n_end + 1)
    for n in range(1, n_end + 1):
        cache.append(dev(K[:, n - 1:n]), dev(V[:, n - 1:n]))
        if n in (1, 3, 31, 32, 33, 50, 80):
            q = synth.query_rows(B, Hq, d, n, workload=54)
            got = cache.decode(dev(q)).float().cpu().numpy().astype(np.float64)
            ref = oracle.decode(q, pos[:n], Kd[:, :n], Vd[:, :n], n, w, s)
            assert float(np.max(np.abs(got - ref))) <= BF16_ABS, "n=%d" % n
