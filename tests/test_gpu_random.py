"""GPU parity over seeded random shapes: prefill and decode through the C ABI
against the fp64 oracle, on shapes drawn from fixed generators.

The fixed-shape tests pin the configurations that are timed; these draw odd
lengths, every GQA group size, both head dims, windows from one slot past the
sinks to past the sequence, 0..40 sinks, sink outliers, fp32 and bf16, the LSE
output, bulk appends that wrap the ring several times, the fused step, and
(batch, kv-head) counts that reach the split, one-task-per-workgroup and
several-tasks-per-workgroup decode plans.  Tolerances are those of the fixed
cases: bf16 max-abs 2e-2, fp32 1e-5 relative to the largest output.
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


def check(got, ref, dtype, what):
    err = float(np.max(np.abs(got - ref))) if got.size else 0.0
    if dtype == torch.float32:
        scale = max(float(np.max(np.abs(ref))), 1e-30) if ref.size else 1.0
        assert err / scale <= F32_REL, "%s: rel err %.3g" % (what, err / scale)
    else:
        assert err <= BF16_ABS, "%s: abs err %.3g" % (what, err)


def prefill_case(seed):
    r = np.random.default_rng(7100 + seed)
    d = int(r.choice([64, 128]))
    G = int(r.choice([1, 2, 4, 8]))
    Hkv = int(r.integers(1, 4))
    B = int(r.integers(1, 4))
    L = int(r.integers(1, 700))
    s = int(r.choice([0, 1, 4, 4, 4, 17, 40]))
    w = int(r.integers(s + 1, s + 801))
    dtype = torch.float32 if seed % 5 == 4 else torch.bfloat16
    outliers = min(s, 4) if seed % 2 else 0
    return B, L, Hkv * G, Hkv, d, w, s, dtype, outliers, seed % 3 == 0


PREFILL_SEEDS = range(24)


@pytest.mark.parametrize("seed", PREFILL_SEEDS, ids=lambda k: "seed%d" % k)
def test_prefill_random_shapes(swa, seed):
    B, L, Hq, Hkv, d, w, s, dtype, outliers, want_lse = prefill_case(seed)
    what = "seed %d: B=%d L=%d %d/%d d=%d SWA(%d,%d) %s" % (seed, B, L, Hq, Hkv, d, w, s, dtype)
    bf = dtype == torch.bfloat16
    Q, K, V = synth.prefill_inputs(B, L, Hq, Hkv, d, seed=seed, workload=71, bf16=bf,
                                   sink_outliers=outliers)
    q, k, v = (dev(a, dtype) for a in (Q, K, V))
    if want_lse:
        O, lse = swa.prefill(q, k, v, w, s, lse=True)
        Or, lr = oracle.prefill(Q, K, V, w, s, want_lse=True)
        # bf16: the denominator sums the bf16-rounded weights (relative error
        # below 2^-8), so log l is good to about 4e-3
        tol = 1e-4 if not bf else 1e-2
        assert np.max(np.abs(host(lse) - lr)) < tol, what + ": lse"
    else:
        O = swa.prefill(q, k, v, w, s)
        Or = oracle.prefill(Q, K, V, w, s)
    check(host(O), Or, dtype, what)


def decode_case(seed):
    r = np.random.default_rng(7300 + seed)
    d = int(r.choice([64, 128]))
    G = int(r.choice([1, 2, 4, 8]))
    Hkv = int(r.choice([1, 2, 4, 8]))
    B = int(r.integers(1, 41))
    s = int(r.choice([0, 1, 4, 4, 17]))
    w = int(r.integers(s + 1, s + 601))
    n = int(r.integers(1, 3 * w + 2))
    while B * Hkv * n > 64 * 1500:  # bound the host arrays
        B = max(1, B // 2)
        n = max(1, (n * 3) // 4)
    dtype = torch.float32 if seed % 4 == 3 else torch.bfloat16
    return B, Hkv, G, d, w, s, n, dtype, seed % 2 == 0


DECODE_SEEDS = range(20)


@pytest.mark.parametrize("seed", DECODE_SEEDS, ids=lambda k: "seed%d" % k)
def test_decode_random_shapes(swa, seed):
    B, Hkv, G, d, w, s, n, dtype, fused = decode_case(seed)
    what = "seed %d: B=%d Hkv=%d G=%d d=%d SWA(%d,%d) n=%d %s%s" % (
        seed, B, Hkv, G, d, w, s, n, dtype, " step" if fused else "")
    bf = dtype == torch.bfloat16
    Hq = G * Hkv
    cache = swa.Cache(B, Hkv, d, w, s, dtype=dtype)
    K, V = synth.position_rows(B, Hkv, d, range(1, n + 1), seed=seed, workload=73, bf16=bf,
                               sink_outliers=min(s, 4))
    q = synth.query_rows(B, Hq, d, n, seed=seed, workload=73, bf16=bf)
    if n > 1:
        cache.append(dev(K[:, :n - 1], dtype), dev(V[:, :n - 1], dtype))
    if fused:
        o = host(cache.step(dev(K[:, n - 1], dtype), dev(V[:, n - 1], dtype), dev(q, dtype)))
    else:
        cache.append(dev(K[:, n - 1:], dtype), dev(V[:, n - 1:], dtype))
        o = host(cache.decode(dev(q, dtype)))
    assert cache.n == n, what
    S = np.asarray(oracle.attended(w, s, n))
    check(o, oracle.decode(q, S, K[:, S - 1], V[:, S - 1], n, w, s), dtype, what)
