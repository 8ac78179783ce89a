"""GPU parity of the learned-sink variant (swa_prefill_lsink, swa_decode_lsink)
against the fp64 oracle with the same per-head logits.  Synthetic logits
(trained values are not available): a spread around the rows' log-sum-exp, so
the sink takes anything from a negligible to a dominant share, plus -inf
(no term).  Tolerances as in test_gpu_parity."""
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


def logits(Hq, seed):
    b = np.random.default_rng(seed).uniform(-2.0, 12.0, Hq).astype(np.float32)
    b[0] = -np.inf  # a head without the term
    return b


@pytest.mark.parametrize("dtype,d,Hq,Hkv,w,s", [
    (torch.bfloat16, 128, 32, 8, 512, 4),
    (torch.bfloat16, 64, 8, 8, 64, 0),
    (torch.float32, 128, 8, 2, 100, 4),
    (torch.float32, 64, 4, 1, 40, 33),
])
def test_prefill_lsink(swa, dtype, d, Hq, Hkv, w, s):
    bf = dtype == torch.bfloat16
    L = 1000 if bf else 300
    Q, K, V = synth.prefill_inputs(1, L, Hq, Hkv, d, seed=w, workload=41, bf16=bf, sink_outliers=4 if bf else 0)
    b = logits(Hq, w)
    O, lse = swa.prefill(dev(Q, dtype), dev(K, dtype), dev(V, dtype), w, s, lse=True,
                         sink_logit=torch.from_numpy(b).cuda())
    Or, lr = oracle.prefill(Q, K, V, w, s, want_lse=True, sink=b.astype(np.float64))
    check(host(O), Or, dtype, "O")
    assert np.max(np.abs(host(lse) - lr)) < (2e-2 if bf else 1e-4)
    # the no-term head equals the plain path
    Op = oracle.prefill(Q, K, V, w, s)
    check(host(O)[:, :, 0], Op[:, :, 0], dtype, "head without a term")


@pytest.mark.parametrize("B,w,n", [(8, 64, 300), (8, 512, 2000), (1, 16384, 16384)])
def test_decode_lsink(swa, B, w, n):
    """Batch decode at a full window, and a long full-history cache whose rows
    are split over workgroups (the term joins in the merge)."""
    Hq, Hkv, d, s = 32, 8, 128, 4
    dtype = torch.bfloat16
    cache = swa.Cache(B, Hkv, d, w, s, dtype=dtype)
    K, V = synth.history_rows(B, Hkv, d, n, workload=42)
    cache.append(dev(K, dtype), dev(V, dtype))
    q = synth.query_rows(B, Hq, d, n, workload=42)
    b = logits(Hq, n)
    o = host(cache.decode(dev(q, dtype), sink_logit=torch.from_numpy(b).cuda()))
    S = oracle.attended(w, s, n)
    idx = np.asarray(S) - 1
    ref = oracle.decode(q, S, K[:, idx], V[:, idx], n, w, s, sink=b.astype(np.float64))
    check(o, ref, dtype, "B=%d w=%d n=%d" % (B, w, n))
