"""GPU parity of the fused generation step (swa_decode_step: append one
position and decode at it, one launch).  It must leave the same cache and
give the same output as swa_cache_append followed by swa_decode -- bit for
bit, since the new row enters the same MFMA lanes either way -- across sink
filling, the ring wrap and the split path, with and without a learned sink;
and match the oracle."""
import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def swa():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    import sliding_window_sink_amd as swa
    return swa


def dev(x, dtype):
    return torch.from_numpy(np.ascontiguousarray(x)).to(device="cuda", dtype=dtype)


def run_pair(swa, B, Hq, Hkv, d, w, s, prompt, steps, dtype, sink=None, check_every=1, workload=71):
    K, V = synth.history_rows(B, Hkv, d, prompt + steps, workload=workload, bf16=dtype != torch.float32)
    fused = swa.Cache(B, Hkv, d, w, s, dtype=dtype)
    plain = swa.Cache(B, Hkv, d, w, s, dtype=dtype)
    if prompt:
        for c in (fused, plain):
            c.append(dev(K[:, :prompt], dtype), dev(V[:, :prompt], dtype))
    sk = None if sink is None else torch.from_numpy(sink).cuda()
    last = None
    for j in range(steps):
        n = prompt + j + 1
        q = dev(synth.query_rows(B, Hq, d, n, workload=workload, bf16=dtype != torch.float32), dtype)
        kn, vn = dev(K[:, n - 1], dtype), dev(V[:, n - 1], dtype)
        of = fused.step(kn, vn, q, sink_logit=sk)
        plain.append(kn.unsqueeze(1).contiguous(), vn.unsqueeze(1).contiguous())
        op = plain.decode(q, sink_logit=sk)
        if j % check_every == 0 or j == steps - 1:
            assert torch.equal(of, op), "output differs at n=%d" % n
            occ = min(n, w)  # slots past the occupied ones were never written (uninitialised memory)
            assert torch.equal(fused.k[:, :, :occ], plain.k[:, :, :occ]) and \
                torch.equal(fused.v[:, :, :occ], plain.v[:, :, :occ]), "cache differs at n=%d" % n
        last = (n, q, of)
    assert fused.n == plain.n == prompt + steps
    return K, V, last


def check_oracle(K, V, last, w, s, sink=None, tol=2e-2):
    """The fused step's output at its last position against the fp64 oracle
    over the history rows it attends."""
    n, q, o = last
    S = np.asarray(oracle.attended(w, s, n))
    ref = oracle.decode(q.float().cpu().numpy(), S, K[:, S - 1], V[:, S - 1], n, w, s, sink=sink)
    err = float(np.max(np.abs(o.float().cpu().numpy() - ref)))
    assert err <= tol, "fused step vs oracle at n=%d: %.3g" % (n, err)


@pytest.mark.parametrize("d,Hq,Hkv,w,s", [(128, 32, 8, 64, 4), (64, 16, 2, 40, 0), (128, 8, 8, 100, 33)])
def test_step_equals_append_decode(swa, d, Hq, Hkv, w, s):
    B = 8
    K, V, last = run_pair(swa, B, Hq, Hkv, d, w, s, prompt=0, steps=150, dtype=torch.bfloat16)
    check_oracle(K, V, last, w, s)


def test_step_with_sink_and_prompt(swa):
    Hq = 32
    sink = np.random.default_rng(3).uniform(-2.0, 12.0, Hq).astype(np.float32)
    sink[0] = -np.inf
    K, V, last = run_pair(swa, 4, Hq, 8, 128, 512, 4, prompt=500, steps=30, dtype=torch.bfloat16, sink=sink)
    check_oracle(K, V, last, 512, 4, sink=sink.astype(np.float64))


def test_step_split_path(swa):
    """A long window whose rows are split over workgroups: the new row lands
    in one split's chunk and the merge sees it once."""
    K, V, last = run_pair(swa, 1, 32, 8, 128, 16384, 4, prompt=16370, steps=30, dtype=torch.bfloat16,
                          check_every=7)
    check_oracle(K, V, last, 16384, 4)


def test_step_fp32_cache(swa):
    K, V, last = run_pair(swa, 2, 8, 2, 64, 48, 4, prompt=3, steps=60, dtype=torch.float32, check_every=5)
    n, q, o = last
    S = np.asarray(oracle.attended(48, 4, n))
    ref = oracle.decode(q.cpu().numpy(), S, K[:, S - 1], V[:, S - 1], n, 48, 4)
    assert np.max(np.abs(o.cpu().numpy() - ref)) <= 1e-5 * np.max(np.abs(ref))


def test_step_batch64_full_window(swa):
    """The bench's decode shape: batch 64, 32/8 heads, SWA(512,4), full window."""
    K, V, last = run_pair(swa, 64, 32, 8, 128, 512, 4, prompt=600, steps=4, dtype=torch.bfloat16)
    check_oracle(K, V, last, 512, 4)


def test_step_batch16_eight_wave_plan(swa):
    """Batch 16 x 8 kv-heads at SWA(512,4): 128 (batch, kv-head) pairs with 16
    chunks each, the plan that gives each pair one 8-wave workgroup and two
    chunks per wave instead of splits and a merge."""
    K, V, last = run_pair(swa, 16, 32, 8, 128, 512, 4, prompt=700, steps=3, dtype=torch.bfloat16)
    check_oracle(K, V, last, 512, 4)
