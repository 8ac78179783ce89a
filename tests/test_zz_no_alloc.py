"""swa_decode_noalloc (the decode entry point that allocates nothing: its
split partials go to a fixed per-GPU array inside the library) against
swa_decode with a caller workspace, through the C ABI.  Same kernels and the
same plan, so the outputs must be bit-identical; the first call is also
checked against the oracle.  Two calls in a row, the second on a smaller
input, so the fixed array is reused with leftovers of the first call in it;
then a call whose plan does not split at all."""
import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu

BF = torch.bfloat16


@pytest.fixture(scope="module")
def swa():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    import sliding_window_sink_amd as swa
    return swa


def dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).to(device="cuda", dtype=BF)


def run_case(swa, B, Hkv, G, d, w, s, n, workload, want_split):
    print("noalloc case B=%d Hkv=%d G=%d d=%d w=%d s=%d n=%d" % (B, Hkv, G, d, w, s, n), flush=True)
    Hq = G * Hkv
    K, V = synth.history_rows(B, Hkv, d, n, workload=workload)
    cache = swa.Cache(B, Hkv, d, w, s, dtype=BF)
    cache.append(dev(K), dev(V))
    assert (cache.workspace_bytes(Hq) > 0) == want_split
    q = synth.query_rows(B, Hq, d, n, workload=workload)
    qd = dev(q)
    ref_gpu = cache.decode(qd)                 # swa_decode, caller workspace
    out = torch.full_like(qd, float("nan"))
    got = cache.decode_noalloc(qd, out)         # swa_decode_noalloc, fixed scratch
    torch.cuda.synchronize()
    assert got.data_ptr() == out.data_ptr()
    assert torch.equal(got, ref_gpu), "noalloc output differs from swa_decode"
    return K, V, q, got


def test_noalloc_matches_decode_two_calls_then_unsplit(swa):
    # 1) a long window split over 64 workgroups per (batch, kv-head)
    B, Hkv, G, d, w, s, n = 1, 8, 4, 128, 16384, 4, 16384
    K, V, q, got = run_case(swa, B, Hkv, G, d, w, s, n, workload=81, want_split=True)
    S = np.asarray(oracle.attended(w, s, n))
    ref = oracle.decode(q, S, K[:, S - 1], V[:, S - 1], n, w, s)
    err = float(np.max(np.abs(got.float().cpu().numpy() - ref)))
    assert err <= 2e-2, "noalloc vs oracle: %.3g" % err
    # 2) right after, a smaller split decode reusing the same array
    run_case(swa, 1, 8, 4, 128, 4096, 4, 3000, workload=82, want_split=True)
    # 3) a plan with no split (the array is not touched)
    run_case(swa, 64, 8, 4, 128, 64, 4, 200, workload=83, want_split=False)


def test_noalloc_rejects_oversized_plan(swa):
    """255 pairs x 8 query heads at w = 1024 would need about 3.2 MB of
    partials, more than the fixed 2 MiB: rejected, nothing enqueued."""
    cache = swa.Cache(255, 1, 128, 1024, 4, dtype=BF)
    cache.n = 1024
    q = torch.zeros((255, 8, 128), dtype=BF, device="cuda")
    out = torch.zeros_like(q)
    with pytest.raises(swa.SwaError) as ei:
        cache.decode_noalloc(q, out)
    assert ei.value.status == swa.SWA_ERR_UNSUPPORTED and "scratch" in str(ei.value)
    torch.cuda.synchronize()
    assert torch.count_nonzero(out).item() == 0
