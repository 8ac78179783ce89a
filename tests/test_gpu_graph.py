"""The generation step inside a captured HIP graph.  A serving loop at small
batch is bound by launch overhead, and capturing its step in a graph is how
it removes that; the bench times the batch-1 step that way.  Each case
captures one fused append + decode step (swa_decode_step) at position n+1,
replays the graph several times with eager work and synchronisations between
the replays, and checks every replay's output bit for bit against the eager
call's, and the eager call against the oracle.  The cases take the three
batch-1 decode plans: one 16-wave workgroup per (b, kv-head) (SWA(512,4)), a
4-wave task (SWA(64,4)), and splits with the merge launch and a workspace
(full causal at 2^14 cached positions)."""
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


def dev(x, dtype=torch.bfloat16):
    return torch.from_numpy(np.ascontiguousarray(x)).to(device="cuda", dtype=dtype)


def host(t):
    return t.float().cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("w,n", [(512, 1000), (64, 300), (2 ** 14 + 64, 2 ** 14)])
def test_step_graph_replay(swa, w, n):
    B, Hkv, G, d, s = 1, 8, 4, 128, 4
    Hq = Hkv * G
    K, V = synth.history_rows(B, Hkv, d, n + 1, workload=83, bf16=True)
    cache = swa.Cache(B, Hkv, d, w, s)
    cache.append(dev(K[:, :n]), dev(V[:, :n]))
    q = dev(synth.query_rows(B, Hq, d, n + 1, workload=83))
    kn, vn = dev(K[:, n]), dev(V[:, n])

    # eager step at position n + 1 (it also sizes any workspace), checked
    # against the oracle; then rewind the count so the capture sees position n + 1 again
    eager = cache.step(kn, vn, q)
    torch.cuda.synchronize()
    S = np.asarray(oracle.attended(w, s, n + 1))
    ref = oracle.decode(host(q), S, K[:, S - 1], V[:, S - 1], n + 1, w, s)
    err = np.max(np.abs(host(eager) - ref))
    assert err < 2e-2, "eager step vs oracle: %g" % err
    cache.n = n

    out = torch.empty_like(q)
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            cache.step(kn, vn, q, out=out)
    torch.cuda.synchronize()
    for r in range(4):
        out.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), "replay %d differs from the eager step" % r
        # eager work between replays: a plain decode on the default stream
        cache.n = n + 1
        other = cache.decode(q)
        torch.cuda.synchronize()
        assert torch.equal(other, eager), "eager decode after replay %d" % r
        cache.n = n
