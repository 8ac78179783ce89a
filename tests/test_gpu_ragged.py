"""GPU parity of ragged and paged batches: swa_prefill_varlen, and the paged
cache (swa_paged_append, swa_paged_decode) with one position count per
sequence.  Every sequence must get what the oracle gives it alone:

- varlen prefill rows (and LSE) against oracle.prefill of each sequence;
- pool bytes after each append, bit-exact: slot j of sequence b (the
  oracle's slot map) sits in row j % page of page block_table[b, j // page]
  and must hold that position's row;
- paged decode against oracle.decode over S_n of each sequence; a sequence
  with n = 0 (its table row left at -1) gives 0.

Sequences draw their rows from their own seeds; lengths mix the empty
sequence, single rows, ragged tails and windows that wrap the ring.
Tolerances as in test_gpu_parity."""
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
    err = float(np.max(np.abs(got - ref))) if got.size else 0.0
    if dtype == torch.float32:
        scale = max(float(np.max(np.abs(ref))), 1e-30)
        assert err / scale <= F32_REL, "%s: rel err %.3g" % (what, err / scale)
    else:
        assert err <= BF16_ABS, "%s: abs err %.3g" % (what, err)


def cu_of(lens):
    return np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)


def _random_varlen(seed):
    """A seeded draw: 1..9 sequences of 0..700 rows, any group size, 0..40
    sinks, a window from one slot past the sinks to past the longest."""
    r = np.random.default_rng(8300 + seed)
    Hkv = int(r.integers(1, 4))
    s = int(r.choice([0, 1, 4, 4, 17, 40]))
    lens = [int(n) for n in r.integers(0, 701, size=int(r.integers(1, 10)))]
    lens[int(r.integers(0, len(lens)))] = max(lens[0], 1)  # at least one non-empty sequence
    dtype = torch.float32 if seed % 3 == 2 else torch.bfloat16
    return (dtype, int(r.choice([64, 128])), Hkv * int(r.choice([1, 2, 4, 8])), Hkv,
            int(r.integers(s + 1, s + 800)), s, lens)


@pytest.mark.parametrize("dtype,d,Hq,Hkv,w,s,lens", [
    (torch.bfloat16, 128, 32, 8, 128, 4, [1, 37, 300, 1000, 129, 0, 64]),
    (torch.bfloat16, 64, 8, 1, 64, 0, [200, 5, 0, 97]),
    (torch.float32, 64, 4, 2, 40, 5, [3, 150, 41]),
] + [_random_varlen(k) for k in range(6)])
def test_prefill_varlen(swa, dtype, d, Hq, Hkv, w, s, lens):
    bf = dtype == torch.bfloat16
    seqs = [synth.prefill_inputs(1, n, Hq, Hkv, d, seed=b, workload=61, bf16=bf, sink_outliers=4 if bf else 0)
            if n else None for b, n in enumerate(lens)]
    cu = cu_of(lens)
    pack = lambda i: np.concatenate([x[i][0] for x in seqs if x is not None], axis=0)
    Q, K, V = pack(0), pack(1), pack(2)
    O, lse = swa.prefill_varlen(dev(Q, dtype), dev(K, dtype), dev(V, dtype), dev(cu, torch.int32), max(lens),
                                w, s, lse=True)
    O, lse = host(O), host(lse)
    for b, x in enumerate(seqs):
        if x is None:
            continue
        Or, lr = oracle.prefill(*x, w, s, want_lse=True)
        rows = slice(cu[b], cu[b + 1])
        check(O[rows], Or[0], dtype, "sequence %d (L=%d)" % (b, lens[b]))
        assert np.max(np.abs(lse[:, rows] - lr[0])) < (2e-2 if bf else 1e-4)


def test_prefill_varlen_equals_batched(swa):
    """Equal lengths: varlen gives bit-identical output to the batched call."""
    B, L, Hq, Hkv, d, w, s = 3, 333, 16, 4, 128, 96, 4
    Q, K, V = synth.prefill_inputs(B, L, Hq, Hkv, d, seed=5, workload=63, bf16=True)
    q, k, v = (dev(x, torch.bfloat16) for x in (Q, K, V))
    ob = swa.prefill(q, k, v, w, s)
    ov = swa.prefill_varlen(q.reshape(B * L, Hq, d), k.reshape(B * L, Hkv, d), v.reshape(B * L, Hkv, d),
                            dev(cu_of([L] * B), torch.int32), L, w, s)
    assert torch.equal(ob.reshape(B * L, Hq, d), ov)


class Seq:
    """One sequence's rows (positions 1..cap) and how many are appended."""

    def __init__(self, b, Hkv, d, cap, workload):
        self.K, self.V = synth.history_rows(1, Hkv, d, cap, seed=b, workload=workload)
        self.n = 0


def paged_setup(swa, B, Hkv, d, w, s, page, extra_pages, empty, seed):
    pps = (w + page - 1) // page
    num_pages = B * pps + extra_pages
    rng = np.random.default_rng(seed)
    table = rng.permutation(num_pages)[:B * pps].reshape(B, pps).astype(np.int32)
    for b in empty:
        table[b] = -1  # never appended to: no pages
    cache = swa.PagedCache(B, Hkv, d, w, s, page, num_pages, block_table=dev(table, torch.int32))
    return cache, table


def append_step(swa, cache, seqs, counts):
    rows_k, rows_v = [], []
    for sq, c in zip(seqs, counts):
        rows_k.append(sq.K[0, sq.n:sq.n + c])
        rows_v.append(sq.V[0, sq.n:sq.n + c])
        sq.n += c
    K = np.concatenate(rows_k, axis=0)
    V = np.concatenate(rows_v, axis=0)
    cache.append(dev(K, torch.bfloat16), dev(V, torch.bfloat16), dev(cu_of(counts), torch.int32))


def check_pool(cache, table, seqs, w, s, page):
    """Every attended slot holds its position's rows.  Only the pages the
    table names are copied back: the pools come from torch.empty, and pages
    (or slots) never written hold arbitrary bits."""
    torch.cuda.synchronize()
    used = np.unique(table[table >= 0])
    where = {int(pg): i for i, pg in enumerate(used)}
    idx = torch.from_numpy(used.astype(np.int64)).cuda()
    # raw bf16 bit patterns: slots a page holds but no sequence has written
    # are never converted to floats
    kp = cache.k[idx].view(torch.int16).cpu().numpy()
    vp = cache.v[idx].view(torch.int16).cpu().numpy()

    def bits(x):  # bf16-exact fp32 -> its bf16 bit pattern
        return (np.ascontiguousarray(x, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16).view(np.int16)

    for b, sq in enumerate(seqs):
        for p in (oracle.attended(w, s, sq.n) if sq.n else []):
            j = oracle.slot(w, s, int(p))
            pg, r = where[int(table[b, j // page])], j % page
            np.testing.assert_array_equal(kp[pg, :, r], bits(sq.K[0, p - 1]), err_msg="b=%d K slot %d" % (b, j))
            np.testing.assert_array_equal(vp[pg, :, r], bits(sq.V[0, p - 1]), err_msg="b=%d V slot %d" % (b, j))


def check_decode(swa, cache, seqs, Hq, d, w, s, step, sink=None):
    B = len(seqs)
    q = np.stack([synth.query_rows(1, Hq, d, 1000 * step + b, workload=64)[0] for b in range(B)])
    sk = None if sink is None else torch.from_numpy(sink).cuda()
    got = host(cache.decode(dev(q, torch.bfloat16), sink_logit=sk))
    for b, sq in enumerate(seqs):
        if sq.n == 0:
            assert np.all(got[b] == 0.0), "empty sequence %d" % b
            continue
        S = np.asarray(oracle.attended(w, s, sq.n))
        ref = oracle.decode(q[b:b + 1], S, sq.K[:, S - 1], sq.V[:, S - 1], sq.n, w, s,
                            sink=None if sink is None else sink.astype(np.float64))
        check(got[b], ref[0], torch.bfloat16, "step %d sequence %d (n=%d)" % (step, b, sq.n))


def test_paged_append_and_decode(swa):
    B, Hq, Hkv, d, w, s, page = 6, 16, 4, 128, 100, 4, 32
    seqs = [Seq(b, Hkv, d, 400, workload=65) for b in range(B)]
    cache, table = paged_setup(swa, B, Hkv, d, w, s, page, extra_pages=5, empty=[0], seed=1)
    # bulk: nothing, one row, a partial window, exactly w, a wrapped ring, a short prompt
    append_step(swa, cache, seqs, [0, 1, 50, 100, 333, 7])
    check_pool(cache, table, seqs, w, s, page)
    check_decode(swa, cache, seqs, Hq, d, w, s, step=0)
    # decode steps in which only some sequences advance
    for step, counts in enumerate([[0, 1, 1, 1, 1, 1], [0, 0, 1, 1, 0, 1], [0, 1, 3, 1, 1, 0]], start=1):
        append_step(swa, cache, seqs, counts)
        check_decode(swa, cache, seqs, Hq, d, w, s, step=step)
    check_pool(cache, table, seqs, w, s, page)
    assert cache.n.cpu().tolist() == [sq.n for sq in seqs]


@pytest.mark.parametrize("d,G,page", [(64, 8, 64), (128, 1, 128)])
def test_paged_shapes(swa, d, G, page):
    B, Hkv, w, s = 5, 2, 256, 4
    Hq = G * Hkv
    seqs = [Seq(b, Hkv, d, 700, workload=66) for b in range(B)]
    cache, table = paged_setup(swa, B, Hkv, d, w, s, page, extra_pages=0, empty=[], seed=2)
    append_step(swa, cache, seqs, [700, 256, 255, 3, 32])
    check_pool(cache, table, seqs, w, s, page)
    check_decode(swa, cache, seqs, Hq, d, w, s, step=0)


@pytest.mark.parametrize("seed", range(6), ids=lambda k: "seed%d" % k)
def test_paged_random(swa, seed):
    """A seeded draw of batch, heads, head dim, window, sinks and page size;
    three append rounds of random row counts (some sequences idle, some
    wrapping the ring), the pool and the decode checked after each."""
    r = np.random.default_rng(8500 + seed)
    B, Hkv, d = int(r.integers(1, 13)), int(r.choice([1, 2, 4, 8])), int(r.choice([64, 128]))
    G = int(r.choice([1, 2, 4, 8]))
    s = int(r.choice([0, 1, 4, 4, 17]))
    w = int(r.integers(s + 1, s + 500))
    page = int(r.choice([32, 64, 128, 256]))  # pages hold a multiple of 32 slots
    cap = 3 * w + 8
    seqs = [Seq(b, Hkv, d, cap, workload=68) for b in range(B)]
    empty = [int(r.integers(0, B))] if B > 1 and seed % 2 else []
    cache, table = paged_setup(swa, B, Hkv, d, w, s, page, extra_pages=int(r.integers(0, 4)), empty=empty,
                               seed=seed)
    for step in range(3):
        counts = [0 if b in empty else int(r.integers(0, w + 1)) for b in range(B)]
        if sum(counts) == 0:  # every round appends something
            counts[next(b for b in range(B) if b not in empty)] = 1
        append_step(swa, cache, seqs, counts)
        check_pool(cache, table, seqs, w, s, page)
        check_decode(swa, cache, seqs, G * Hkv, d, w, s, step=step)
    assert cache.n.cpu().tolist() == [sq.n for sq in seqs]


@pytest.mark.parametrize("w,npos", [(256, 400), (576, 1200)])
def test_paged_eight_wave_workgroups(swa, w, npos):
    """32 sequences x 8 kv-heads at w = 256 and 576: each (sequence, kv-head)
    task gets a whole 8-wave workgroup in the paged decode too.  At w = 576 a
    sequence holds up to 18 chunks, so some waves have one more than others
    and request it with their first (ragged counts: partial last chunks)."""
    B, Hkv, d, s, page, G = 32, 8, 128, 4, 64, 4
    Hq = G * Hkv
    seqs = [Seq(b, Hkv, d, npos, workload=67) for b in range(B)]
    cache, table = paged_setup(swa, B, Hkv, d, w, s, page, extra_pages=3, empty=[5], seed=3)
    counts = [0 if b == 5 else (37 * b) % npos + 1 for b in range(B)]
    append_step(swa, cache, seqs, counts)
    check_pool(cache, table, seqs, w, s, page)
    check_decode(swa, cache, seqs, Hq, d, w, s, step=0)


def test_paged_split_and_sink(swa):
    """Long windows split over workgroups (partials merged), with ragged n
    and a learned sink."""
    B, Hq, Hkv, d, w, s, page = 2, 32, 8, 128, 4096, 4, 256
    seqs = [Seq(b, Hkv, d, 5000, workload=67) for b in range(B)]
    cache, table = paged_setup(swa, B, Hkv, d, w, s, page, extra_pages=3, empty=[], seed=3)
    assert cache.workspace_bytes(Hq) > 0
    append_step(swa, cache, seqs, [5000, 1234])
    check_decode(swa, cache, seqs, Hq, d, w, s, step=0)
    sink = np.random.default_rng(9).uniform(-2.0, 12.0, Hq).astype(np.float32)
    sink[0] = -np.inf
    check_decode(swa, cache, seqs, Hq, d, w, s, step=1, sink=sink)


def test_paged_batch16_w512(swa):
    """16 sequences x 8 kv-heads at SWA(512,4) (128 pairs, 16 chunks each):
    the plan that gives each pair one 8-wave workgroup with two chunks per
    wave, in the paged decode."""
    B, Hkv, d, w, s, page, G = 16, 8, 128, 512, 4, 64, 4
    seqs = [Seq(b, Hkv, d, 900, workload=69) for b in range(B)]
    cache, table = paged_setup(swa, B, Hkv, d, w, s, page, extra_pages=2, empty=[], seed=4)
    append_step(swa, cache, seqs, [600 + 19 * b for b in range(B)])
    check_pool(cache, table, seqs, w, s, page)
    check_decode(swa, cache, seqs, G * Hkv, d, w, s, step=0)


def test_paged_sixteen_wave_workgroups(swa):
    """3 sequences x 8 kv-heads at SWA(512,4), pages of 64: the paged decode
    takes one 16-wave workgroup per (sequence, kv-head), ragged n included."""
    B, Hkv, d, w, s, page, G = 3, 8, 128, 512, 4, 64, 4
    seqs = [Seq(b, Hkv, d, 1200, workload=70) for b in range(B)]
    cache, table = paged_setup(swa, B, Hkv, d, w, s, page, extra_pages=1, empty=[], seed=5)
    assert cache.workspace_bytes(G * Hkv) == 0
    append_step(swa, cache, seqs, [1200, 333, 40])
    check_pool(cache, table, seqs, w, s, page)
    check_decode(swa, cache, seqs, G * Hkv, d, w, s, step=0)


class FullSeq:
    """One sequence's Q, K, V at positions 1..cap, and how many are cached."""

    def __init__(self, b, cap, Hq, Hkv, d, workload):
        Q, K, V = synth.prefill_inputs(1, cap, Hq, Hkv, d, seed=b, workload=workload, bf16=True, sink_outliers=4)
        self.Q, self.K, self.V, self.n = Q, K, V, 0


def paged_chunk_case(swa, B, Hkv, G, d, w, s, page, hist, chunks, seed, out_dtype=torch.bfloat16, workload=71):
    """Sequences with hist[b] cached positions (appended in two rounds) each
    run a chunk of chunks[b] new positions through swa_paged_prefill_chunk;
    every chunk row against the oracle's prefill of its own sequence, the
    pools after the chunk's append, and the new position counts."""
    Hq = G * Hkv
    seqs = [FullSeq(b, hist[b] + chunks[b], Hq, Hkv, d, workload) for b in range(B)]
    cache, table = paged_setup(swa, B, Hkv, d, w, s, page, extra_pages=2, empty=[], seed=seed)
    for frac in (0.5, 1.0):  # the history in two rounds, so some rings wrap between them
        counts = [int(round(h * frac)) - sq.n for h, sq in zip(hist, seqs)]
        if sum(counts):
            append_step(swa, cache, seqs, counts)
    assert cache.n.cpu().tolist() == list(hist)
    cu = cu_of(chunks)
    pack = lambda name: np.concatenate([getattr(sq, name)[0, h:h + c] for sq, h, c in zip(seqs, hist, chunks)], 0)
    O, lse = cache.prefill_chunk(dev(pack("Q"), torch.bfloat16), dev(pack("K"), torch.bfloat16),
                                 dev(pack("V"), torch.bfloat16), dev(cu, torch.int32), max(chunks), lse=True,
                                 out_dtype=out_dtype)
    assert O.dtype == out_dtype
    O, lse = host(O), host(lse)
    for b, sq in enumerate(seqs):
        if not chunks[b]:
            continue
        ref, lref = oracle.prefill(sq.Q, sq.K, sq.V, w, s, want_lse=True)
        rows = slice(cu[b], cu[b + 1])
        check(O[rows], ref[0, hist[b]:], torch.bfloat16, "sequence %d (n=%d, C=%d)" % (b, hist[b], chunks[b]))
        assert np.max(np.abs(lse[:, rows] - lref[0, :, hist[b]:])) < 2e-2, "lse of sequence %d" % b
    for sq, c in zip(seqs, chunks):
        sq.n += c
    check_pool(cache, table, seqs, w, s, page)
    assert cache.n.cpu().tolist() == [sq.n for sq in seqs]


def test_paged_chunked_prefill(swa):
    """An empty cache (the chunk holds the sinks), n < s (sinks split between
    the pages and the chunk), a partial ring, an idle sequence, a wrapped
    ring with a chunk longer than the window."""
    paged_chunk_case(swa, 5, 2, 4, 128, 100, 4, 32, hist=[0, 3, 50, 100, 333], chunks=[70, 1, 64, 0, 200], seed=11)


def test_paged_chunked_prefill_full_windows(swa):
    """SWA(512,4), pages of 64: full rings at different heads, 300..512-row chunks."""
    paged_chunk_case(swa, 3, 2, 4, 128, 512, 4, 64, hist=[1000, 600, 77], chunks=[512, 300, 511], seed=12)


@pytest.mark.parametrize("d,G,page,out_dtype", [(64, 8, 128, torch.float32), (128, 1, 32, torch.bfloat16)])
def test_paged_chunked_prefill_shapes(swa, d, G, page, out_dtype):
    paged_chunk_case(swa, 4, 2, G, d, 256, 4, page, hist=[700, 5, 256, 0], chunks=[33, 129, 256, 1], seed=13,
                     out_dtype=out_dtype)


@pytest.mark.parametrize("seed", range(6), ids=lambda k: "seed%d" % k)
def test_paged_chunked_prefill_random(swa, seed):
    r = np.random.default_rng(8700 + seed)
    B, Hkv, d = int(r.integers(1, 7)), int(r.choice([1, 2, 4])), int(r.choice([64, 128]))
    G = int(r.choice([1, 2, 4, 8]))
    s = int(r.choice([0, 1, 4, 4, 17]))
    w = int(r.integers(s + 1, s + 400))
    page = int(r.choice([32, 64, 128, 256]))
    hist = [int(x) for x in r.integers(0, 2 * w + 2, size=B)]
    chunks = [int(x) for x in r.integers(0, w + 50, size=B)]
    chunks[int(r.integers(0, B))] = max(chunks[0], 1)  # at least one new row
    paged_chunk_case(swa, B, Hkv, G, d, w, s, page, hist, chunks, seed=seed,
                     out_dtype=torch.float32 if seed % 3 == 2 else torch.bfloat16)
