"""Pins for the fp64 oracle (CPU only).

Each check ties the oracle to something other than itself: worked examples the
pages print (tests/golden/), a library routine on the special cases the method
reduces to (torch's scaled_dot_product_attention in fp64), closed forms, and an
independent brute force over every (t, i) pair.  The mutant tests at the end
plant plausible mistakes in copies of the set definition and check that the
pins catch each one.
"""
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from oracle import brute
import synth


def _ranges(spec):
    out = []
    for part in spec.split(","):
        a, b = part.split("-")
        out.extend(range(int(a), int(b) + 1))
    return out


def _golden_sets(golden_dir):
    rows = []
    with open(os.path.join(golden_dir, "attended_sets.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            lhs, rhs = line.split("|")
            w, s, t = (int(x) for x in lhs.split())
            rows.append((w, s, t, _ranges(rhs.strip())))
    return rows


# --- attended sets -----------------------------------------------------------

def test_golden_attended_sets(golden_dir):
    rows = _golden_sets(golden_dir)
    assert len(rows) >= 10
    for w, s, t, expect in rows:
        got = oracle.attended(w, s, t).tolist()
        assert got == expect, (w, s, t)
        assert [i for i in range(max(1, t - 2 * w), t + 1) if brute.member(w, s, t, i)] == \
            [i for i in expect if i >= max(1, t - 2 * w)]


def test_attended_exhaustive_vs_predicate():
    for w in range(1, 17):
        for s in range(0, w):
            for t in range(1, 65):
                got = oracle.attended(w, s, t).tolist()
                want = [i for i in range(1, t + 1) if brute.member(w, s, t, i)]
                assert got == want, (w, s, t)
                assert len(got) == min(t, w)
                assert t in got  # a query always sees itself


def test_attended_rejects_bad_args():
    for w, s, t in [(4, 4, 1), (4, 5, 3), (0, 0, 1), (4, -1, 2), (4, 1, 0)]:
        with pytest.raises(ValueError):
            oracle.attended(w, s, t)


# --- outputs vs brute force and library routines ------------------------------

CASES = [  # B, L, Hq, Hkv, d, w, s
    (1, 37, 1, 1, 8, 8, 2),
    (2, 50, 4, 2, 16, 12, 4),
    (1, 70, 8, 2, 8, 16, 0),
    (1, 33, 2, 1, 4, 5, 4),
    (2, 41, 3, 3, 8, 64, 4),
]


def _inputs(B, L, Hq, Hkv, d, seed):
    return synth.prefill_inputs(B, L, Hq, Hkv, d, seed=seed, workload=101, bf16=False)


@pytest.mark.parametrize("case", CASES)
def test_prefill_vs_brute(case):
    B, L, Hq, Hkv, d, w, s = case
    Q, K, V = _inputs(B, L, Hq, Hkv, d, seed=sum(case))
    O = oracle.prefill(Q, K, V, w, s)
    Ob = brute.prefill(Q, K, V, w, s)
    assert np.max(np.abs(O - Ob)) < 1e-12


def _sdpa(Q, K, V, mask=None, causal=False):
    q = torch.from_numpy(np.asarray(Q, dtype=np.float64)).permute(0, 2, 1, 3)
    k = torch.from_numpy(np.asarray(K, dtype=np.float64)).permute(0, 2, 1, 3)
    v = torch.from_numpy(np.asarray(V, dtype=np.float64)).permute(0, 2, 1, 3)
    o = F.scaled_dot_product_attention(q, k, v, attn_mask=mask, is_causal=causal,
                                       enable_gqa=True)
    return o.permute(0, 2, 1, 3).numpy()


@pytest.mark.parametrize("Hq,Hkv", [(1, 1), (4, 1), (8, 2)])
def test_full_window_is_causal_softmax(Hq, Hkv):
    """w >= L: every earlier token is attended, whatever s is."""
    B, L, d = 2, 40, 16
    Q, K, V = _inputs(B, L, Hq, Hkv, d, seed=7 + Hq)
    ref = _sdpa(Q, K, V, causal=True)
    for w, s in [(L, 4), (L + 9, 0), (4096, 4)]:
        O = oracle.prefill(Q, K, V, w, s)
        assert np.max(np.abs(O - ref)) < 1e-12


def test_no_sinks_is_windowed_softmax():
    """s = 0 is the page's windowed softmax: i from max(1, t-w+1) to t."""
    B, L, Hq, Hkv, d, w = 1, 60, 4, 2, 8, 9
    Q, K, V = _inputs(B, L, Hq, Hkv, d, seed=3)
    band = torch.zeros(L, L, dtype=torch.bool)
    for t in range(1, L + 1):
        band[t - 1, max(1, t - w + 1) - 1:t] = True
    ref = _sdpa(Q, K, V, mask=band)
    O = oracle.prefill(Q, K, V, w, 0)
    assert np.max(np.abs(O - ref)) < 1e-12


def test_sink_mask_via_library():
    """General s: the library routine with the mask built from 'first s plus
    the most recent w-s' as explicit index ranges."""
    B, L, Hq, Hkv, d, w, s = 1, 90, 4, 1, 8, 20, 4
    Q, K, V = _inputs(B, L, Hq, Hkv, d, seed=5)
    m = torch.zeros(L, L, dtype=torch.bool)
    for t in range(1, L + 1):
        m[t - 1, :min(s, t)] = True
        m[t - 1, max(s + 1, t - (w - s) + 1) - 1:t] = True
    O = oracle.prefill(Q, K, V, w, s)
    assert np.max(np.abs(O - _sdpa(Q, K, V, mask=m))) < 1e-12


def test_sink_invariance_early_rows():
    """For t <= w the row does not depend on s: it is the causal row."""
    B, L, Hq, Hkv, d, w = 1, 48, 2, 1, 8, 16
    Q, K, V = _inputs(B, L, Hq, Hkv, d, seed=11)
    causal = _sdpa(Q, K, V, causal=True)
    for s in range(0, w):
        O = oracle.prefill(Q, K, V, w, s)
        assert np.max(np.abs(O[:, :w] - causal[:, :w])) < 1e-12
        if s:  # beyond the window the sinks do change the rows
            O0 = oracle.prefill(Q, K, V, w, 0)
            assert np.max(np.abs(O[:, w:] - O0[:, w:])) > 1e-6


def test_first_row_is_first_value():
    Q, K, V = _inputs(2, 10, 4, 2, 8, seed=2)
    O = oracle.prefill(Q, K, V, 5, 2)
    np.testing.assert_array_equal(O[:, 0], np.repeat(V[:, 0].astype(np.float64), 2, axis=1))


def test_one_hot_probe_reveals_set():
    """Q = 0 gives equal weights, so with one-hot V rows O[t, c] = 1/|S_t| iff
    position block+c+1 is attended, exactly."""
    L, d, w, s = 64, 32, 10, 3
    for block in (0, 32):
        Q, K, V = synth.one_hot_probe(1, L, 1, 1, d, block)
        O = oracle.prefill(Q, K, V, w, s)
        for t in range(1, L + 1):
            S = set(oracle.attended(w, s, t).tolist())
            for c in range(d):
                i = block + c + 1
                want = 1.0 / min(t, w) if i in S else 0.0
                assert O[0, t - 1, 0, c] == want


def test_constant_values():
    Q, K, _ = _inputs(1, 30, 2, 1, 8, seed=4)
    V = np.full_like(K, 0.375)
    O = oracle.prefill(Q, K, V, 7, 2)
    assert np.max(np.abs(O - 0.375)) < 1e-15


def test_eviction_invariance():
    """Changing keys/values outside S_t leaves row t unchanged (bit-exact)."""
    L, w, s = 40, 10, 2
    Q, K, V = _inputs(1, L, 2, 1, 8, seed=9)
    O = oracle.prefill(Q, K, V, w, s)
    t = L
    evicted = [i for i in range(1, t + 1) if i not in set(oracle.attended(w, s, t).tolist())]
    K2, V2 = K.copy(), V.copy()
    for i in evicted:
        K2[:, i - 1] = 1e4
        V2[:, i - 1] = -1e4
    O2 = oracle.prefill(Q, K2, V2, w, s)
    np.testing.assert_array_equal(O[:, t - 1], O2[:, t - 1])


def test_lse_matches_dense():
    B, L, Hq, Hkv, d, w, s = 1, 30, 2, 1, 8, 7, 2
    Q, K, V = _inputs(B, L, Hq, Hkv, d, seed=13)
    _, lse = oracle.prefill(Q, K, V, w, s, want_lse=True)
    M = brute.mask(w, s, L)
    for h in range(Hq):
        sc = Q[0, :, h].astype(np.float64) @ K[0, :, 0].astype(np.float64).T / np.sqrt(d)
        sc = np.where(M, sc, -np.inf)
        ref = np.log(np.exp(sc).sum(axis=1))
        assert np.max(np.abs(lse[0, h] - ref)) < 1e-12


def test_bf16_inputs_are_exact():
    Q, K, V = synth.prefill_inputs(1, 16, 2, 1, 8, seed=1, workload=1, bf16=True)
    for a in (Q, K, V):
        assert np.all((a.view(np.uint32) & 0xFFFF) == 0)


# --- decode -----------------------------------------------------------------

def test_decode_equals_prefill_row():
    B, L, Hq, Hkv, d, w, s = 2, 45, 4, 2, 8, 12, 3
    Q, K, V = _inputs(B, L, Hq, Hkv, d, seed=21)
    O = oracle.prefill(Q, K, V, w, s)
    for n in (1, 3, 12, 13, 30, 45):
        full = np.arange(1, n + 1)
        Od = oracle.decode(Q[:, n - 1], full, K[:, :n], V[:, :n], n, w, s)
        np.testing.assert_array_equal(Od, O[:, n - 1])
        # only the attended rows supplied (any superset works)
        Sn = oracle.attended(w, s, n)
        Od2 = oracle.decode(Q[:, n - 1], Sn, K[:, Sn - 1], V[:, Sn - 1], n, w, s)
        np.testing.assert_array_equal(Od2, O[:, n - 1])
        if n > w:  # drop one attended row: the oracle refuses
            keep = Sn[1:]
            with pytest.raises(KeyError):
                oracle.decode(Q[:, n - 1], keep, K[:, keep - 1], V[:, keep - 1], n, w, s)


# --- the constant-size cache ------------------------------------------------

def test_ring_cache_holds_attended_set():
    for w in range(1, 13):
        for s in range(0, w):
            rc = oracle.RingCache(w, s)
            for n in range(1, 50):
                j = rc.append(n)
                assert j == oracle.slot(w, s, n)
                ret = rc.retained()
                assert ret == brute.retained_after(w, s, n)
                assert ret == oracle.attended(w, s, n).tolist()
                occupied = sorted(k for k in range(w) if rc.held[k])
                assert occupied == list(range(min(n, w)))
                for k in range(w):  # payload follows its position
                    if rc.held[k]:
                        assert rc.rows[k] == rc.held[k]


def test_ring_golden_example():
    """SWA(64,4) after 200 tokens keeps positions 1-4 and 141-200: 4 sinks and
    60 recent positions (ai-blog.deepmagic.app, "他們測了什麼")."""
    rc = oracle.RingCache(64, 4)
    for _ in range(200):
        rc.append()
    assert rc.retained() == list(range(1, 5)) + list(range(141, 201))


def test_kv_bytes_per_token_example(golden_dir):
    """The per-token KV footprint accounting used for the Qwen3-4B-shaped
    workload: 36 layers x 8 KV heads x 128 dims x (K, V) x 2 bytes."""
    import json
    with open(os.path.join(golden_dir, "kv_bytes.json")) as f:
        g = json.load(f)
    per_tok = g["layers"] * g["kv_heads"] * g["head_dim"] * 2 * g["bytes_per_elem"]
    assert per_tok == g["bytes_per_token"]
    assert per_tok / 1024 == g["kib_per_token"]
    assert abs(g["tokens"] * per_tok / 2**30 - g["gib_at_tokens"]) < 0.05


# --- the pins catch planted mistakes ------------------------------------------

MUTANTS = {
    "window excludes sinks": lambda w, s, t, i: 1 <= i <= t and (i <= s or i > t - w),
    "window off by one": lambda w, s, t, i: 1 <= i <= t and (i <= s or i >= t - (w - s)),
    "no sinks": lambda w, s, t, i: 1 <= i <= t and i > t - (w - s),
    "query excludes itself": lambda w, s, t, i: 1 <= i < t and (i <= s or i > t - (w - s) - 1),
    "sinks not capped by t": lambda w, s, t, i: (i <= s) or (1 <= i <= t and i > t - (w - s)),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant_sets(name, golden_dir):
    pred = MUTANTS[name]
    caught = False
    for w, s, t, expect in _golden_sets(golden_dir):
        got = [i for i in range(1, t + 1 + s) if pred(w, s, t, i)]
        if got != expect:
            caught = True
    for w in range(2, 9):
        for s in range(0, w):
            for t in range(1, 20):
                got = [i for i in range(1, t + 1 + s) if pred(w, s, t, i)]
                if len(got) != min(t, w):
                    caught = True
    assert caught, name


def test_pins_catch_mutant_arithmetic():
    """Wrong scale, a transposed score, or the wrong GQA head map each move the
    outputs away from the library routine used in test_full_window_is_causal_softmax."""
    B, L, Hq, Hkv, d = 1, 20, 4, 2, 8
    Q, K, V = _inputs(B, L, Hq, Hkv, d, seed=17)
    ref = _sdpa(Q, K, V, causal=True)
    assert np.max(np.abs(oracle.prefill(Q, K, V, L, 0) - ref)) < 1e-12
    # scale 1/d instead of 1/sqrt(d): feed Q scaled by 1/sqrt(d)
    assert np.max(np.abs(oracle.prefill(Q / np.sqrt(d), K, V, L, 0) - ref)) > 1e-3
    # K and V swapped
    assert np.max(np.abs(oracle.prefill(Q, V, K, L, 0) - ref)) > 1e-3
    # heads interleaved (h % Hkv) rather than grouped (h // G): the library
    # routine given explicitly tiled K/V heads computes that wrong mapping
    G = Hq // Hkv
    Kt = np.tile(K, (1, 1, G, 1))
    Vt = np.tile(V, (1, 1, G, 1))
    wrong = _sdpa(Q, Kt, Vt, causal=True)
    assert np.max(np.abs(wrong - ref)) > 1e-3
    assert np.max(np.abs(oracle.prefill(Q, K, V, L, 0) - wrong)) > 1e-3


# --- learned-sink variant --------------------------------------------------------

def _lsink_inputs(seed, B=2, L=60, Hq=4, Hkv=2, d=16):
    rng = np.random.default_rng(seed)
    Q = rng.standard_normal((B, L, Hq, d)).astype(np.float32)
    K = rng.standard_normal((B, L, Hkv, d)).astype(np.float32)
    V = rng.standard_normal((B, L, Hkv, d)).astype(np.float32)
    return Q, K, V


def test_lsink_absent_is_plain():
    """A logit of -inf adds exp(-inf) = 0: bit-identical to the plain oracle."""
    Q, K, V = _lsink_inputs(1)
    a, la = oracle.prefill(Q, K, V, 16, 4, want_lse=True)
    b, lb = oracle.prefill(Q, K, V, 16, 4, want_lse=True, sink=np.full(4, -np.inf))
    assert np.array_equal(a, b) and np.array_equal(la, lb)


@pytest.mark.parametrize("w,s", [(16, 4), (8, 0), (100, 4), (10, 9)])
def test_lsink_matches_extra_key_brute_force(w, s):
    """The C oracle against a dense brute force that models the sink as one
    extra key column with a zero value."""
    Q, K, V = _lsink_inputs(w + s)
    sink = np.array([-1.0, 0.5, 2.0, 6.0])
    np.testing.assert_allclose(oracle.prefill(Q, K, V, w, s, sink=sink),
                               brute.prefill(Q, K, V, w, s, sink=sink), rtol=0, atol=1e-12)


def test_lsink_identity_with_plain_lse():
    """Adding e^b to the denominator scales each row by 1/(1 + e^(b - LSE))
    and moves the log-sum-exp to logaddexp(LSE, b); checked against the
    plain oracle's outputs for logits far below, near and far above LSE."""
    Q, K, V = _lsink_inputs(7)
    O, lse = oracle.prefill(Q, K, V, 20, 4, want_lse=True)
    for sink in (np.array([-30.0, -5.0, 0.0, 3.0]), np.array([2.0, 4.0, 8.0, 40.0])):
        Os, ls = oracle.prefill(Q, K, V, 20, 4, want_lse=True, sink=sink)
        b = sink[None, :, None]                                  # [1, Hq, 1] against lse [B, Hq, L]
        scale = 1.0 / (1.0 + np.exp(b - lse))                    # [B, Hq, L]
        np.testing.assert_allclose(Os, O * scale.transpose(0, 2, 1)[..., None], rtol=1e-12, atol=1e-15)
        np.testing.assert_allclose(ls, np.logaddexp(lse, b), rtol=1e-13, atol=1e-12)


def test_lsink_closed_form_zero_query():
    """Q = 0 and V = 1: every attended score is 0, so x_t = |S_t| / (|S_t| + e^b)."""
    B, L, Hq, Hkv, d, w, s = 1, 50, 2, 1, 8, 12, 3
    Q = np.zeros((B, L, Hq, d), np.float32)
    K = np.random.default_rng(3).standard_normal((B, L, Hkv, d)).astype(np.float32)
    V = np.ones((B, L, Hkv, d), np.float32)
    sink = np.array([0.0, np.log(5.0)])
    O = oracle.prefill(Q, K, V, w, s, sink=sink)
    for t in range(1, L + 1):
        n = min(t, w)
        for h in range(Hq):
            np.testing.assert_allclose(O[0, t - 1, h], n / (n + np.exp(sink[h])), rtol=1e-14)


def test_lsink_decode_equals_prefill_row():
    Q, K, V = _lsink_inputs(11, L=40)
    sink = np.array([1.0, -2.0, 3.5, 0.25])
    O = oracle.prefill(Q, K, V, 10, 2, sink=sink)
    for t in (1, 9, 10, 11, 40):
        o = oracle.decode(Q[:, t - 1], np.arange(1, t + 1), K[:, :t], V[:, :t], t, 10, 2, sink=sink)
        np.testing.assert_allclose(o, O[:, t - 1], rtol=0, atol=1e-13)


# --- fp8 (OCP E4M3) cache codes ---------------------------------------------------

from oracle import fp8  # noqa: E402


def test_e4m3_points_of_the_format():
    """Values the format fixes: 1.0 = 0.0111.000, the largest finite 448 =
    0.1111.110, the smallest normal 2^-6, the smallest subnormal 2^-9, the
    NaN code S.1111.111, a negative code."""
    assert fp8.decode(0x38) == 1.0
    assert fp8.decode(0x7E) == 448.0
    assert fp8.decode(0x08) == 2.0 ** -6
    assert fp8.decode(0x01) == 2.0 ** -9
    assert fp8.decode(0x07) == 7 * 2.0 ** -9
    assert np.isnan(fp8.decode(0x7F)) and np.isnan(fp8.decode(0xFF))
    assert fp8.decode(0xB8) == -1.0 and fp8.decode(0x80) == 0.0 and np.signbit(fp8.decode(0x80))
    assert fp8.encode(448.0) == 0x7E and fp8.encode(1.0) == 0x38 and fp8.encode(-2.0 ** -9) == 0x81


def test_e4m3_round_trip_and_order():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    v = fp8.decode(codes)
    assert np.array_equal(fp8.encode(v), codes)              # every finite code, both zeros
    pos = fp8.decode(np.arange(0x7F))
    assert np.all(np.diff(pos) > 0)                          # codes 0..0x7E are increasing
    assert len(np.unique(np.abs(v))) == 127


def test_e4m3_nearest_ties_to_even():
    """Midpoints round to the even mantissa; anything else to the nearer value."""
    pos = fp8.decode(np.arange(0x7F))
    mids = (pos[:-1] + pos[1:]) / 2
    got = fp8.encode(mids)
    want = np.where(np.arange(0x7E) % 2 == 0, np.arange(0x7E), np.arange(1, 0x7F))
    assert np.array_equal(got, want.astype(np.uint8))
    eps = (pos[1:] - pos[:-1]) * 1e-3
    assert np.array_equal(fp8.encode(mids - eps), np.arange(0x7E, dtype=np.uint8))
    assert np.array_equal(fp8.encode(mids + eps), np.arange(1, 0x7F, dtype=np.uint8))


def test_e4m3_quantize_saturates_and_dequantizes_within_half_ulp():
    x = np.array([0.3, -5.0, 1000.0, -1e6, 2.4, 7e-4], np.float32)
    q = fp8.quantize(x, 2.0)
    assert q[2] == 0x7E and q[3] == 0xFE                    # clamped to +-448
    d = fp8.dequantize(q, 2.0)
    inside = np.abs(x / 2.0) <= 448
    rel = np.abs(d[inside] - x[inside]) / np.maximum(np.abs(x[inside]), 2.0 * 2.0 ** -6)
    assert np.all(rel <= 2.0 ** -4 + 1e-12)                  # half an ulp of a 3-bit mantissa


def test_batch_row_history_is_keyed_by_row_and_prefix_stable():
    """The per-row generator the batch-16 full-causal checks use: a row is
    reproducible alone, rows differ, a longer history extends a shorter one,
    and values are bf16-exact N(0,1) draws."""
    a_k, a_v = synth.batch_row_history(3, 2, 8, 40000, workload=9)
    b_k, b_v = synth.batch_row_history(3, 2, 8, 20000, workload=9)
    c_k, _ = synth.batch_row_history(4, 2, 8, 20000, workload=9)
    assert a_k.shape == (1, 40000, 2, 8) and b_k.shape == (1, 20000, 2, 8)
    np.testing.assert_array_equal(a_k[:, :20000], b_k)
    np.testing.assert_array_equal(a_v[:, :20000], b_v)
    assert not np.array_equal(b_k, c_k)
    np.testing.assert_array_equal(synth.bf16_round(a_k), a_k)
    assert abs(float(a_k.std()) - 1.0) < 0.05 and abs(float(a_k.mean())) < 0.05
