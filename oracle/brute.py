"""Independent NumPy brute force for SWA(w,s).  TEST INFRASTRUCTURE ONLY.

Membership is decided by a predicate over every (t, i) pair rather than by the
two index ranges the C oracle walks:

    i in S_t  <=>  i <= t  and  (i <= s  or  i > t - (w - s))

(the query attends the first s tokens plus the most recent w - s, itself
included; paper.rainbus.top summary, "滑窗注意力 SWA(w, s)" section and method
steps, step 2; ai-blog.deepmagic.app, "他們測了什麼").  The softmax is a dense
fp64 matrix computation with -inf outside the mask.
"""
from __future__ import annotations

import numpy as np


def member(w: int, s: int, t: int, i: int) -> bool:
    """Is 1-based position i attended by the query at 1-based position t?"""
    return 1 <= i <= t and (i <= s or i > t - (w - s))


def mask(w: int, s: int, L: int) -> np.ndarray:
    """Boolean [L, L] matrix, M[t-1, i-1] = member(w, s, t, i)."""
    t = np.arange(1, L + 1)[:, None]
    i = np.arange(1, L + 1)[None, :]
    return (i <= t) & ((i <= s) | (i > t - (w - s)))


def prefill(Q, K, V, w: int, s: int, sink=None) -> np.ndarray:
    """Dense masked softmax in fp64.  Q [B,L,Hq,d], K/V [B,L,Hkv,d].

    sink: optional learned-sink logit per query head, taken here as one more
    key column that every row attends with score sink[h] and a zero value."""
    Q = np.asarray(Q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    B, L, Hq, d = Q.shape
    Hkv = K.shape[2]
    G = Hq // Hkv
    M = mask(w, s, L)
    O = np.empty_like(Q)
    for b in range(B):
        for h in range(Hq):
            q = Q[b, :, h, :]
            k = K[b, :, h // G, :]
            v = V[b, :, h // G, :]
            sc = (q @ k.T) / np.sqrt(d)
            sc = np.where(M, sc, -np.inf)
            if sink is not None:
                sc = np.concatenate([sc, np.full((L, 1), float(sink[h]))], axis=1)
                v = np.concatenate([v, np.zeros((1, d))], axis=0)
            sc = sc - sc.max(axis=1, keepdims=True)
            p = np.exp(sc)
            O[b, :, h, :] = (p @ v) / p.sum(axis=1, keepdims=True)
    return O


def retained_after(w: int, s: int, n: int) -> list:
    """Positions a cache of capacity w must still hold after n appends: the
    members of S_n, by the predicate."""
    return [i for i in range(1, n + 1) if member(w, s, n, i)]
