"""Seeded synthetic inputs shared by the tests, the bench and the smoke check.

This module holds no attention arithmetic: it only draws numbers.  Both the
oracle and the HIP library receive the arrays it returns; neither imports it.

Recipe
------
* Every draw comes from ``numpy.random.default_rng(key)`` with an integer key
  tuple ``(seed, workload, layer, step, tensor)`` so any tensor can be
  regenerated on its own, without replaying the ones before it.
* Values are i.i.d. N(0, 1) in fp32.  For bf16 workloads they are rounded to
  the nearest bf16 (ties to even) on the host, so the oracle and the device
  read bit-identical values.
* Sink outliers: one direction g ~ N(0, I_d), normalised, is drawn per seed and
  shared by every (batch, kv-head); the keys at the first ``n_sinks`` positions
  get ``scale * sqrt(d) * g_hat`` added (then bf16 rounding), which makes the
  sink logits large for queries aligned with g_hat.
* Per-position decode rows use ``step = position`` so a long stream can be
  regenerated position by position.
"""
from __future__ import annotations

import numpy as np

# tensor tags inside the rng key
_Q, _K, _V, _DIR = 0, 1, 2, 3


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to the nearest bf16 (ties to even); returns fp32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16) << 16
    out = (r & 0xFFFFFFFF).astype(np.uint32).view(np.float32)
    nan = np.isnan(x)
    if nan.any():
        out = out.copy()
        out[nan] = np.nan
    return out.reshape(x.shape)


def normal(shape, key, bf16: bool) -> np.ndarray:
    a = np.random.default_rng(list(key)).standard_normal(shape, dtype=np.float32)
    return bf16_round(a) if bf16 else a


def sink_direction(d: int, seed: int) -> np.ndarray:
    g = np.random.default_rng([seed, _DIR]).standard_normal(d).astype(np.float64)
    return (g / np.linalg.norm(g)).astype(np.float32)


def add_sink_outliers(K: np.ndarray, first_pos: int, n_sinks: int, scale: float,
                      seed: int, bf16: bool) -> np.ndarray:
    """K [B, P, Hkv, d] holds positions first_pos..first_pos+P-1 (1-based);
    keys at positions <= n_sinks get the shared outlier added."""
    d = K.shape[-1]
    g = sink_direction(d, seed) * np.float32(scale * np.sqrt(d))
    K = K.copy()
    for j in range(K.shape[1]):
        if first_pos + j <= n_sinks:
            K[:, j] = K[:, j] + g
    return bf16_round(K) if bf16 else K


def prefill_inputs(B, L, Hq, Hkv, d, *, seed=0, workload=1, layer=0, bf16=True,
                   sink_outliers=0, outlier_scale=8.0):
    """Q [B,L,Hq,d], K, V [B,L,Hkv,d] as fp32 arrays (bf16-exact if bf16)."""
    Q = normal((B, L, Hq, d), (seed, workload, layer, 0, _Q), bf16)
    K = normal((B, L, Hkv, d), (seed, workload, layer, 0, _K), bf16)
    V = normal((B, L, Hkv, d), (seed, workload, layer, 0, _V), bf16)
    if sink_outliers:
        K = add_sink_outliers(K, 1, sink_outliers, outlier_scale, seed, bf16)
    return Q, K, V


def position_rows(B, Hkv, d, positions, *, seed=0, workload=3, layer=0, bf16=True,
                  sink_outliers=0, outlier_scale=8.0):
    """K, V rows [B, len(positions), Hkv, d] for the given 1-based positions,
    each drawn from its own key so any position can be regenerated alone."""
    positions = list(positions)
    K = np.empty((B, len(positions), Hkv, d), dtype=np.float32)
    V = np.empty_like(K)
    for j, p in enumerate(positions):
        K[:, j] = normal((B, Hkv, d), (seed, workload, layer, int(p), _K), bf16)
        V[:, j] = normal((B, Hkv, d), (seed, workload, layer, int(p), _V), bf16)
        if sink_outliers and p <= sink_outliers:
            K[:, j:j + 1] = add_sink_outliers(K[:, j:j + 1], int(p), sink_outliers,
                                              outlier_scale, seed, bf16)
    return K, V


def history_rows(B, Hkv, d, n, *, seed=0, workload=4, layer=0, bf16=True):
    """K, V rows [B, n, Hkv, d] for positions 1..n drawn in bulk from one key
    each (for full-history caches too long to draw position by position)."""
    K = normal((B, n, Hkv, d), (seed, workload, layer, 0, _K, 1), bf16)
    V = normal((B, n, Hkv, d), (seed, workload, layer, 0, _V, 1), bf16)
    return K, V


ROW_BLOCK = 1 << 14  # positions per key in batch_row_history


def batch_row_history(b, Hkv, d, n, *, seed=0, workload=4, layer=0, bf16=True):
    """K, V rows [1, n, Hkv, d] for positions 1..n of batch row b alone, drawn
    in blocks of ROW_BLOCK positions with the key (seed, workload, layer,
    block, tensor, 2, b): one row of a wide batch can be regenerated (and
    checked) without drawing the others, and a longer n extends a shorter
    one."""
    nb = (n + ROW_BLOCK - 1) // ROW_BLOCK
    K = np.empty((1, nb * ROW_BLOCK, Hkv, d), dtype=np.float32)
    V = np.empty_like(K)
    for j in range(nb):
        sl = slice(j * ROW_BLOCK, (j + 1) * ROW_BLOCK)
        K[0, sl] = normal((ROW_BLOCK, Hkv, d), (seed, workload, layer, j, _K, 2, b), bf16)
        V[0, sl] = normal((ROW_BLOCK, Hkv, d), (seed, workload, layer, j, _V, 2, b), bf16)
    return K[:, :n], V[:, :n]


def prompt_rows(B, Hkv, d, first, count, **kw):
    """Rows for positions first..first+count-1 (one key per position)."""
    return position_rows(B, Hkv, d, range(first, first + count), **kw)


def query_rows(B, Hq, d, position, *, seed=0, workload=3, layer=0, bf16=True):
    """The decode query [B, Hq, d] at a 1-based position."""
    return normal((B, Hq, d), (seed, workload, layer, int(position), _Q), bf16)


def one_hot_probe(B, L, Hq, Hkv, d, block: int):
    """Q = 0 and V[:, i] = e_{(i - block) } for i in [block, block + d) (zero
    elsewhere): with a zero query every attended row gets equal weight, so
    O[t, c] = 1/|S_t| exactly when position block+c+1 is attended by t, else 0.
    K is random (it cannot matter when Q = 0)."""
    Q = np.zeros((B, L, Hq, d), dtype=np.float32)
    K = normal((B, L, Hkv, d), (0, 99, 0, block, _K), True)
    V = np.zeros((B, L, Hkv, d), dtype=np.float32)
    for c in range(d):
        i = block + c
        if i < L:
            V[:, i, :, c] = 1.0
    return Q, K, V
