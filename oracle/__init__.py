"""fp64 CPU oracle for SWA(w,s) attention with attention sinks.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  It shares no code
with the HIP library in ``sliding_window_sink_amd`` and never imports it.

Contents
--------
* ``prefill`` / ``decode`` -- thin ctypes wrappers over ``swa_oracle.c`` (plain
  fp64 masked softmax over the attended set S_t; see that file's header for the
  passages it follows).
* ``attended`` -- the attended set S_t as the C oracle enumerates it.
* ``slot`` / ``RingCache`` -- the constant-size cache: s pinned sink slots plus
  a (w-s)-slot ring, simulated one appended position at a time.  The pages say
  only that the cache becomes constant-size, capped at the window, by an
  eviction policy that keeps the sinks and the recent tokens
  (paper.rainbus.top summary, "KV 缓存" background section; 163.com article,
  "研究方法"; ai-blog.deepmagic.app, "他們測了什麼").  The slot formula used
  here is one reading of that policy: position p <= s lives in slot
  p-1 for good; position p > s lives in slot s + ((p-s-1) mod (w-s)), so a new
  position overwrites exactly the one that just left the window.
* ``brute`` -- an independent NumPy brute force (dense predicate mask).

Pins: every function here is checked by ``tests/test_oracle.py`` against
closed forms, library routines on special cases, worked examples printed on the
pages (``tests/golden/``) and brute-force enumeration.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "swa_oracle.c")
_LIB = os.path.join(_HERE, "libswa_oracle.so")
_lib = None


def build(force: bool = False) -> str:
    """Compile swa_oracle.c with gcc into oracle/libswa_oracle.so."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(
            ["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-fno-fast-math",
             "-o", tmp, _SRC, "-lm", "-lpthread"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        build()
        lib = ctypes.CDLL(_LIB)
        f32p = ctypes.POINTER(ctypes.c_float)
        f64p = ctypes.POINTER(ctypes.c_double)
        i64p = ctypes.POINTER(ctypes.c_int64)
        lib.swa_oracle_attended.argtypes = [ctypes.c_int64] * 3 + [i64p]
        lib.swa_oracle_attended.restype = ctypes.c_int64
        lib.swa_oracle_prefill.argtypes = [f32p, f32p, f32p, f64p, f64p] + [ctypes.c_int] * 5 + [
            ctypes.c_int64, ctypes.c_int64, ctypes.c_int]
        lib.swa_oracle_prefill.restype = ctypes.c_int
        lib.swa_oracle_decode.argtypes = [f32p, i64p, ctypes.c_int64, f32p, f32p, f64p, f64p] + [
            ctypes.c_int] * 4 + [ctypes.c_int64] * 3 + [ctypes.c_int]
        lib.swa_oracle_decode.restype = ctypes.c_int
        lib.swa_oracle_prefill_lsink.argtypes = [f32p, f32p, f32p, f64p, f64p, f64p] + [ctypes.c_int] * 5 + [
            ctypes.c_int64, ctypes.c_int64, ctypes.c_int]
        lib.swa_oracle_prefill_lsink.restype = ctypes.c_int
        lib.swa_oracle_decode_lsink.argtypes = [f32p, i64p, ctypes.c_int64, f32p, f32p, f64p, f64p, f64p] + [
            ctypes.c_int] * 4 + [ctypes.c_int64] * 3 + [ctypes.c_int]
        lib.swa_oracle_decode_lsink.restype = ctypes.c_int
        _lib = lib
    return _lib


def default_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def _f32(a):
    a = np.ascontiguousarray(a, dtype=np.float32)
    return a, a.ctypes.data_as(ctypes.POINTER(ctypes.c_float))


def attended(w: int, s: int, t: int) -> np.ndarray:
    """1-based members of S_t, increasing, as the C oracle enumerates them."""
    lib = _load()
    out = np.empty(max(int(t), 1), dtype=np.int64)
    n = lib.swa_oracle_attended(int(w), int(s), int(t),
                                out.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)))
    if n < 0:
        raise ValueError("invalid (w, s, t) = (%d, %d, %d)" % (w, s, t))
    return out[:n].copy()


def _sink_arg(sink, Hq):
    """Learned-sink logits: None, or Hq values (fp64 copy kept alive by the caller)."""
    if sink is None:
        return None, None
    a = np.ascontiguousarray(sink, dtype=np.float64).reshape(-1)
    if a.shape != (Hq,):
        raise ValueError("sink must hold one logit per query head")
    return a, a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def prefill(Q, K, V, w: int, s: int, want_lse: bool = False, threads: int | None = None, sink=None):
    """O[b,t,h] = softmax over S_t of q.k/sqrt(d), times V, in fp64.

    Q: [B, L, Hq, d]; K, V: [B, L, Hkv, d] (any float dtype; read as fp32).
    sink: optional learned-sink logit per query head (an extra e^sink in the
    denominator, no value).  Returns O [B, L, Hq, d] float64 (and lse
    [B, Hq, L] if asked).
    """
    lib = _load()
    Q, qp = _f32(Q)
    K, kp = _f32(K)
    V, vp = _f32(V)
    B, L, Hq, d = Q.shape
    Hkv = K.shape[2]
    if K.shape != (B, L, Hkv, d) or V.shape != K.shape:
        raise ValueError("shape mismatch")
    O = np.empty((B, L, Hq, d), dtype=np.float64)
    lse = np.empty((B, Hq, L), dtype=np.float64) if want_lse else None
    sk, skp = _sink_arg(sink, Hq)
    rc = lib.swa_oracle_prefill_lsink(
        qp, kp, vp, O.ctypes.data_as(ctypes.POINTER(ctypes.c_double)),
        lse.ctypes.data_as(ctypes.POINTER(ctypes.c_double)) if want_lse else None, skp,
        B, L, Hq, Hkv, d, int(w), int(s), threads or default_threads())
    if rc != 0:
        raise ValueError("oracle prefill failed (%d)" % rc)
    return (O, lse) if want_lse else O


def decode(Q, pos, Kh, Vh, n: int, w: int, s: int, want_lse: bool = False,
           threads: int | None = None, sink=None):
    """Output of the query rows Q [B, Hq, d] at 1-based position n.

    The history is given as rows Kh, Vh [B, npos, Hkv, d] for the strictly
    increasing 1-based positions ``pos``; it must include every member of S_n
    (extra positions are ignored).  Raises KeyError if one is missing.
    """
    lib = _load()
    Q, qp = _f32(Q)
    Kh, kp = _f32(Kh)
    Vh, vp = _f32(Vh)
    pos = np.ascontiguousarray(pos, dtype=np.int64)
    B, Hq, d = Q.shape
    npos, Hkv = Kh.shape[1], Kh.shape[2]
    if Kh.shape != (B, npos, Hkv, d) or Vh.shape != Kh.shape or pos.shape != (npos,):
        raise ValueError("shape mismatch")
    O = np.empty((B, Hq, d), dtype=np.float64)
    lse = np.empty((B, Hq), dtype=np.float64) if want_lse else None
    sk, skp = _sink_arg(sink, Hq)
    rc = lib.swa_oracle_decode_lsink(
        qp, pos.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), npos, kp, vp,
        O.ctypes.data_as(ctypes.POINTER(ctypes.c_double)),
        lse.ctypes.data_as(ctypes.POINTER(ctypes.c_double)) if want_lse else None, skp,
        B, Hq, Hkv, d, int(n), int(w), int(s), threads or default_threads())
    if rc == -3:
        raise KeyError("history lacks a member of S_n")
    if rc != 0:
        raise ValueError("oracle decode failed (%d)" % rc)
    return (O, lse) if want_lse else O


# --- the constant-size cache ------------------------------------------------

def slot(w: int, s: int, p: int) -> int:
    """0-based cache slot that 1-based position p is written to."""
    if p < 1 or s < 0 or w <= s:
        raise ValueError("invalid (w, s, p)")
    if p <= s:
        return p - 1
    return s + (p - s - 1) % (w - s)


class RingCache:
    """The cache of one sequence, one appended position at a time.

    ``held[j]`` is the 1-based position whose row sits in slot j (0 if empty).
    Rows are arbitrary payloads (e.g. numpy vectors) kept beside it.
    """

    def __init__(self, w: int, s: int):
        if s < 0 or w <= s:
            raise ValueError("need 0 <= s < w")
        self.w, self.s, self.n = w, s, 0
        self.held = [0] * w
        self.rows = [None] * w

    def append(self, row=None):
        self.n += 1
        j = slot(self.w, self.s, self.n)
        self.held[j] = self.n
        self.rows[j] = row
        return j

    def retained(self) -> list:
        return sorted(p for p in self.held if p)


from . import brute  # noqa: E402  (re-export)

__all__ = ["build", "attended", "prefill", "decode", "slot", "RingCache", "brute",
           "default_threads"]
