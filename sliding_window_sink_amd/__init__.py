"""libswa: SWA(w,s) sliding-window attention with attention sinks on MI355X.

A thin ctypes binding over the C ABI declared in include/swa.h.  It only
marshals arguments: tensors become device pointers, the current torch stream
becomes the HIP stream, errors become exceptions.  Every step of the
computation runs in the HIP kernels of libswa.so; there is no fallback, and
importing this package raises if the library has not been built
(``python sliding_window_sink_amd/build.py``).

    import torch, sliding_window_sink_amd as swa
    O = swa.prefill(Q, K, V, w=512, s=4)                 # [B, L, Hq, d]
    cache = swa.Cache(B, Hkv, d, w=512, s=4, dtype=torch.bfloat16)
    cache.append(K_new, V_new)                            # [B, n_new, Hkv, d]
    o = cache.decode(q)                                   # [B, Hq, d]
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libswa.so")

SWA_OK, SWA_ERR_INVALID_ARG, SWA_ERR_UNSUPPORTED, SWA_ERR_HIP, SWA_ERR_STATE = range(5)
SWA_F32, SWA_BF16, SWA_FP8_E4M3 = 0, 1, 2
STATUS_NAMES = {0: "SWA_OK", 1: "SWA_ERR_INVALID_ARG", 2: "SWA_ERR_UNSUPPORTED",
                3: "SWA_ERR_HIP", 4: "SWA_ERR_STATE"}

EXPORTED = ("swa_prefill", "swa_cache_init", "swa_cache_append", "swa_decode", "swa_prefill_chunk",
            "swa_prefill_lsink", "swa_decode_lsink", "swa_cache_append_fp8", "swa_decode_fp8",
            "swa_prefill_varlen", "swa_paged_cache_init", "swa_paged_append", "swa_paged_decode",
            "swa_paged_prefill_chunk",
            "swa_paged_decode_workspace_bytes", "swa_decode_step", "swa_decode_noalloc",
            "swa_decode_workspace_bytes", "swa_cache_slot", "swa_attended_count",
            "swa_last_error")


class SwaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__("%s: %s" % (STATUS_NAMES.get(status, status), message))
        self.status = status


class swa_cache(ctypes.Structure):
    _fields_ = [("k", ctypes.c_void_p), ("v", ctypes.c_void_p), ("n", ctypes.c_int64),
                ("B", ctypes.c_int), ("Hkv", ctypes.c_int), ("d", ctypes.c_int),
                ("w", ctypes.c_int), ("s", ctypes.c_int), ("dt", ctypes.c_int)]


class swa_paged_cache(ctypes.Structure):
    _fields_ = [("k_pool", ctypes.c_void_p), ("v_pool", ctypes.c_void_p), ("block_table", ctypes.c_void_p),
                ("n", ctypes.c_void_p), ("B", ctypes.c_int), ("num_pages", ctypes.c_int), ("page", ctypes.c_int),
                ("pages_per_seq", ctypes.c_int), ("Hkv", ctypes.c_int), ("d", ctypes.c_int), ("w", ctypes.c_int),
                ("s", ctypes.c_int), ("dt", ctypes.c_int)]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError("libswa.so is not built; run `python sliding_window_sink_amd/build.py`")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i, i64, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_size_t
    cp = ctypes.POINTER(swa_cache)
    lib.swa_prefill.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, i, i, i, vp]
    lib.swa_prefill.restype = i
    lib.swa_cache_init.argtypes = [cp, vp, vp, i, i, i, i, i, i]
    lib.swa_cache_init.restype = i
    lib.swa_cache_append.argtypes = [cp, vp, vp, i, vp]
    lib.swa_cache_append.restype = i
    lib.swa_decode.argtypes = [cp, vp, vp, i, vp, sz, vp]
    lib.swa_decode.restype = i
    lib.swa_prefill_lsink.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, i, i, vp]
    lib.swa_prefill_lsink.restype = i
    lib.swa_decode_noalloc.argtypes = [cp, vp, vp, i, vp]
    lib.swa_decode_noalloc.restype = i
    lib.swa_decode_lsink.argtypes = [cp, vp, vp, vp, i, vp, sz, vp]
    lib.swa_decode_lsink.restype = i
    lib.swa_cache_append_fp8.argtypes = [cp, vp, vp, i, vp, vp]
    lib.swa_cache_append_fp8.restype = i
    lib.swa_decode_fp8.argtypes = [cp, vp, vp, vp, vp, i, vp, sz, vp]
    lib.swa_decode_fp8.restype = i
    lib.swa_decode_step.argtypes = [cp, vp, vp, vp, vp, vp, i, vp, sz, vp]
    lib.swa_decode_step.restype = i
    pp = ctypes.POINTER(swa_paged_cache)
    lib.swa_prefill_varlen.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, i, i, i, vp]
    lib.swa_prefill_varlen.restype = i
    lib.swa_paged_cache_init.argtypes = [pp, vp, vp, vp, vp, i, i, i, i, i, i, i, i]
    lib.swa_paged_cache_init.restype = i
    lib.swa_paged_append.argtypes = [pp, vp, vp, vp, i, vp]
    lib.swa_paged_append.restype = i
    lib.swa_paged_decode.argtypes = [pp, vp, vp, vp, i, vp, sz, vp]
    lib.swa_paged_decode.restype = i
    lib.swa_paged_prefill_chunk.argtypes = [pp, vp, vp, vp, vp, vp, vp, i, i, i, i, vp]
    lib.swa_paged_prefill_chunk.restype = i
    lib.swa_paged_decode_workspace_bytes.argtypes = [pp, i]
    lib.swa_paged_decode_workspace_bytes.restype = sz
    lib.swa_prefill_chunk.argtypes = [cp, vp, vp, vp, vp, vp, i, i, i, vp]
    lib.swa_prefill_chunk.restype = i
    lib.swa_decode_workspace_bytes.argtypes = [cp, i]
    lib.swa_decode_workspace_bytes.restype = sz
    lib.swa_cache_slot.argtypes = [i, i, i64]
    lib.swa_cache_slot.restype = i64
    lib.swa_attended_count.argtypes = [i, i, i64]
    lib.swa_attended_count.restype = i64
    lib.swa_last_error.argtypes = []
    lib.swa_last_error.restype = ctypes.c_char_p
    return lib


lib = _load()


def last_error() -> str:
    return lib.swa_last_error().decode()


def _check(status: int):
    if status != SWA_OK:
        raise SwaError(status, last_error())


def _dt(dtype) -> int:
    if dtype == torch.bfloat16:
        return SWA_BF16
    if dtype == torch.float32:
        return SWA_F32
    if dtype == torch.float8_e4m3fn:
        return SWA_FP8_E4M3  # cache element type only
    raise TypeError("libswa supports torch.bfloat16 and torch.float32 (and float8_e4m3fn caches), got %s" % dtype)


def _ptr(t: torch.Tensor | None):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _dense(t: torch.Tensor, name: str):
    if not t.is_cuda:
        raise ValueError("%s must be a device tensor" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)


def cache_slot(w: int, s: int, p: int) -> int:
    """0-based slot of 1-based position p (-1 if invalid)."""
    return lib.swa_cache_slot(int(w), int(s), int(p))


def attended_count(w: int, s: int, t: int) -> int:
    return lib.swa_attended_count(int(w), int(s), int(t))


def _sink(sink_logit, Hq, device):
    if sink_logit is None:
        return None
    _dense(sink_logit, "sink_logit")
    if sink_logit.dtype != torch.float32 or sink_logit.shape != (Hq,):
        raise ValueError("sink_logit must be a float32 tensor of one logit per query head")
    return sink_logit


def prefill(Q, K, V, w: int, s: int, *, out=None, lse: bool = False, out_dtype=None, sink_logit=None,
            stream=None):
    """SWA(w,s) attention of every prompt row.  Q [B,L,Hq,d]; K, V [B,L,Hkv,d]
    with G = Hq/Hkv query heads per kv-head.  out_dtype: Q's dtype (default),
    or torch.float32 for bfloat16 inputs."""
    for t, nm in ((Q, "Q"), (K, "K"), (V, "V")):
        _dense(t, nm)
    B, L, Hq, d = Q.shape
    Hkv = K.shape[2]
    if K.shape != (B, L, Hkv, d) or V.shape != K.shape:
        raise ValueError("K and V must be [B, L, Hkv, d] matching Q")
    if Hq % Hkv:
        raise ValueError("Hq = %d is not a multiple of Hkv = %d" % (Hq, Hkv))
    if K.dtype != Q.dtype or V.dtype != Q.dtype:
        raise TypeError("Q, K and V must share one dtype")
    if out is None:
        out = torch.empty(Q.shape, dtype=out_dtype or Q.dtype, device=Q.device)
    else:
        _dense(out, "out")
        if out.shape != Q.shape or (out_dtype is not None and out.dtype != out_dtype):
            raise ValueError("out must match Q's shape (and out_dtype)")
    lse_t = torch.empty((B, Hq, L), dtype=torch.float32, device=Q.device) if lse else None
    sk = _sink(sink_logit, Hq, Q.device)
    if sk is None:
        _check(lib.swa_prefill(_ptr(Q), _ptr(K), _ptr(V), _ptr(out), _ptr(lse_t), B, L, Hq, Hq // Hkv, d,
                               int(w), int(s), _dt(Q.dtype), _dt(out.dtype), _stream(stream)))
    else:
        _check(lib.swa_prefill_lsink(_ptr(Q), _ptr(K), _ptr(V), _ptr(out), _ptr(lse_t), _ptr(sk), B, L, Hq,
                                     Hq // Hkv, d, int(w), int(s), _dt(Q.dtype), _dt(out.dtype), _stream(stream)))
    return (out, lse_t) if lse else out


def prefill_varlen(Q, K, V, cu_seqlens, max_len: int, w: int, s: int, *, out=None, lse: bool = False,
                   out_dtype=None, stream=None):
    """SWA(w,s) prefill of B packed sequences: Q [total, Hq, d]; K, V
    [total, Hkv, d]; cu_seqlens int32 device [B + 1] (sequence b is rows
    cu_seqlens[b] .. cu_seqlens[b+1]-1); max_len >= the longest sequence."""
    for t, nm in ((Q, "Q"), (K, "K"), (V, "V"), (cu_seqlens, "cu_seqlens")):
        _dense(t, nm)
    total, Hq, d = Q.shape
    Hkv = K.shape[1]
    if K.shape != (total, Hkv, d) or V.shape != K.shape:
        raise ValueError("K and V must be [total, Hkv, d] matching Q")
    if cu_seqlens.dtype != torch.int32 or cu_seqlens.dim() != 1:
        raise ValueError("cu_seqlens must be a 1-D int32 tensor")
    if Hq % Hkv:
        raise ValueError("Hq = %d is not a multiple of Hkv = %d" % (Hq, Hkv))
    if K.dtype != Q.dtype or V.dtype != Q.dtype:
        raise TypeError("Q, K and V must share one dtype")
    if out is None:
        out = torch.empty(Q.shape, dtype=out_dtype or Q.dtype, device=Q.device)
    else:
        _dense(out, "out")
        if out.shape != Q.shape:
            raise ValueError("out must match Q's shape")
    lse_t = torch.empty((Hq, total), dtype=torch.float32, device=Q.device) if lse else None
    _check(lib.swa_prefill_varlen(_ptr(Q), _ptr(K), _ptr(V), _ptr(out), _ptr(lse_t), _ptr(cu_seqlens),
                                  cu_seqlens.numel() - 1, total, int(max_len), Hq, Hq // Hkv, d, int(w), int(s),
                                  _dt(Q.dtype), _dt(out.dtype), _stream(stream)))
    return (out, lse_t) if lse else out


class PagedCache:
    """A paged cache (swa_paged_cache): bf16 page pools [num_pages, Hkv, page, d],
    a block table int32 [B, ceil(w / page)] and per-sequence position counts
    int64 [B], all device tensors owned here (pass block_table to use your
    own).  The table starts at -1 (no page); assign pages before appending."""

    def __init__(self, B: int, Hkv: int, d: int, w: int, s: int, page: int, num_pages: int,
                 device="cuda", block_table=None):
        self.k = torch.empty((num_pages, Hkv, page, d), dtype=torch.bfloat16, device=device)
        self.v = torch.empty_like(self.k)
        pps = (w + page - 1) // page
        if block_table is None:
            block_table = torch.full((B, pps), -1, dtype=torch.int32, device=device)
        _dense(block_table, "block_table")
        if block_table.dtype != torch.int32 or block_table.shape != (B, pps):
            raise ValueError("block_table must be int32 [B, ceil(w / page)]")
        self.block_table = block_table
        self.n = torch.zeros(B, dtype=torch.int64, device=device)
        self.c = swa_paged_cache()
        _check(lib.swa_paged_cache_init(ctypes.byref(self.c), _ptr(self.k), _ptr(self.v), _ptr(self.block_table),
                                        _ptr(self.n), B, num_pages, page, Hkv, d, int(w), int(s), SWA_BF16))
        self._ws = None

    def append(self, K_new, V_new, cu_seqlens, stream=None):
        """Sequence b appends rows cu_seqlens[b] .. cu_seqlens[b+1]-1 of the
        packed K_new, V_new [total, Hkv, d]; n advances on the device."""
        for t, nm in ((K_new, "K_new"), (V_new, "V_new"), (cu_seqlens, "cu_seqlens")):
            _dense(t, nm)
        c = self.c
        if K_new.dim() != 3 or K_new.shape[1:] != (c.Hkv, c.d) or V_new.shape != K_new.shape:
            raise ValueError("K_new, V_new must be [total, Hkv, d]")
        if K_new.dtype != torch.bfloat16 or V_new.dtype != torch.bfloat16:
            raise TypeError("new rows must be bfloat16")
        if cu_seqlens.dtype != torch.int32 or cu_seqlens.shape != (c.B + 1,):
            raise ValueError("cu_seqlens must be int32 [B + 1]")
        _check(lib.swa_paged_append(ctypes.byref(c), _ptr(K_new), _ptr(V_new), _ptr(cu_seqlens), K_new.shape[0],
                                    _stream(stream)))

    def workspace_bytes(self, Hq: int) -> int:
        return lib.swa_paged_decode_workspace_bytes(ctypes.byref(self.c), Hq // self.c.Hkv)

    def prefill_chunk(self, Q, K_new, V_new, cu_seqlens, max_chunk: int, *, out=None, lse: bool = False,
                      out_dtype=None, stream=None):
        """Sequence b's chunk rows cu_seqlens[b] .. cu_seqlens[b+1]-1 of the
        packed Q [total, Hq, d] (positions n[b]+1 ..) attend its pages and its
        chunk, then every chunk is appended (swa_paged_prefill_chunk).
        K_new, V_new [total, Hkv, d]; max_chunk >= the longest chunk."""
        for t, nm in ((Q, "Q"), (K_new, "K_new"), (V_new, "V_new"), (cu_seqlens, "cu_seqlens")):
            _dense(t, nm)
        c = self.c
        total, Hq, d = Q.shape
        if d != c.d or Hq % c.Hkv or K_new.shape != (total, c.Hkv, d) or V_new.shape != K_new.shape:
            raise ValueError("Q [total, G * Hkv, d] and K_new, V_new [total, Hkv, d] must match the cache")
        if Q.dtype != torch.bfloat16 or K_new.dtype != Q.dtype or V_new.dtype != Q.dtype:
            raise TypeError("Q, K_new and V_new must be bfloat16")
        if cu_seqlens.dtype != torch.int32 or cu_seqlens.shape != (c.B + 1,):
            raise ValueError("cu_seqlens must be int32 [B + 1]")
        if out is None:
            out = torch.empty(Q.shape, dtype=out_dtype or Q.dtype, device=Q.device)
        else:
            _dense(out, "out")
            if out.shape != Q.shape or (out_dtype is not None and out.dtype != out_dtype):
                raise ValueError("out must match Q's shape (and out_dtype)")
        lse_t = torch.empty((Hq, total), dtype=torch.float32, device=Q.device) if lse else None
        _check(lib.swa_paged_prefill_chunk(ctypes.byref(c), _ptr(Q), _ptr(K_new), _ptr(V_new), _ptr(out),
                                           _ptr(lse_t), _ptr(cu_seqlens), total, int(max_chunk), Hq // c.Hkv,
                                           _dt(out.dtype), _stream(stream)))
        return (out, lse_t) if lse else out

    def decode(self, Q, *, out=None, workspace=None, sink_logit=None, stream=None):
        _dense(Q, "Q")
        c = self.c
        B, Hq, d = Q.shape
        if B != c.B or d != c.d or Hq % c.Hkv:
            raise ValueError("Q must be [B, G * Hkv, d] matching the cache")
        if Q.dtype != torch.bfloat16:
            raise TypeError("Q must be bfloat16")
        if out is None:
            out = torch.empty_like(Q)
        need = self.workspace_bytes(Hq)
        if workspace is None and need:
            if self._ws is None or self._ws.numel() < need:
                self._ws = torch.empty(need, dtype=torch.uint8, device=Q.device)
            workspace = self._ws
        sk = _sink(sink_logit, Hq, Q.device)
        wsb = workspace.numel() if workspace is not None else 0
        _check(lib.swa_paged_decode(ctypes.byref(c), _ptr(Q), _ptr(out), _ptr(sk), Hq // c.Hkv, _ptr(workspace),
                                    wsb, _stream(stream)))
        return out


class Cache:
    """One layer's constant-size cache: K, V buffers [B, Hkv, w, d] plus the
    count of positions appended so far.  Mirrors the swa_cache struct.

    dtype=torch.float8_e4m3fn makes an E4M3 cache: kv_scale (float32 device
    tensor [2, Hkv]: K scales, then V scales) is then required; new rows and
    queries are bfloat16 and are quantised / attended through
    swa_cache_append_fp8 and swa_decode_fp8."""

    def __init__(self, B: int, Hkv: int, d: int, w: int, s: int, dtype=torch.bfloat16,
                 device="cuda", Hq: int | None = None, k=None, v=None, kv_scale=None):
        # Caller buffers are read and written as [B, Hkv, w, d] of `dtype` by
        # every kernel on this cache: check them here, before the C side sees
        # a pointer (it can only check NULL and alignment).
        for t, nm in ((k, "k"), (v, "v")):
            if t is None:
                continue
            _dense(t, nm)
            if tuple(t.shape) != (B, Hkv, w, d) or t.dtype != dtype:
                raise ValueError("%s must be a %s tensor [B, Hkv, w, d] = %s, got %s %s"
                                 % (nm, dtype, (B, Hkv, w, d), t.dtype, tuple(t.shape)))
        if k is not None and v is not None and k.device != v.device:
            raise ValueError("k and v must be on the same device")
        if (k is None) != (v is None):
            ref = k if k is not None else v
            device = ref.device
        self.k = k if k is not None else torch.empty((B, Hkv, w, d), dtype=dtype, device=device)
        self.v = v if v is not None else torch.empty((B, Hkv, w, d), dtype=dtype, device=device)
        self.fp8 = dtype == torch.float8_e4m3fn
        if self.fp8:
            if kv_scale is None:
                raise ValueError("an fp8 cache needs kv_scale [2, Hkv]")
            _dense(kv_scale, "kv_scale")
            if kv_scale.dtype != torch.float32 or kv_scale.shape != (2, Hkv):
                raise ValueError("kv_scale must be a float32 tensor [2, Hkv]")
        elif kv_scale is not None:
            raise ValueError("kv_scale is for fp8 caches only")
        self.kv_scale = kv_scale
        self.c = swa_cache()
        _check(lib.swa_cache_init(ctypes.byref(self.c), _ptr(self.k), _ptr(self.v), B, Hkv, d,
                                  int(w), int(s), _dt(dtype)))
        self.Hq = Hq
        self._ws = None

    @property
    def compute_dtype(self):
        """dtype of new rows, queries and outputs."""
        return torch.bfloat16 if self.fp8 else self.k.dtype

    @property
    def n(self) -> int:
        return self.c.n

    @n.setter
    def n(self, value: int):
        self.c.n = int(value)

    def group(self, Hq: int) -> int:
        if Hq % self.c.Hkv:
            raise ValueError("Hq = %d is not a multiple of Hkv = %d" % (Hq, self.c.Hkv))
        return Hq // self.c.Hkv

    def workspace_bytes(self, Hq: int) -> int:
        return lib.swa_decode_workspace_bytes(ctypes.byref(self.c), self.group(int(Hq)))

    def append(self, K_new, V_new, stream=None):
        _dense(K_new, "K_new")
        _dense(V_new, "V_new")
        c = self.c
        if K_new.dim() != 4 or K_new.shape[0] != c.B or K_new.shape[2:] != (c.Hkv, c.d) \
                or V_new.shape != K_new.shape:
            raise ValueError("K_new, V_new must be [B, n_new, Hkv, d]")
        if K_new.dtype != self.compute_dtype or V_new.dtype != self.compute_dtype:
            raise TypeError("new rows must be %s" % self.compute_dtype)
        if self.fp8:
            _check(lib.swa_cache_append_fp8(ctypes.byref(c), _ptr(K_new), _ptr(V_new), K_new.shape[1],
                                            _ptr(self.kv_scale), _stream(stream)))
        else:
            _check(lib.swa_cache_append(ctypes.byref(c), _ptr(K_new), _ptr(V_new), K_new.shape[1],
                                        _stream(stream)))

    def prefill_chunk(self, Q, K_new, V_new, *, out=None, lse: bool = False, out_dtype=None, stream=None):
        """Positions n+1..n+C attend the cache and the chunk, then the chunk
        is appended.  Q [B, C, Hq, d]; K_new, V_new [B, C, Hkv, d]."""
        for t, nm in ((Q, "Q"), (K_new, "K_new"), (V_new, "V_new")):
            _dense(t, nm)
        c = self.c
        B, C, Hq, d = Q.shape
        if B != c.B or d != c.d or K_new.shape != (B, C, c.Hkv, d) or V_new.shape != K_new.shape:
            raise ValueError("Q [B, C, Hq, d] and K_new, V_new [B, C, Hkv, d] must match the cache")
        if Q.dtype != self.k.dtype or K_new.dtype != Q.dtype or V_new.dtype != Q.dtype:
            raise TypeError("Q, K_new and V_new must have the cache dtype")
        if out is None:
            out = torch.empty(Q.shape, dtype=out_dtype or Q.dtype, device=Q.device)
        else:
            _dense(out, "out")
            if out.shape != Q.shape or (out_dtype is not None and out.dtype != out_dtype):
                raise ValueError("out must match Q's shape (and out_dtype)")
        lse_t = torch.empty((B, Hq, C), dtype=torch.float32, device=Q.device) if lse else None
        _check(lib.swa_prefill_chunk(ctypes.byref(c), _ptr(Q), _ptr(K_new), _ptr(V_new), _ptr(out), _ptr(lse_t),
                                     C, self.group(Hq), _dt(out.dtype), _stream(stream)))
        return (out, lse_t) if lse else out

    def step(self, K_new, V_new, Q, *, out=None, workspace=None, sink_logit=None, stream=None):
        """Append one position (K_new, V_new [B, Hkv, d]) and decode Q at it,
        in one launch (swa_decode_step)."""
        for t, nm in ((K_new, "K_new"), (V_new, "V_new"), (Q, "Q")):
            _dense(t, nm)
        c = self.c
        B, Hq, d = Q.shape
        if K_new.shape[0] != c.B or K_new.shape[-2:] != (c.Hkv, c.d) or K_new.numel() != c.B * c.Hkv * c.d \
                or V_new.shape != K_new.shape:
            raise ValueError("K_new, V_new must be [B, Hkv, d] (or [B, 1, Hkv, d])")
        if B != c.B or d != c.d:
            raise ValueError("Q must be [B, Hq, d] matching the cache")
        if Q.dtype != self.k.dtype or K_new.dtype != Q.dtype or V_new.dtype != Q.dtype:
            raise TypeError("K_new, V_new and Q must have the cache dtype")
        if out is None:
            out = torch.empty_like(Q)
        need = self.workspace_bytes(Hq)
        if workspace is None and need:
            if self._ws is None or self._ws.numel() < need:
                self._ws = torch.empty(need, dtype=torch.uint8, device=Q.device)
            workspace = self._ws
        sk = _sink(sink_logit, Hq, Q.device)
        wsb = workspace.numel() if workspace is not None else 0
        _check(lib.swa_decode_step(ctypes.byref(c), _ptr(K_new), _ptr(V_new), _ptr(Q), _ptr(out), _ptr(sk),
                                   self.group(Hq), _ptr(workspace), wsb, _stream(stream)))
        return out

    def decode_noalloc(self, Q, out, stream=None):
        """swa_decode_noalloc: decode with the library's fixed per-GPU scratch
        instead of a workspace; allocates nothing (out is required)."""
        _dense(Q, "Q")
        _dense(out, "out")
        c = self.c
        B, Hq, d = Q.shape
        if B != c.B or d != c.d or out.shape != Q.shape:
            raise ValueError("Q and out must be [B, Hq, d] matching the cache")
        if Q.dtype != self.compute_dtype or out.dtype != Q.dtype:
            raise TypeError("Q and out must be %s" % self.compute_dtype)
        if self.fp8:
            raise TypeError("swa_decode_noalloc takes bf16 and fp32 caches")
        _check(lib.swa_decode_noalloc(ctypes.byref(c), _ptr(Q), _ptr(out), self.group(Hq), _stream(stream)))
        return out

    def decode(self, Q, *, out=None, workspace=None, sink_logit=None, stream=None):
        _dense(Q, "Q")
        c = self.c
        B, Hq, d = Q.shape
        if B != c.B or d != c.d:
            raise ValueError("Q must be [B, Hq, d] matching the cache")
        if Q.dtype != self.compute_dtype:
            raise TypeError("Q must be %s" % self.compute_dtype)
        if out is None:
            out = torch.empty_like(Q)
        need = self.workspace_bytes(Hq)
        if workspace is None and need:
            if self._ws is None or self._ws.numel() < need:
                self._ws = torch.empty(need, dtype=torch.uint8, device=Q.device)
            workspace = self._ws
        sk = _sink(sink_logit, Hq, Q.device)
        wsb = workspace.numel() if workspace is not None else 0
        if self.fp8:
            _check(lib.swa_decode_fp8(ctypes.byref(c), _ptr(Q), _ptr(out), _ptr(self.kv_scale), _ptr(sk),
                                      self.group(Hq), _ptr(workspace), wsb, _stream(stream)))
        elif sk is None:
            _check(lib.swa_decode(ctypes.byref(c), _ptr(Q), _ptr(out), self.group(Hq), _ptr(workspace), wsb,
                                  _stream(stream)))
        else:
            _check(lib.swa_decode_lsink(ctypes.byref(c), _ptr(Q), _ptr(out), _ptr(sk), self.group(Hq),
                                        _ptr(workspace), wsb, _stream(stream)))
        return out


__all__ = ["prefill", "prefill_varlen", "Cache", "PagedCache", "cache_slot", "attended_count", "last_error", "SwaError",
           "LIB_PATH", "EXPORTED", "lib"]
