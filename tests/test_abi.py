"""The C ABI on the CPU: the library loads, exports what include/swa.h
declares, its host-only functions agree with the oracle, and bad arguments are
rejected before anything reaches the device (so these run without a GPU)."""
import ctypes
import os
import re

import pytest

import oracle
from oracle import brute

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def swa():
    import sliding_window_sink_amd as swa
    return swa


def _declared():
    with open(os.path.join(ROOT, "include", "swa.h")) as f:
        text = f.read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*(swa_[a-z_0-9]+)\s*\(", text, re.M)))


def test_exports_every_declared_symbol(swa):
    names = _declared()
    assert "swa_prefill" in names and "swa_decode" in names and len(names) >= 8
    lib = ctypes.CDLL(swa.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(swa.EXPORTED) == names


def test_slot_map_matches_oracle(swa):
    for w in range(1, 20):
        for s in range(0, w):
            for p in range(1, 80):
                assert swa.cache_slot(w, s, p) == oracle.slot(w, s, p)
    assert swa.cache_slot(262144, 4, 262144) == 262143
    assert swa.cache_slot(576, 4, 8192) == oracle.slot(576, 4, 8192)
    assert swa.cache_slot(4, 4, 1) == -1 and swa.cache_slot(4, 1, 0) == -1


def test_attended_count(swa):
    for w in range(1, 20):
        for s in range(0, w):
            for t in range(1, 60):
                assert swa.attended_count(w, s, t) == len(brute.retained_after(w, s, t)) == min(t, w)
    assert swa.attended_count(64, 4, 10**12) == 64
    assert swa.attended_count(64, 64, 5) == -1


# --- validation without a device --------------------------------------------

A = 0x10000  # a 16-byte aligned fake device address: never dereferenced


def _prefill(swa, **kw):
    args = dict(Q=A, K=A, V=A, O=A, lse=None, B=1, L=16, Hq=4, G=4, d=128, w=8, s=4,
                in_dt=swa.SWA_BF16, out_dt=None)
    args.update(kw)
    if args["out_dt"] is None:
        args["out_dt"] = args["in_dt"]
    st = swa.lib.swa_prefill(*(ctypes.c_void_p(args[k]) if k in "QKVO" else args[k]
                               for k in ("Q", "K", "V", "O", "lse", "B", "L", "Hq", "G", "d",
                                         "w", "s", "in_dt", "out_dt")), None)
    return st, swa.last_error()


@pytest.mark.parametrize("kw,status,needle", [
    (dict(Q=0), 1, "NULL"),
    (dict(O=0), 1, "NULL"),
    (dict(K=A + 8), 1, "aligned"),
    (dict(lse=A + 2), 1, "aligned"),
    (dict(B=0), 1, "B ="),
    (dict(L=-1), 1, "L ="),
    (dict(Hq=6, G=4), 1, "multiple"),
    (dict(Hq=0, G=1), 1, "head count"),
    (dict(G=0), 1, "positive"),
    (dict(Hq=3, G=3), 2, "query heads"),
    (dict(Hq=16, G=16), 2, "query heads"),
    (dict(d=96), 2, "64 and 128"),
    (dict(d=0), 1, "positive"),
    (dict(w=4, s=4), 1, "window"),
    (dict(s=-1), 1, "sink"),
    (dict(in_dt=7), 1, "in_dt"),
    (dict(out_dt=7), 1, "out_dt"),
    (dict(in_dt=0, out_dt=1), 2, "out_dt"),
])
def test_prefill_rejects(swa, kw, status, needle):
    st, msg = _prefill(swa, **kw)
    assert st == status, (kw, st, msg)
    assert needle in msg


def test_prefill_empty_is_noop(swa):
    st, msg = _prefill(swa, L=0)
    assert st == 0 and msg == ""


def _cache(swa, **kw):
    args = dict(k=A, v=A, B=2, Hkv=8, d=128, w=64, s=4, dt=swa.SWA_BF16)
    args.update(kw)
    c = swa.swa_cache()
    st = swa.lib.swa_cache_init(ctypes.byref(c), ctypes.c_void_p(args["k"]), ctypes.c_void_p(args["v"]),
                                args["B"], args["Hkv"], args["d"], args["w"], args["s"], args["dt"])
    return st, c


def test_cache_init(swa):
    st, c = _cache(swa)
    assert st == 0 and c.n == 0 and c.w == 64 and c.s == 4 and c.k == A
    for kw, code in [(dict(k=0), 1), (dict(v=A + 4), 1), (dict(w=4, s=4), 1), (dict(d=80), 2),
                     (dict(B=0), 1), (dict(dt=3), 1)]:
        assert _cache(swa, **kw)[0] == code, kw


def test_cache_append_and_decode_reject(swa):
    st, c = _cache(swa)
    lib = swa.lib
    assert lib.swa_cache_append(ctypes.byref(c), ctypes.c_void_p(A), ctypes.c_void_p(A), 0, None) == 1
    assert "n_new" in swa.last_error()
    assert lib.swa_cache_append(ctypes.byref(c), None, ctypes.c_void_p(A), 1, None) == 1
    assert c.n == 0  # untouched by rejected calls
    # decode on an empty cache
    assert lib.swa_decode(ctypes.byref(c), ctypes.c_void_p(A), ctypes.c_void_p(A), 4, None, 0, None) == 4
    assert "empty" in swa.last_error()
    c.n = 10
    assert lib.swa_decode(ctypes.byref(c), ctypes.c_void_p(A), ctypes.c_void_p(A), 0, None, 0, None) == 1
    assert lib.swa_decode(ctypes.byref(c), ctypes.c_void_p(A), ctypes.c_void_p(A), 3, None, 0, None) == 2
    assert lib.swa_decode(ctypes.byref(c), None, ctypes.c_void_p(A), 4, None, 0, None) == 1
    c.n = -1
    assert lib.swa_decode(ctypes.byref(c), ctypes.c_void_p(A), ctypes.c_void_p(A), 4, None, 0, None) == 4


def test_prefill_chunk_rejects(swa):
    st, c = _cache(swa)
    lib = swa.lib
    a = ctypes.c_void_p(A)
    call = lambda **kw: lib.swa_prefill_chunk(ctypes.byref(c), kw.get("Q", a), a, a, kw.get("O", a), None,
                                              kw.get("C", 4), kw.get("G", 4), kw.get("out_dt", swa.SWA_BF16), None)
    assert call(C=0) == 1 and "C =" in swa.last_error()
    assert call(G=3) == 2
    assert call(Q=None) == 1
    assert call(O=ctypes.c_void_p(A + 4)) == 1
    assert call(out_dt=7) == 1
    st32, c32 = _cache(swa, dt=swa.SWA_F32)
    assert lib.swa_prefill_chunk(ctypes.byref(c32), a, a, a, a, None, 4, 4, swa.SWA_BF16, None) == 2
    assert c.n == 0 and c32.n == 0  # untouched by rejected calls


def test_fp8_cache_calls_reject(swa):
    """An E4M3 cache takes only the fp8 append/decode calls (they carry the
    scales), and those take only an E4M3 cache; scales are required."""
    lib = swa.lib
    a = ctypes.c_void_p(A)
    st, c8 = _cache(swa, dt=swa.SWA_FP8_E4M3)
    assert st == 0 and c8.dt == swa.SWA_FP8_E4M3
    st, c16 = _cache(swa)
    assert lib.swa_cache_append(ctypes.byref(c8), a, a, 1, None) == 2
    assert "swa_cache_append_fp8" in swa.last_error()
    c8.n = 10
    assert lib.swa_decode(ctypes.byref(c8), a, a, 4, None, 0, None) == 2
    assert lib.swa_decode_lsink(ctypes.byref(c8), a, a, a, 4, None, 0, None) == 2
    assert lib.swa_prefill_chunk(ctypes.byref(c8), a, a, a, a, None, 4, 4, swa.SWA_BF16, None) == 2
    # the fp8 calls refuse other caches, and missing or misaligned scales
    assert lib.swa_cache_append_fp8(ctypes.byref(c16), a, a, 1, a, None) == 1
    assert lib.swa_cache_append_fp8(ctypes.byref(c8), a, a, 1, None, None) == 1
    assert "kv_scale" in swa.last_error()
    assert lib.swa_cache_append_fp8(ctypes.byref(c8), a, a, 1, ctypes.c_void_p(A + 2), None) == 1
    assert lib.swa_cache_append_fp8(ctypes.byref(c8), a, a, 0, a, None) == 1
    c16.n = 10
    assert lib.swa_decode_fp8(ctypes.byref(c16), a, a, a, None, 4, None, 0, None) == 1
    assert lib.swa_decode_fp8(ctypes.byref(c8), a, a, None, None, 4, None, 0, None) == 1
    assert lib.swa_decode_fp8(ctypes.byref(c8), a, a, a, None, 3, None, 0, None) == 2
    c8.n = 0
    assert lib.swa_decode_fp8(ctypes.byref(c8), a, a, a, None, 4, None, 0, None) == 4
    assert c8.n == 0 and c16.n == 10  # untouched by rejected calls


def _paged(swa, **kw):
    args = dict(k=A, v=A, bt=A, n=A, B=4, num_pages=64, page=64, Hkv=8, d=128, w=512, s=4, dt=swa.SWA_BF16)
    args.update(kw)
    c = swa.swa_paged_cache()
    vp = ctypes.c_void_p
    st = swa.lib.swa_paged_cache_init(ctypes.byref(c), vp(args["k"]), vp(args["v"]), vp(args["bt"]), vp(args["n"]),
                                      args["B"], args["num_pages"], args["page"], args["Hkv"], args["d"],
                                      args["w"], args["s"], args["dt"])
    return st, c


def test_paged_cache_init(swa):
    st, c = _paged(swa)
    assert st == 0 and c.pages_per_seq == 8 and c.page == 64
    st, c = _paged(swa, w=100, page=32)
    assert st == 0 and c.pages_per_seq == 4
    for kw, code in [(dict(page=48), 2), (dict(page=16), 2), (dict(page=8192), 2), (dict(dt=swa.SWA_F32), 2),
                     (dict(dt=swa.SWA_FP8_E4M3), 2), (dict(bt=0), 1), (dict(n=0), 1), (dict(n=A + 4), 1),
                     (dict(k=A + 8), 1), (dict(num_pages=0), 1), (dict(B=0), 1), (dict(w=4, s=4), 1),
                     (dict(d=96), 2)]:
        assert _paged(swa, **kw)[0] == code, kw


def test_paged_calls_reject(swa):
    lib = swa.lib
    a = ctypes.c_void_p(A)
    st, c = _paged(swa)
    assert lib.swa_paged_append(ctypes.byref(c), a, a, None, 4, None) == 1
    assert lib.swa_paged_append(ctypes.byref(c), a, a, a, -1, None) == 1
    assert lib.swa_paged_append(ctypes.byref(c), ctypes.c_void_p(A + 8), a, a, 4, None) == 1
    assert lib.swa_paged_decode(ctypes.byref(c), a, a, None, 3, None, 0, None) == 2
    assert lib.swa_paged_decode(ctypes.byref(c), None, a, None, 4, None, 0, None) == 1
    assert lib.swa_paged_decode(ctypes.byref(c), a, a, ctypes.c_void_p(A + 2), 4, None, 0, None) == 1
    # a tampered struct is re-checked by every call
    c.pages_per_seq = 3
    assert lib.swa_paged_decode(ctypes.byref(c), a, a, None, 4, None, 0, None) == 1
    assert "pages_per_seq" in swa.last_error()
    # long windows split over workgroups: the workspace is required
    st, c = _paged(swa, B=1, w=262144, page=256)
    ws = lib.swa_paged_decode_workspace_bytes(ctypes.byref(c), 4)
    assert st == 0 and ws > 0
    assert lib.swa_paged_decode(ctypes.byref(c), a, a, None, 4, a, 16, None) == 1
    assert "workspace" in swa.last_error()


def test_paged_prefill_chunk_rejects(swa):
    lib = swa.lib
    a = ctypes.c_void_p(A)
    st, c = _paged(swa)
    assert st == 0
    f = lib.swa_paged_prefill_chunk
    assert f(ctypes.byref(c), a, a, a, a, None, None, 8, 4, 4, 1, None) == 1        # no cu_seqlens
    assert f(ctypes.byref(c), a, a, a, a, None, ctypes.c_void_p(A + 2), 8, 4, 4, 1, None) == 1
    assert f(ctypes.byref(c), a, a, a, a, None, a, 8, 9, 4, 1, None) == 1           # max_chunk > total
    assert f(ctypes.byref(c), a, a, a, a, None, a, -1, 0, 4, 1, None) == 1
    assert f(ctypes.byref(c), ctypes.c_void_p(A + 8), a, a, a, None, a, 8, 4, 4, 1, None) == 1
    assert f(ctypes.byref(c), a, a, a, a, ctypes.c_void_p(A + 2), a, 8, 4, 4, 1, None) == 1
    assert f(ctypes.byref(c), a, a, a, a, None, a, 8, 4, 3, 1, None) == 2           # G = 3
    assert f(ctypes.byref(c), a, a, a, a, None, a, 8, 4, 4, 2, None) == 2           # fp8 output
    assert f(ctypes.byref(c), a, a, a, a, None, a, 0, 0, 4, 1, None) == 0           # nothing to do
    c.page = 48
    assert f(ctypes.byref(c), a, a, a, a, None, a, 8, 4, 4, 1, None) == 2
    assert "page" in swa.last_error()


def test_prefill_varlen_rejects(swa):
    lib = swa.lib
    a = ctypes.c_void_p(A)
    call = lambda **kw: lib.swa_prefill_varlen(
        a, a, a, a, None, kw.get("cu", a), kw.get("B", 3), kw.get("total", 100), kw.get("max_len", 60),
        32, kw.get("G", 4), kw.get("d", 128), 512, 4, swa.SWA_BF16, swa.SWA_BF16, None)
    assert call(cu=None) == 1 and "cu_seqlens" in swa.last_error()
    assert call(cu=ctypes.c_void_p(A + 2)) == 1
    assert call(total=-1) == 1
    assert call(max_len=101) == 1
    assert call(G=3) == 2
    assert call(d=96) == 2
    assert call(B=0) == 1
    assert call(total=0, max_len=0) == 0  # nothing to do


def test_decode_step_rejects(swa):
    lib = swa.lib
    a = ctypes.c_void_p(A)
    st, c = _cache(swa)
    call = lambda cc, **kw: lib.swa_decode_step(ctypes.byref(cc), kw.get("K", a), a, kw.get("Q", a), a, None,
                                                kw.get("G", 4), None, 0, None)
    assert call(c, K=None) == 1
    assert call(c, K=ctypes.c_void_p(A + 8)) == 1
    assert call(c, G=3) == 2
    assert call(c, Q=None) == 1
    st, c8 = _cache(swa, dt=swa.SWA_FP8_E4M3)
    assert call(c8) == 2
    st, c32 = _cache(swa, dt=swa.SWA_F32)
    assert call(c32, G=3) == 2
    assert c.n == 0 and c8.n == 0 and c32.n == 0  # untouched by rejected calls


def test_decode_workspace_sizing(swa):
    # short windows need no workspace
    st, c = _cache(swa, B=64, w=512)
    assert swa.lib.swa_decode_workspace_bytes(ctypes.byref(c), 4) == 0
    # a long full-history cache at batch 1 splits the rows over workgroups
    st, c = _cache(swa, B=1, w=262144, s=4)
    ws = swa.lib.swa_decode_workspace_bytes(ctypes.byref(c), 4)
    assert ws > 0 and ws % (32 * (128 + 2) * 4) == 0
    # decode refuses a workspace that is too small (before any launch)
    c.n = 262144
    assert swa.lib.swa_decode(ctypes.byref(c), ctypes.c_void_p(A), ctypes.c_void_p(A), 4,
                              ctypes.c_void_p(A), 16, None) == 1
    assert "workspace" in swa.last_error()


def test_product_never_touches_oracle():
    """The HIP path and its binding import nothing from oracle/ (and the
    oracle imports nothing from the product)."""
    pkg = os.path.join(ROOT, "sliding_window_sink_amd")
    for dirpath, _, files in os.walk(pkg):
        for fn in files:
            if fn.endswith((".py", ".cpp", ".hip", ".h")):
                with open(os.path.join(dirpath, fn)) as f:
                    text = f.read()
                assert not re.search(r"^\s*(import|from)\s+oracle\b", text, re.M), fn
                assert "swa_oracle" not in text and "libswa_oracle" not in text, fn
    for fn in os.listdir(os.path.join(ROOT, "oracle")):
        if fn.endswith((".py", ".c")):
            with open(os.path.join(ROOT, "oracle", fn)) as f:
                text = f.read()
            assert not re.search(r"^\s*(import|from)\s+sliding_window_sink_amd", text, re.M), fn
            assert "#include \"swa.h\"" not in text and "libswa.so" not in text, fn


def test_cache_rejects_bad_caller_buffers(swa):
    """Cache(k=, v=) checks the caller's buffers before any pointer reaches
    the C side: host tensors, wrong shape, wrong dtype, strided views."""
    import torch
    good = torch.empty((2, 1, 8, 64), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="device tensor"):
        swa.Cache(2, 1, 64, 8, 4, dtype=torch.bfloat16, k=good, v=good)


def test_decode_noalloc_rejects_before_device(swa):
    """swa_decode_noalloc validates like swa_decode, and a plan whose split
    partials exceed the fixed 2 MiB scratch is refused before any device
    call (255 pairs x 8 query heads at w = 1024: about 3.2 MB)."""
    c = swa.swa_cache()
    assert swa.lib.swa_cache_init(ctypes.byref(c), ctypes.c_void_p(A), ctypes.c_void_p(A), 255, 1, 128,
                                  1024, 4, swa.SWA_BF16) == 0
    c.n = 1024
    st = swa.lib.swa_decode_noalloc(ctypes.byref(c), ctypes.c_void_p(A), ctypes.c_void_p(A), 8, None)
    assert st == swa.SWA_ERR_UNSUPPORTED and "scratch" in swa.last_error()
    c.n = 0
    st = swa.lib.swa_decode_noalloc(ctypes.byref(c), ctypes.c_void_p(A), ctypes.c_void_p(A), 8, None)
    assert st == swa.SWA_ERR_STATE
    c.n = 1024
    st = swa.lib.swa_decode_noalloc(ctypes.byref(c), ctypes.c_void_p(A), ctypes.c_void_p(A + 4), 8, None)
    assert st == swa.SWA_ERR_INVALID_ARG and "aligned" in swa.last_error()


def test_peaks_library_exports_its_header():
    """The bench's peak probes (libswa_peaks.so) export what
    include/swa_peaks.h declares, and refuse bad arguments before any launch."""
    with open(os.path.join(ROOT, "include", "swa_peaks.h")) as f:
        names = sorted(set(re.findall(r"^\s*int\s+(swa_peak_[a-z_0-9]+)\s*\(", f.read(), re.M)))
    assert names == ["swa_peak_mfma", "swa_peak_stream_read"]
    lib = ctypes.CDLL(os.path.join(ROOT, "sliding_window_sink_amd", "libswa_peaks.so"))
    for n in names:
        assert hasattr(lib, n), n
    lib.swa_peak_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int,
                                         ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    lib.swa_peak_mfma.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    assert lib.swa_peak_stream_read(None, 1 << 20, ctypes.c_void_p(A), 8, 4, 0, None) == 1
    assert lib.swa_peak_stream_read(ctypes.c_void_p(A + 4), 1 << 20, ctypes.c_void_p(A), 8, 4, 0, None) == 1
    assert lib.swa_peak_stream_read(ctypes.c_void_p(A), 1 << 20, ctypes.c_void_p(A), 8, 3, 0, None) == 1
    assert lib.swa_peak_mfma(ctypes.c_void_p(A), None, 8, 10, None) == 1
    assert lib.swa_peak_mfma(ctypes.c_void_p(A), ctypes.c_void_p(A), 0, 10, None) == 1
