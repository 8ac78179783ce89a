// libswa C ABI: argument validation, error reporting, cache bookkeeping and
// kernel dispatch.  Every check happens before anything is enqueued, so a
// rejected call touches no device memory.
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "swa.h"
#include "swa_internal.h"

namespace {

thread_local char g_err[512];

void clear_error() { g_err[0] = '\0'; }

swa_status fail(swa_status st, const char *fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return st;
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }
bool dtype_ok(swa_dtype dt) { return dt == SWA_F32 || dt == SWA_BF16; }  // compute dtypes
bool cache_dtype_ok(swa_dtype dt) { return dtype_ok(dt) || dt == SWA_FP8_E4M3; }
int elem_bytes(swa_dtype dt) { return dt == SWA_F32 ? 4 : dt == SWA_BF16 ? 2 : 1; }
bool group_ok(int G) { return G == 1 || G == 2 || G == 4 || G == 8; }
swa::Dt to_dt(swa_dtype dt)
{
    return dt == SWA_BF16 ? swa::Dt::BF16 : dt == SWA_FP8_E4M3 ? swa::Dt::FP8 : swa::Dt::F32;
}

swa_status check_window(int w, int s)
{
    if (s < 0) return fail(SWA_ERR_INVALID_ARG, "s = %d: the sink count must be >= 0", s);
    if (w <= s) return fail(SWA_ERR_INVALID_ARG, "w = %d, s = %d: the window must exceed the sink count", w, s);
    return SWA_OK;
}

swa_status check_head_dim(int d)
{
    if (d < 1) return fail(SWA_ERR_INVALID_ARG, "d = %d: head dimension must be positive", d);
    if (d != 64 && d != 128) return fail(SWA_ERR_UNSUPPORTED, "d = %d: supported head dimensions are 64 and 128", d);
    return SWA_OK;
}

swa_status check_group(int G)
{
    if (G < 1) return fail(SWA_ERR_INVALID_ARG, "G = %d: query heads per kv-head must be positive", G);
    if (!group_ok(G)) return fail(SWA_ERR_UNSUPPORTED, "G = %d: supported query heads per kv-head are 1, 2, 4, 8", G);
    return SWA_OK;
}

swa_status check_cache(const swa_cache *c)
{
    if (!c) return fail(SWA_ERR_INVALID_ARG, "cache is NULL");
    if (!c->k || !c->v) return fail(SWA_ERR_INVALID_ARG, "cache buffers are NULL");
    if (!aligned16(c->k) || !aligned16(c->v)) return fail(SWA_ERR_INVALID_ARG, "cache buffers must be 16-byte aligned");
    if (c->B < 1 || c->Hkv < 1) return fail(SWA_ERR_INVALID_ARG, "cache has B = %d, Hkv = %d", c->B, c->Hkv);
    if (c->n < 0) return fail(SWA_ERR_STATE, "cache position count is negative (%lld)", (long long)c->n);
    if (!cache_dtype_ok(c->dt)) return fail(SWA_ERR_INVALID_ARG, "cache dtype %d is not a swa_dtype", (int)c->dt);
    swa_status st = check_window(c->w, c->s);
    if (st != SWA_OK) return st;
    return check_head_dim(c->d);
}

// The fp8 cache takes its own append and decode calls (they carry the scales).
swa_status check_cache_kind(const swa_cache *c, bool fp8)
{
    if (fp8 && c->dt != SWA_FP8_E4M3) return fail(SWA_ERR_INVALID_ARG, "this call takes an SWA_FP8_E4M3 cache");
    if (!fp8 && c->dt == SWA_FP8_E4M3)
        return fail(SWA_ERR_UNSUPPORTED, "an SWA_FP8_E4M3 cache takes swa_cache_append_fp8 and swa_decode_fp8");
    return SWA_OK;
}

swa_status check_scale(const float *kv_scale)
{
    if (!kv_scale) return fail(SWA_ERR_INVALID_ARG, "kv_scale must not be NULL");
    if ((uintptr_t)kv_scale & 3u) return fail(SWA_ERR_INVALID_ARG, "kv_scale must be 4-byte aligned");
    return SWA_OK;
}

swa_status hip_status(hipError_t e, const char *what)
{
    if (e == hipSuccess) return SWA_OK;
    return fail(SWA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

}  // namespace

namespace {
// cu_seqlens set: varlen mode (L = the longest sequence, total = packed rows).
swa_status prefill_impl(const void *Q, const void *K, const void *V, void *O, float *lse, const float *sink_logit,
                        int B, int L, int Hq, int G, int d, int w, int s, swa_dtype in_dt, swa_dtype out_dt,
                        void *hip_stream, const int32_t *cu_seqlens = nullptr, int total = 0)
{
    clear_error();
    if (sink_logit && ((uintptr_t)sink_logit & 3u)) return fail(SWA_ERR_INVALID_ARG, "sink_logit must be 4-byte aligned");
    if (!Q || !K || !V || !O) return fail(SWA_ERR_INVALID_ARG, "Q, K, V and O must not be NULL");
    if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(O))
        return fail(SWA_ERR_INVALID_ARG, "Q, K, V and O must be 16-byte aligned");
    if (lse && ((uintptr_t)lse & 3u)) return fail(SWA_ERR_INVALID_ARG, "lse must be 4-byte aligned");
    if (B < 1 || L < 0) return fail(SWA_ERR_INVALID_ARG, "B = %d, L = %d: need B >= 1 and L >= 0", B, L);
    if (!dtype_ok(in_dt)) return fail(SWA_ERR_INVALID_ARG, "in_dt %d is not a swa_dtype", (int)in_dt);
    if (!dtype_ok(out_dt)) return fail(SWA_ERR_INVALID_ARG, "out_dt %d is not a swa_dtype", (int)out_dt);
    if (out_dt != in_dt && !(in_dt == SWA_BF16 && out_dt == SWA_F32))
        return fail(SWA_ERR_UNSUPPORTED, "out_dt must equal in_dt, or be fp32 for bf16 inputs");
    if (Hq < 1) return fail(SWA_ERR_INVALID_ARG, "Hq = %d: head count must be positive", Hq);
    swa_status st;
    if ((st = check_group(G)) != SWA_OK) return st;
    if (Hq % G) return fail(SWA_ERR_INVALID_ARG, "Hq = %d is not a multiple of G = %d", Hq, G);
    if ((st = check_head_dim(d)) != SWA_OK) return st;
    if ((st = check_window(w, s)) != SWA_OK) return st;
    const int Hkv = Hq / G;
    // K/V rows of one (batch, kv-head) are addressed through a buffer
    // descriptor with a 32-bit byte range.
    const long long rows = cu_seqlens ? (long long)total : L;
    if (rows * Hkv * d * (in_dt == SWA_BF16 ? 2 : 4) >= 0x7fffffffLL)
        return fail(SWA_ERR_UNSUPPORTED, "%s*Hkv*d = %lld elements: one sequence's K or V must stay under 2 GiB",
                    cu_seqlens ? "total" : "L", rows * Hkv * d);
    const long long blocks = ((long long)L + 128 / G - 1) / (128 / G) * B * Hkv;
    if (blocks > 0x7fffffffLL) return fail(SWA_ERR_UNSUPPORTED, "B*L*Hkv too large for one launch");
    if (L == 0 || (cu_seqlens && total == 0)) return SWA_OK;
    swa::PrefillParams p{Q, K, V, O, lse, B, L, Hq, Hkv, w, s};
    p.sink_logit = sink_logit;
    if (cu_seqlens) {
        p.cu_seqlens = cu_seqlens;
        p.total = total;
        return hip_status(swa::launch_prefill_varlen(to_dt(in_dt), to_dt(out_dt), d, G, p, (hipStream_t)hip_stream),
                          "varlen prefill launch");
    }
    return hip_status(swa::launch_prefill(to_dt(in_dt), to_dt(out_dt), d, G, p, (hipStream_t)hip_stream),
                      "prefill launch");
}
}  // namespace

namespace {
// K_new set: fused step -- the new position's rows are appended (slot of
// position c->n + 1) and attended in the same launch; c->n is not changed here.
// fixed_scratch: split partials go to the library's fixed per-GPU array
// (swa_decode_noalloc) instead of the caller's workspace.
swa_status decode_impl(const swa_cache *c, const void *Q, void *O, const float *sink_logit, const float *kv_scale,
                       int G, void *workspace, size_t ws_bytes, void *hip_stream, const void *K_new = nullptr,
                       const void *V_new = nullptr, bool fixed_scratch = false)
{
    if (sink_logit && ((uintptr_t)sink_logit & 3u)) return fail(SWA_ERR_INVALID_ARG, "sink_logit must be 4-byte aligned");
    swa_status st = check_cache(c);
    if (st != SWA_OK) return st;
    if ((st = check_cache_kind(c, kv_scale != nullptr)) != SWA_OK) return st;
    if (!Q || !O) return fail(SWA_ERR_INVALID_ARG, "Q and O must not be NULL");
    if (!aligned16(Q) || !aligned16(O)) return fail(SWA_ERR_INVALID_ARG, "Q and O must be 16-byte aligned");
    if ((st = check_group(G)) != SWA_OK) return st;
    const int Hq = G * c->Hkv;
    const int64_t n = K_new ? c->n + 1 : c->n;  // the query position
    if (n == 0) return fail(SWA_ERR_STATE, "decode on an empty cache (no position appended)");
    // one (batch, kv-head) block of the cache is read through a buffer
    // descriptor with a 32-bit byte range
    if ((long long)c->w * c->d * elem_bytes(c->dt) >= 0x7fffffffLL)
        return fail(SWA_ERR_UNSUPPORTED, "w*d = %lld elements: one (batch, kv-head) cache block must stay under 2 GiB",
                    (long long)c->w * c->d);

    const int nvalid = (int)(n < c->w ? n : c->w);
    int ns, rps, max_ns, ppw, wpw;
    swa::decode_plan(c->B, c->Hkv, nvalid, &ns, &rps, &max_ns, &ppw, &wpw, c->dt == SWA_BF16);
    swa::DecodeParams p;
    p.Kc = c->k;
    p.Vc = c->v;
    p.Q = Q;
    p.O = O;
    p.part = nullptr;
    p.B = c->B;
    p.Hq = Hq;
    p.Hkv = c->Hkv;
    p.w = c->w;
    p.nvalid = nvalid;
    p.nsplit = ns;
    p.rows_per_split = rps;
    p.pairs_per_wg = ppw;
    p.waves_per_wg = wpw;
    p.sink_logit = sink_logit;
    p.kv_scale = kv_scale;
    if (ns > 1 && fixed_scratch) {
        const size_t need = (size_t)c->B * Hq * ns * (c->d + 2) * sizeof(float);
        if (need > swa::kDecodeScratchBytes)
            return fail(SWA_ERR_UNSUPPORTED,
                        "this decode splits into %d partials per query head and needs %zu bytes of scratch; "
                        "the fixed scratch holds %zu (use swa_decode with a workspace)",
                        ns, need, swa::kDecodeScratchBytes);
        int dev = -1;
        st = hip_status(hipGetDevice(&dev), "hipGetDevice");
        if (st != SWA_OK) return st;
        if (hip_stream) {
            hipDevice_t sdev = -1;
            st = hip_status(hipStreamGetDevice((hipStream_t)hip_stream, &sdev), "hipStreamGetDevice");
            if (st != SWA_OK) return st;
            if (sdev != dev)
                return fail(SWA_ERR_INVALID_ARG, "the stream belongs to device %d but device %d is current", (int)sdev,
                            dev);
        }
        void *ptr = nullptr;
        st = hip_status(swa::decode_scratch(dev, &ptr), "fixed scratch lookup");
        if (st != SWA_OK) return st;
        p.part = (float *)ptr;
    } else if (ns > 1) {
        const size_t need = (size_t)c->B * Hq * ns * (c->d + 2) * sizeof(float);
        if (!workspace || ws_bytes < need)
            return fail(SWA_ERR_INVALID_ARG, "decode needs a workspace of %zu bytes (got %zu)", need,
                        workspace ? ws_bytes : (size_t)0);
        if (!aligned16(workspace)) return fail(SWA_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
        p.part = (float *)workspace;
    }
    if (K_new) {
        p.Kn = K_new;
        p.Vn = V_new;
        p.new_slot = (int)(n <= c->s ? n - 1 : c->s + (n - c->s - 1) % (c->w - c->s));
        return hip_status(swa::launch_decode_step(c->d, G, p, (hipStream_t)hip_stream), "decode step launch");
    }
    return hip_status(swa::launch_decode(to_dt(c->dt), c->d, G, p, (hipStream_t)hip_stream),
                      "decode launch");
}
swa_status append_impl(swa_cache *c, const void *K_new, const void *V_new, int n_new, const float *kv_scale,
                       void *hip_stream)
{
    swa_status st = check_cache(c);
    if (st != SWA_OK) return st;
    if ((st = check_cache_kind(c, kv_scale != nullptr)) != SWA_OK) return st;
    if (!K_new || !V_new) return fail(SWA_ERR_INVALID_ARG, "K_new and V_new must not be NULL");
    if (!aligned16(K_new) || !aligned16(V_new)) return fail(SWA_ERR_INVALID_ARG, "K_new and V_new must be 16-byte aligned");
    if (n_new < 1) return fail(SWA_ERR_INVALID_ARG, "n_new = %d: need at least one new position", n_new);
    if (c->n > INT64_MAX - n_new) return fail(SWA_ERR_STATE, "position count would overflow");

    const int64_t n = c->n, N = n + n_new, w = c->w, s = c->s;
    swa::AppendParams p;
    p.Kn = K_new;
    p.Vn = V_new;
    p.Kc = c->k;
    p.Vc = c->v;
    p.B = c->B;
    p.Hkv = c->Hkv;
    p.w = c->w;
    p.s = c->s;
    p.n_new = n_new;
    p.n_before = n;
    // New positions still attended after the append (members of S_N): the
    // sinks among them, and the most recent w - s positions.
    p.a1 = n + 1;
    p.b1 = N < s ? N : s;
    int64_t a2 = N - (w - s) + 1;
    if (a2 < s + 1) a2 = s + 1;
    if (a2 < n + 1) a2 = n + 1;
    p.a2 = a2;
    p.b2 = N;
    p.kv_scale = kv_scale;
    st = hip_status(swa::launch_append(to_dt(c->dt), c->d, p, (hipStream_t)hip_stream), "append launch");
    if (st == SWA_OK) c->n = N;
    return st;
}

swa_status check_paged(const swa_paged_cache *c)
{
    if (!c) return fail(SWA_ERR_INVALID_ARG, "paged cache is NULL");
    if (!c->k_pool || !c->v_pool || !c->block_table || !c->n)
        return fail(SWA_ERR_INVALID_ARG, "pools, block table and position counts must not be NULL");
    if (!aligned16(c->k_pool) || !aligned16(c->v_pool)) return fail(SWA_ERR_INVALID_ARG, "pools must be 16-byte aligned");
    if (((uintptr_t)c->block_table & 3u) || ((uintptr_t)c->n & 7u))
        return fail(SWA_ERR_INVALID_ARG, "block_table must be 4-byte and n 8-byte aligned");
    if (c->B < 1 || c->Hkv < 1 || c->num_pages < 1)
        return fail(SWA_ERR_INVALID_ARG, "B = %d, Hkv = %d, num_pages = %d: need each >= 1", c->B, c->Hkv, c->num_pages);
    if (c->dt != SWA_BF16) return fail(SWA_ERR_UNSUPPORTED, "paged caches are bf16");
    swa_status st = check_window(c->w, c->s);
    if (st != SWA_OK) return st;
    if ((st = check_head_dim(c->d)) != SWA_OK) return st;
    if (c->page < 32 || c->page > 4096 || c->page % 32)
        return fail(SWA_ERR_UNSUPPORTED, "page = %d: pages hold a multiple of 32 slots, 32 .. 4096", c->page);
    if (c->pages_per_seq != (c->w + c->page - 1) / c->page)
        return fail(SWA_ERR_INVALID_ARG, "pages_per_seq = %d, expected ceil(w / page) = %d", c->pages_per_seq,
                    (c->w + c->page - 1) / c->page);
    // a page of one kv-head, and a whole page, stay far below 2 GiB; the pool
    // is indexed in 64-bit arithmetic
    return SWA_OK;
}

}  // namespace

extern "C" {

const char *swa_last_error(void) { return g_err; }

int64_t swa_cache_slot(int w, int s, int64_t p)
{
    if (s < 0 || w <= s || p < 1) return -1;
    if (p <= s) return p - 1;
    return s + (p - s - 1) % (w - s);
}

int64_t swa_attended_count(int w, int s, int64_t t)
{
    if (s < 0 || w <= s || t < 1) return -1;
    return t < w ? t : w;
}

swa_status swa_prefill(const void *Q, const void *K, const void *V, void *O, float *lse, int B, int L, int Hq,
                       int G, int d, int w, int s, swa_dtype in_dt, swa_dtype out_dt, void *hip_stream)
{
    return prefill_impl(Q, K, V, O, lse, nullptr, B, L, Hq, G, d, w, s, in_dt, out_dt, hip_stream);
}

swa_status swa_prefill_lsink(const void *Q, const void *K, const void *V, void *O, float *lse,
                             const float *sink_logit, int B, int L, int Hq, int G, int d, int w, int s,
                             swa_dtype in_dt, swa_dtype out_dt, void *hip_stream)
{
    if (!sink_logit) {
        clear_error();
        return fail(SWA_ERR_INVALID_ARG, "sink_logit must not be NULL");
    }
    return prefill_impl(Q, K, V, O, lse, sink_logit, B, L, Hq, G, d, w, s, in_dt, out_dt, hip_stream);
}

swa_status swa_cache_init(swa_cache *c, void *k_buf, void *v_buf, int B, int Hkv, int d, int w, int s, swa_dtype dt)
{
    clear_error();
    if (!c) return fail(SWA_ERR_INVALID_ARG, "cache is NULL");
    swa_cache t;
    memset(&t, 0, sizeof t);
    t.k = k_buf;
    t.v = v_buf;
    t.n = 0;
    t.B = B;
    t.Hkv = Hkv;
    t.d = d;
    t.w = w;
    t.s = s;
    t.dt = dt;
    swa_status st = check_cache(&t);
    if (st != SWA_OK) return st;
    *c = t;
    return SWA_OK;
}

swa_status swa_cache_append(swa_cache *c, const void *K_new, const void *V_new, int n_new, void *hip_stream)
{
    clear_error();
    return append_impl(c, K_new, V_new, n_new, nullptr, hip_stream);
}

swa_status swa_cache_append_fp8(swa_cache *c, const void *K_new, const void *V_new, int n_new, const float *kv_scale,
                                void *hip_stream)
{
    clear_error();
    swa_status st = check_scale(kv_scale);
    if (st != SWA_OK) return st;
    return append_impl(c, K_new, V_new, n_new, kv_scale, hip_stream);
}

swa_status swa_prefill_chunk(swa_cache *c, const void *Q, const void *K_new, const void *V_new, void *O, float *lse,
                             int C, int G, swa_dtype out_dt, void *hip_stream)
{
    clear_error();
    swa_status st = check_cache(c);
    if (st != SWA_OK) return st;
    if ((st = check_cache_kind(c, false)) != SWA_OK) return st;
    if (!Q || !K_new || !V_new || !O) return fail(SWA_ERR_INVALID_ARG, "Q, K_new, V_new and O must not be NULL");
    if (!aligned16(Q) || !aligned16(K_new) || !aligned16(V_new) || !aligned16(O))
        return fail(SWA_ERR_INVALID_ARG, "Q, K_new, V_new and O must be 16-byte aligned");
    if (lse && ((uintptr_t)lse & 3u)) return fail(SWA_ERR_INVALID_ARG, "lse must be 4-byte aligned");
    if (C < 1) return fail(SWA_ERR_INVALID_ARG, "C = %d: need at least one new position", C);
    if (!dtype_ok(out_dt)) return fail(SWA_ERR_INVALID_ARG, "out_dt %d is not a swa_dtype", (int)out_dt);
    if (out_dt != c->dt && !(c->dt == SWA_BF16 && out_dt == SWA_F32))
        return fail(SWA_ERR_UNSUPPORTED, "out_dt must equal the cache dtype, or be fp32 for a bf16 cache");
    if ((st = check_group(G)) != SWA_OK) return st;
    if (c->n > INT64_MAX - C) return fail(SWA_ERR_STATE, "position count would overflow");
    const int es = c->dt == SWA_BF16 ? 2 : 4;
    if ((long long)C * c->Hkv * c->d * es >= 0x7fffffffLL || (long long)c->w * c->d * es >= 0x7fffffffLL)
        return fail(SWA_ERR_UNSUPPORTED, "one sequence's chunk rows or one cache block must stay under 2 GiB");
    const int Hq = G * c->Hkv;
    if (((long long)C + 128 / G - 1) / (128 / G) * c->B * c->Hkv > 0x7fffffffLL)
        return fail(SWA_ERR_UNSUPPORTED, "B*C*Hkv too large for one launch");

    const int64_t n = c->n, w = c->w, s = c->s;
    if (c->dt == SWA_BF16 && out_dt == SWA_BF16 && !lse && C * G <= 16) {
        // A short chunk (C rows x G heads fit the 16 columns of the decode
        // kernel's MFMA tile) goes through the decode kernel in its
        // multi-query mode when the cache needs no split: the cache is read
        // once per (b, kv-head) as in decode, and the chunk's rows are written
        // into their slots by the same launch.
        const int nvalid = (int)(n < w ? n : w);
        int ns, rps, max_ns, ppw, wpw;
        swa::decode_plan(c->B, c->Hkv, nvalid, &ns, &rps, &max_ns, &ppw, &wpw, true);
        if (ns == 1) {
            swa::DecodeParams p;
            p.Kc = c->k;
            p.Vc = c->v;
            p.Q = Q;
            p.O = O;
            p.part = nullptr;
            p.B = c->B;
            p.Hq = Hq;
            p.Hkv = c->Hkv;
            p.w = c->w;
            p.nvalid = nvalid;
            p.nsplit = 1;
            p.rows_per_split = rps;
            p.pairs_per_wg = 1;
            p.waves_per_wg = wpw;  // 4 (the planner's 1-, 2- or 4-task workgroups become one task each), 8 or 16
            p.Kn = K_new;
            p.Vn = V_new;
            p.mq_c = C;
            p.s = c->s;
            p.ring_head = n > s ? (int)((n - s - 1) % (w - s)) : 0;
            p.n0 = n;
            st = hip_status(swa::launch_decode_mq(c->d, G, p, (hipStream_t)hip_stream), "multi-query decode launch");
            if (st != SWA_OK) return st;
            c->n += C;
            return SWA_OK;
        }
    }
    swa::PrefillParams p{Q, K_new, V_new, O, lse, c->B, C, Hq, c->Hkv, c->w, c->s};
    p.Kc = c->k;
    p.Vc = c->v;
    p.nvalid = (int)(n < w ? n : w);
    p.sinks_in = (int)(n < s ? n : s);
    p.ring_any = n > s;
    p.ring_head = n > s ? (int)((n - s - 1) % (w - s)) : 0;
    p.ring_full = n - s >= w - s;
    p.sk = (int)(s - n <= 0 ? 0 : (s - n < C ? s - n : C));
    st = hip_status(swa::launch_prefill_chunk(to_dt(c->dt), to_dt(out_dt), c->d, G, p, (hipStream_t)hip_stream),
                    "chunk prefill launch");
    if (st != SWA_OK) return st;
    // then the chunk joins the cache (after the attention has read the slots
    // that its later rows evict)
    return swa_cache_append(c, K_new, V_new, C, hip_stream);
}

swa_status swa_prefill_varlen(const void *Q, const void *K, const void *V, void *O, float *lse,
                              const int32_t *cu_seqlens, int B, int total, int max_len, int Hq, int G, int d, int w,
                              int s, swa_dtype in_dt, swa_dtype out_dt, void *hip_stream)
{
    clear_error();
    if (!cu_seqlens || ((uintptr_t)cu_seqlens & 3u))
        return fail(SWA_ERR_INVALID_ARG, "cu_seqlens must be a non-NULL, 4-byte aligned device array");
    if (total < 0 || max_len < 0)
        return fail(SWA_ERR_INVALID_ARG, "total = %d, max_len = %d: need both >= 0", total, max_len);
    if (max_len > total) return fail(SWA_ERR_INVALID_ARG, "max_len = %d exceeds total = %d", max_len, total);
    return prefill_impl(Q, K, V, O, lse, nullptr, B, max_len, Hq, G, d, w, s, in_dt, out_dt, hip_stream, cu_seqlens,
                        total);
}

swa_status swa_paged_cache_init(swa_paged_cache *c, void *k_pool, void *v_pool, const int32_t *block_table,
                                int64_t *n, int B, int num_pages, int page, int Hkv, int d, int w, int s,
                                swa_dtype dt)
{
    clear_error();
    if (!c) return fail(SWA_ERR_INVALID_ARG, "paged cache is NULL");
    swa_paged_cache t;
    memset(&t, 0, sizeof t);
    t.k_pool = k_pool;
    t.v_pool = v_pool;
    t.block_table = block_table;
    t.n = n;
    t.B = B;
    t.num_pages = num_pages;
    t.page = page;
    t.pages_per_seq = page > 0 ? (w + page - 1) / page : 0;
    t.Hkv = Hkv;
    t.d = d;
    t.w = w;
    t.s = s;
    t.dt = dt;
    swa_status st = check_paged(&t);
    if (st != SWA_OK) return st;
    *c = t;
    return SWA_OK;
}

swa_status swa_paged_append(const swa_paged_cache *c, const void *K_new, const void *V_new,
                            const int32_t *cu_seqlens, int total, void *hip_stream)
{
    clear_error();
    swa_status st = check_paged(c);
    if (st != SWA_OK) return st;
    if (!K_new || !V_new || !cu_seqlens) return fail(SWA_ERR_INVALID_ARG, "K_new, V_new and cu_seqlens must not be NULL");
    if (!aligned16(K_new) || !aligned16(V_new)) return fail(SWA_ERR_INVALID_ARG, "K_new and V_new must be 16-byte aligned");
    if ((uintptr_t)cu_seqlens & 3u) return fail(SWA_ERR_INVALID_ARG, "cu_seqlens must be 4-byte aligned");
    if (total < 0) return fail(SWA_ERR_INVALID_ARG, "total = %d: need total >= 0", total);
    swa::PagedAppendParams p;
    p.c.Kp = c->k_pool;
    p.c.Vp = c->v_pool;
    p.c.block_table = c->block_table;
    p.c.n = c->n;
    p.c.num_pages = c->num_pages;
    p.c.page = c->page;
    p.c.pages_per_seq = c->pages_per_seq;
    p.Kn = K_new;
    p.Vn = V_new;
    p.cu_seqlens = cu_seqlens;
    p.B = c->B;
    p.Hkv = c->Hkv;
    p.w = c->w;
    p.s = c->s;
    p.total = total;
    return hip_status(swa::launch_paged_append(to_dt(c->dt), c->d, p, (hipStream_t)hip_stream), "paged append launch");
}

swa_status swa_paged_prefill_chunk(const swa_paged_cache *c, const void *Q, const void *K_new, const void *V_new,
                                   void *O, float *lse, const int32_t *cu_seqlens, int total, int max_chunk, int G,
                                   swa_dtype out_dt, void *hip_stream)
{
    clear_error();
    swa_status st = check_paged(c);
    if (st != SWA_OK) return st;
    if (!Q || !K_new || !V_new || !O || !cu_seqlens)
        return fail(SWA_ERR_INVALID_ARG, "Q, K_new, V_new, O and cu_seqlens must not be NULL");
    if (!aligned16(Q) || !aligned16(K_new) || !aligned16(V_new) || !aligned16(O))
        return fail(SWA_ERR_INVALID_ARG, "Q, K_new, V_new and O must be 16-byte aligned");
    if (lse && ((uintptr_t)lse & 3u)) return fail(SWA_ERR_INVALID_ARG, "lse must be 4-byte aligned");
    if ((uintptr_t)cu_seqlens & 3u) return fail(SWA_ERR_INVALID_ARG, "cu_seqlens must be 4-byte aligned");
    if (total < 0 || max_chunk < 0)
        return fail(SWA_ERR_INVALID_ARG, "total = %d, max_chunk = %d: need both >= 0", total, max_chunk);
    if (max_chunk > total) return fail(SWA_ERR_INVALID_ARG, "max_chunk = %d exceeds total = %d", max_chunk, total);
    if (out_dt != SWA_BF16 && out_dt != SWA_F32)
        return fail(SWA_ERR_UNSUPPORTED, "out_dt must be bf16 (the cache dtype) or fp32");
    if ((st = check_group(G)) != SWA_OK) return st;
    const int Hq = G * c->Hkv;
    // one sequence's chunk rows are addressed through a buffer descriptor
    // with a 32-bit byte range
    if ((long long)total * c->Hkv * c->d * 2 >= 0x7fffffffLL)
        return fail(SWA_ERR_UNSUPPORTED, "total*Hkv*d = %lld elements: the chunk rows must stay under 2 GiB",
                    (long long)total * c->Hkv * c->d);
    if (((long long)max_chunk + 128 / G - 1) / (128 / G) * c->B * c->Hkv > 0x7fffffffLL)
        return fail(SWA_ERR_UNSUPPORTED, "B*max_chunk*Hkv too large for one launch");
    if (total == 0 || max_chunk == 0) return SWA_OK;  // no new position anywhere
    swa::PrefillParams p{Q, K_new, V_new, O, lse, c->B, max_chunk, Hq, c->Hkv, c->w, c->s};
    p.cu_seqlens = cu_seqlens;
    p.total = total;
    p.pg.Kp = c->k_pool;
    p.pg.Vp = c->v_pool;
    p.pg.block_table = c->block_table;
    p.pg.n = c->n;
    p.pg.num_pages = c->num_pages;
    p.pg.page = c->page;
    p.pg.pages_per_seq = c->pages_per_seq;
    st = hip_status(swa::launch_prefill_chunk_paged(to_dt(out_dt), c->d, G, p, (hipStream_t)hip_stream),
                    "paged chunk prefill launch");
    if (st != SWA_OK) return st;
    // then each sequence's chunk joins its pages and n[b] advances (after the
    // attention has read the slots that its later rows evict)
    return swa_paged_append(c, K_new, V_new, cu_seqlens, total, hip_stream);
}

size_t swa_paged_decode_workspace_bytes(const swa_paged_cache *c, int G)
{
    if (!c || c->B < 1 || c->Hkv < 1 || c->w < 1 || c->d < 1 || G < 1) return 0;
    int ns, rps, max_ns, ppw, wpw;
    swa::decode_plan(c->B, c->Hkv, c->w, &ns, &rps, &max_ns, &ppw, &wpw, c->dt == SWA_BF16);
    if (ns <= 1) return 0;
    return (size_t)c->B * G * c->Hkv * ns * (c->d + 2) * sizeof(float);
}

swa_status swa_paged_decode(const swa_paged_cache *c, const void *Q, void *O, const float *sink_logit, int G,
                            void *workspace, size_t ws_bytes, void *hip_stream)
{
    clear_error();
    swa_status st = check_paged(c);
    if (st != SWA_OK) return st;
    if (!Q || !O) return fail(SWA_ERR_INVALID_ARG, "Q and O must not be NULL");
    if (!aligned16(Q) || !aligned16(O)) return fail(SWA_ERR_INVALID_ARG, "Q and O must be 16-byte aligned");
    if (sink_logit && ((uintptr_t)sink_logit & 3u)) return fail(SWA_ERR_INVALID_ARG, "sink_logit must be 4-byte aligned");
    if ((st = check_group(G)) != SWA_OK) return st;
    const int Hq = G * c->Hkv;
    // every sequence is planned for a full window (its n is on the device)
    int ns, rps, max_ns, ppw, wpw;
    swa::decode_plan(c->B, c->Hkv, c->w, &ns, &rps, &max_ns, &ppw, &wpw, c->dt == SWA_BF16);
    swa::DecodeParams p;
    p.Kc = nullptr;
    p.Vc = nullptr;
    p.Q = Q;
    p.O = O;
    p.part = nullptr;
    p.B = c->B;
    p.Hq = Hq;
    p.Hkv = c->Hkv;
    p.w = c->w;
    p.nvalid = c->w;
    p.nsplit = ns;
    p.rows_per_split = rps;
    p.pairs_per_wg = ppw;
    p.waves_per_wg = wpw;
    p.sink_logit = sink_logit;
    p.pg.Kp = c->k_pool;
    p.pg.Vp = c->v_pool;
    p.pg.block_table = c->block_table;
    p.pg.n = c->n;
    p.pg.num_pages = c->num_pages;
    p.pg.page = c->page;
    p.pg.pages_per_seq = c->pages_per_seq;
    if (ns > 1) {
        const size_t need = (size_t)c->B * Hq * ns * (c->d + 2) * sizeof(float);
        if (!workspace || ws_bytes < need)
            return fail(SWA_ERR_INVALID_ARG, "paged decode needs a workspace of %zu bytes (got %zu)", need,
                        workspace ? ws_bytes : (size_t)0);
        if (!aligned16(workspace)) return fail(SWA_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
        p.part = (float *)workspace;
    }
    return hip_status(swa::launch_decode_paged(c->d, G, p, (hipStream_t)hip_stream), "paged decode launch");
}

size_t swa_decode_workspace_bytes(const swa_cache *c, int G)
{
    if (!c || c->B < 1 || c->Hkv < 1 || c->w < 1 || c->d < 1 || G < 1) return 0;
    const long long Hq = (long long)G * c->Hkv;
    int ns, rps, max_ns, ppw, wpw;
    swa::decode_plan(c->B, c->Hkv, c->w, &ns, &rps, &max_ns, &ppw, &wpw, c->dt == SWA_BF16);
    if (max_ns <= 1) return 0;
    return (size_t)c->B * Hq * max_ns * (c->d + 2) * sizeof(float);
}

swa_status swa_decode(const swa_cache *c, const void *Q, void *O, int G, void *workspace, size_t ws_bytes,
                      void *hip_stream)
{
    clear_error();
    return decode_impl(c, Q, O, nullptr, nullptr, G, workspace, ws_bytes, hip_stream);
}

swa_status swa_decode_noalloc(const swa_cache *c, const void *Q, void *O, int G, void *hip_stream)
{
    clear_error();
    return decode_impl(c, Q, O, nullptr, nullptr, G, nullptr, 0, hip_stream, nullptr, nullptr, true);
}

swa_status swa_decode_lsink(const swa_cache *c, const void *Q, void *O, const float *sink_logit, int G,
                            void *workspace, size_t ws_bytes, void *hip_stream)
{
    clear_error();
    if (!sink_logit) return fail(SWA_ERR_INVALID_ARG, "sink_logit must not be NULL");
    return decode_impl(c, Q, O, sink_logit, nullptr, G, workspace, ws_bytes, hip_stream);
}

swa_status swa_decode_step(swa_cache *c, const void *K_new, const void *V_new, const void *Q, void *O,
                           const float *sink_logit, int G, void *workspace, size_t ws_bytes, void *hip_stream)
{
    clear_error();
    swa_status st = check_cache(c);
    if (st != SWA_OK) return st;
    if (!K_new || !V_new) return fail(SWA_ERR_INVALID_ARG, "K_new and V_new must not be NULL");
    if (!aligned16(K_new) || !aligned16(V_new)) return fail(SWA_ERR_INVALID_ARG, "K_new and V_new must be 16-byte aligned");
    if (c->dt == SWA_FP8_E4M3)
        return fail(SWA_ERR_UNSUPPORTED, "an SWA_FP8_E4M3 cache takes swa_cache_append_fp8 and swa_decode_fp8");
    if (c->n == INT64_MAX) return fail(SWA_ERR_STATE, "position count would overflow");
    if (c->dt == SWA_F32) {
        // no fused fp32 kernel: the append and the decode, one launch each
        if (sink_logit && ((uintptr_t)sink_logit & 3u))
            return fail(SWA_ERR_INVALID_ARG, "sink_logit must be 4-byte aligned");
        swa_cache t = *c;
        if ((st = check_group(G)) != SWA_OK) return st;
        if (!Q || !O || !aligned16(Q) || !aligned16(O))
            return fail(SWA_ERR_INVALID_ARG, "Q and O must be non-NULL and 16-byte aligned");
        t.n += 1;
        const size_t need = swa_decode_workspace_bytes(&t, G);
        if (need && (!workspace || ws_bytes < need))
            return fail(SWA_ERR_INVALID_ARG, "decode needs a workspace of %zu bytes (got %zu)", need,
                        workspace ? ws_bytes : (size_t)0);
        if ((st = swa_cache_append(c, K_new, V_new, 1, hip_stream)) != SWA_OK) return st;
        return decode_impl(c, Q, O, sink_logit, nullptr, G, workspace, ws_bytes, hip_stream);
    }
    st = decode_impl(c, Q, O, sink_logit, nullptr, G, workspace, ws_bytes, hip_stream, K_new, V_new);
    if (st == SWA_OK) c->n += 1;
    return st;
}

swa_status swa_decode_fp8(const swa_cache *c, const void *Q, void *O, const float *kv_scale, const float *sink_logit,
                          int G, void *workspace, size_t ws_bytes, void *hip_stream)
{
    clear_error();
    swa_status st = check_scale(kv_scale);
    if (st != SWA_OK) return st;
    return decode_impl(c, Q, O, sink_logit, kv_scale, G, workspace, ws_bytes, hip_stream);
}

}  // extern "C"
