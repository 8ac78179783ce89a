// Internal interface between the C ABI (api.cpp) and the HIP kernels.
// Not installed; the public surface is include/swa.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace swa {

enum class Dt { F32 = 0, BF16 = 1, FP8 = 2 };  // FP8: OCP E4M3 cache elements

// Paged cache with one position count per sequence.  Sequence b's slot j
// (the dense cache's slot numbering) lives in row j % page of page
// block_table[b * pages_per_seq + j / page]; a page holds [Hkv, page, d].
struct PagedParams {
    void *Kp = nullptr, *Vp = nullptr;     // page pools [num_pages, Hkv, page, d]
    const int32_t *block_table = nullptr;  // [B, pages_per_seq]
    int64_t *n = nullptr;                  // [B] positions appended so far
    int num_pages = 0, page = 0, pages_per_seq = 0;
};

struct PrefillParams {
    const void *Q, *K, *V;
    void *O;
    float *lse;   // nullable, [B, Hq, L]
    int B, L, Hq, Hkv, w, s;
    const float *sink_logit = nullptr;  // nullable, [Hq]: learned-sink logit per query head
    // Chunk mode only (rows are positions n+1..n+L after a cache of n):
    const void *Kc = nullptr, *Vc = nullptr;  // cache buffers [B, Hkv, w, d]
    int nvalid = 0;     // occupied slots, min(n, w)
    int sinks_in = 0;   // sink slots filled, min(s, n)
    int ring_head = 0;  // ring index of position n, (n-s-1) mod (w-s), when n > s
    int ring_full = 0;  // n - s >= w - s
    int ring_any = 0;   // n > s
    int sk = 0;         // sink positions inside the chunk, clamp(s - n, 0, L)
    // Varlen mode: B sequences packed along the row axis (Q, O [total, Hq, d];
    // K, V [total, Hkv, d]); sequence b is rows cu_seqlens[b] .. cu_seqlens[b+1]-1
    // and L is the longest; lse is [Hq, total].
    const int32_t *cu_seqlens = nullptr;
    int total = 0;
    // Paged chunk mode (with varlen rows): the cache is the page pools, and
    // sequence b follows its own n[b] (the fields nvalid .. sk above unused).
    PagedParams pg;
};

struct PagedAppendParams {
    PagedParams c;
    const void *Kn, *Vn;         // [total, Hkv, d], sequence b's rows at cu_seqlens[b]..
    const int32_t *cu_seqlens;   // [B + 1]
    int B, Hkv, w, s, total;
};

struct AppendParams {
    const void *Kn, *Vn;  // [B, n_new, Hkv, d]
    void *Kc, *Vc;        // [B, Hkv, w, d]
    int B, Hkv, w, s, n_new;
    int64_t n_before;     // positions already in the cache
    // survivors: 1-based positions [a1, b1] and [a2, b2] (empty when a > b)
    int64_t a1, b1, a2, b2;
    const float *kv_scale = nullptr;  // fp8 cache: [2, Hkv] (K scales, then V scales)
    // Filled by the launcher from the ranges above (32-bit, so the kernel does
    // no 64-bit division): survivor counts, first source rows and first slots.
    int n1 = 0, n2 = 0, src1 = 0, src2 = 0, slot1 = 0, slot2 = 0;
};

struct DecodeParams {
    const void *Kc, *Vc;  // [B, Hkv, w, d]
    const void *Q;        // [B, Hq, d]
    void *O;              // [B, Hq, d]
    float *part;          // split partials, [B*Hq, nsplit, d + 2] fp32; null if nsplit == 1
    int B, Hq, Hkv, w;
    int nvalid;           // occupied slots = min(n, w)
    int nsplit, rows_per_split;
    int pairs_per_wg;     // bf16 kernel: (b, kv-head, split) tasks per workgroup (1, 2 or 4)
    int waves_per_wg = 4; // bf16 kernel: 4, or 8 or 16 (then one task per workgroup)
    const float *sink_logit = nullptr;  // nullable, [Hq]: learned-sink logit per query head
    const float *kv_scale = nullptr;    // fp8 cache: [2, Hkv] (K scales, then V scales)
    // Paged kernel only: rows come from the page pools through the block
    // table, and sequence b attends min(pg.n[b], w) slots (nvalid unused).
    PagedParams pg;
    // Fused step only: the new position's rows [B, Hkv, d] and the slot they
    // go to; the kernel reads them in place of that slot and writes them there.
    // Multi-query decode: the chunk's rows [B, mq_c, Hkv, d].
    const void *Kn = nullptr, *Vn = nullptr;
    int new_slot = -1;
    // Multi-query decode only (a chunk of mq_c rows after a cache of n0
    // positions, Q and O [B, mq_c, Hq, d]): the sinks s and the ring offset
    // of position n0 (ring_head, when n0 > s).
    int mq_c = 0, s = 0, ring_head = 0;
    int64_t n0 = 0;
};

hipError_t launch_prefill(Dt in, Dt out, int d, int G, const PrefillParams &p, hipStream_t st);
// Varlen mode (p.cu_seqlens set): grid over the longest sequence, p.L = its length.
hipError_t launch_prefill_varlen(Dt in, Dt out, int d, int G, const PrefillParams &p, hipStream_t st);
// Paged cache: survivors of each sequence's new rows into their slots, then n[b] += its count.
hipError_t launch_paged_append(Dt dt, int d, const PagedAppendParams &p, hipStream_t st);
// Chunk mode: rows attend the cache described by p.Kc.. plus the chunk itself.
hipError_t launch_prefill_chunk(Dt in, Dt out, int d, int G, const PrefillParams &p, hipStream_t st);
// Paged chunk mode: bf16 rows and pools, varlen chunk rows (p.cu_seqlens), each
// sequence after its own n[b] (p.pg.n).
hipError_t launch_prefill_chunk_paged(Dt out, int d, int G, const PrefillParams &p, hipStream_t st);
hipError_t launch_append(Dt dt, int d, const AppendParams &p, hipStream_t st);
hipError_t launch_decode(Dt dt, int d, int G, const DecodeParams &p, hipStream_t st);
// bf16 paged cache (p.pg), per-sequence position counts.
hipError_t launch_decode_paged(int d, int G, const DecodeParams &p, hipStream_t st);
// bf16 cache: append one position (p.Kn, p.Vn into p.new_slot) and decode, in one launch.
hipError_t launch_decode_step(int d, int G, const DecodeParams &p, hipStream_t st);
// bf16 cache, no splits (p.nsplit == 1, one task per workgroup): rows n0+1..n0+mq_c
// attend the cache and the chunk (p.Kn, p.Vn) up to themselves, then the
// chunk's rows go into their slots; p.mq_c * G <= 16.
hipError_t launch_decode_mq(int d, int G, const DecodeParams &p, hipStream_t st);

// Fixed per-GPU scratch of swa_decode_noalloc (split partials).  Returns the
// device address of the array on `device`, which must be the current device;
// the address is looked up on the first call for that device and kept.
constexpr size_t kDecodeScratchBytes = 2u << 20;
constexpr int kMaxDevices = 64;
hipError_t decode_scratch(int device, void **ptr);

// Cache rows per chunk of the decode kernel (one MFMA step of keys); the
// planner sizes splits in whole chunks.
constexpr int kDecodeChunk = 32;

// Split plan for decode: how many workgroups share one (b, kv-head) and how
// many cache rows each takes.  max_splits bounds nsplit for every nvalid up
// to the given one (it sizes the workspace).
// allow16: the cache's kernel may take 16-wave workgroups (bf16 caches).
void decode_plan(int B, int Hkv, int nvalid, int *nsplit, int *rows_per_split, int *max_splits,
                 int *pairs_per_wg, int *waves_per_wg, bool allow16);

}  // namespace swa
