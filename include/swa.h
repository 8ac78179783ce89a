/*
 * swa.h -- C ABI of libswa: SWA(w,s) sliding-window softmax attention with
 * attention sinks on AMD Instinct MI355X (gfx950).
 *
 * The method (paper.rainbus.top summary of arXiv 2608.28444, section
 * "滑窗注意力 SWA(w, s)" with its windowed-softmax equation, and method steps,
 * step 2; ai-blog.deepmagic.app post, section "他們測了什麼"): a query at
 * 1-based position t attends the first s tokens and the most recent w-s
 * tokens, itself included,
 *
 *     S_t = { i : 1 <= i <= min(s,t) } U { i : max(s+1, t-w+s+1) <= i <= t },
 *
 * so |S_t| = min(t, w), and the softmax of q_t.k_i / sqrt(d) is normalised
 * over S_t only (d = head dimension).  s = 0 is the plain windowed softmax;
 * w >= t makes the row full causal attention.  The KV cache then stops growing
 * at w rows per (sequence, kv-head) (same summary, "KV 缓存" background
 * section; 163.com article, section "研究方法"): s pinned sink slots plus a
 * (w-s)-slot ring buffer.
 *
 * Conventions shared by every call
 * --------------------------------
 * - Inputs are post-RoPE; positions are implicit (row t of a prefill is
 *   position t, a cache counts its own appended positions).
 * - Grouped-query attention: Hq query heads share Hkv key/value heads, query
 *   head h reads kv head h / (Hq/Hkv).  Supported Hq/Hkv: 1, 2, 4, 8.
 * - Head dimension d: 64 or 128.  dtype: SWA_BF16 or SWA_F32; inputs, outputs
 *   and cache share one dtype (an fp8 cache, with bf16 inputs and outputs,
 *   has calls of its own).  bf16 inputs use bf16 MFMA with fp32
 *   accumulation and fp32 softmax; f32 uses fp32 MFMA throughout.
 * - Every tensor is dense row-major with the layout given below, in device
 *   memory, 16-byte aligned.  The caller owns all memory; the library never
 *   allocates, frees or retains device memory.
 * - Every call that touches the device enqueues on `hip_stream` (a
 *   hipStream_t; NULL = the default stream) and returns without waiting.
 * - Errors: argument and state errors are found before anything is enqueued;
 *   then no memory is touched, the return value says what kind of error it
 *   was and swa_last_error() gives a message.  A failed kernel launch returns
 *   SWA_ERR_HIP.  No call aborts and no C++ exception crosses this boundary.
 */
#ifndef SWA_H
#define SWA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    SWA_OK = 0,
    SWA_ERR_INVALID_ARG = 1, /* null/misaligned pointer, bad size, s >= w, ...      */
    SWA_ERR_UNSUPPORTED = 2, /* a valid value the library has no kernel for (d=96) */
    SWA_ERR_HIP = 3,         /* the HIP runtime reported an error                   */
    SWA_ERR_STATE = 4        /* e.g. decode on an empty cache                       */
} swa_status;

/* SWA_FP8_E4M3 is a cache element type only (see swa_cache_append_fp8). */
typedef enum { SWA_F32 = 0, SWA_BF16 = 1, SWA_FP8_E4M3 = 2 } swa_dtype;

/*
 * Prefill: every row of a prompt attends its own S_t.
 *   O[b,t,h,:] = sum_{i in S_t} softmax_i(Q[b,t,h,:].K[b,i,h/G,:]/sqrt(d)) V[b,i,h/G,:]
 * Passage: the windowed-softmax equation of the SWA(w,s) section cited above,
 * with the sum running over S_t.
 *
 *   Q : [B, L, Hq, d]   K, V : [B, L, Hq/G, d]   (dtype in_dt)
 *   O : [B, L, Hq, d]   (dtype out_dt)
 *   G : query heads per kv-head (grouped-query attention); query head h reads
 *       kv-head h/G.  G in {1, 2, 4, 8}, Hq a multiple of G.
 *   out_dt : in_dt, or SWA_F32 for SWA_BF16 inputs (the fp32 normalised
 *       output, before the bf16 rounding of the plain bf16 path).
 *   lse  : optional (NULL = not written), fp32 [B, Hq, L],
 *          lse[b,h,t] = ln sum_{i in S_t} exp(Q.K/sqrt(d))
 *   B >= 1, L >= 0 (L = 0 enqueues nothing), w > s >= 0 (w >= L is full causal).
 * Q, K, V are read only; O (and lse) are written in full.
 */
swa_status swa_prefill(const void *Q, const void *K, const void *V, void *O, float *lse,
                       int B, int L, int Hq, int G, int d, int w, int s,
                       swa_dtype in_dt, swa_dtype out_dt, void *hip_stream);

/*
 * Learned-sink variant of swa_prefill: sink_logit (device, fp32, [Hq]) adds
 * one more term e^{sink_logit[h]} to the softmax denominator of every row of
 * query head h, with no value vector; lse includes it.  The reading of the
 * pages' "SWA (learned sink)" student (the Hugging Face follow-up story's
 * Qwen3-4B study), which they do not define further.  Logits must be finite
 * or -INFINITY (no term).  sink_logit must not be NULL; other arguments and
 * errors as swa_prefill.
 */
swa_status swa_prefill_lsink(const void *Q, const void *K, const void *V, void *O, float *lse,
                             const float *sink_logit, int B, int L, int Hq, int G, int d, int w, int s,
                             swa_dtype in_dt, swa_dtype out_dt, void *hip_stream);

/*
 * The constant-size cache of one layer.  Plain data owned by the caller: the
 * two buffers k and v, each [B, Hkv, w, d] of dtype dt, and the host-side
 * count n of positions appended so far (n grows without bound; the buffers do
 * not).  1-based position p is stored in slot swa_cache_slot(w, s, p) of its
 * (b, kv-head); after n appends the occupied slots 0..min(n,w)-1 hold exactly
 * the positions of S_n.  Copying the two buffers and n snapshots the cache.
 */
typedef struct {
    void *k;
    void *v;
    int64_t n;
    int B, Hkv, d, w, s;
    swa_dtype dt;
} swa_cache;

/* Fills *c (n = 0).  Does not touch the buffers: slots are written before
 * they are read.  Errors: null c/k_buf/v_buf, misalignment, bad sizes. */
swa_status swa_cache_init(swa_cache *c, void *k_buf, void *v_buf, int B, int Hkv, int d,
                          int w, int s, swa_dtype dt);

/*
 * Appends positions n+1 .. n+n_new of every sequence.  Passage: the cache
 * policy of the paper.rainbus.top summary ("KV 缓存" background section and
 * "滑窗注意力 SWA(w, s)": the cache holds only the s sinks and the most recent
 * w - s tokens, so it stops growing at w rows) and of the 163.com article
 * ("研究方法": the window evicts the older tokens, the sinks stay).
 *   K_new, V_new : [B, n_new, Hkv, d] in c->dt, read only.
 *   Only the rows that are still in S_{n+n_new} are written, each to
 *   swa_cache_slot(w, s, p) of its (b, kv-head) (a bulk append longer than
 *   the ring leaves the same cache as appending one position at a time).
 *   c->n is advanced on the host at enqueue time; later calls on the same
 *   stream see the new rows.  n_new >= 1.
 * Ownership: the caller keeps K_new/V_new alive until the stream has run the
 * call.  Errors: SWA_ERR_INVALID_ARG for a bad cache, NULL or misaligned
 * rows, n_new < 1; SWA_ERR_UNSUPPORTED for an fp8 cache (it takes
 * swa_cache_append_fp8); SWA_ERR_STATE if c->n would overflow.  On error
 * nothing is enqueued and c is unchanged.
 */
swa_status swa_cache_append(swa_cache *c, const void *K_new, const void *V_new, int n_new,
                            void *hip_stream);

/*
 * Decode: the query rows at position n = c->n attend S_n, i.e. every occupied
 * slot of the cache (slot order does not matter to a softmax).  Passage: the
 * windowed-softmax equation of the paper.rainbus.top summary's SWA(w, s)
 * section, evaluated for the newest position over the constant-size cache
 * of its "KV 缓存" section (ai-blog.deepmagic.app, "他們測了什麼": the method
 * changes only the mask and which cache rows are kept).
 *   Q, O : [B, G * c->Hkv, d], dtype c->dt; G query heads share each kv-head
 *          (G in {1, 2, 4, 8}).
 *   workspace : device scratch of at least swa_decode_workspace_bytes(c, G)
 *               bytes when that is non-zero (long windows are split over
 *               several workgroups whose partial results meet there); may be
 *               NULL when the size is 0.  Not retained after the stream has
 *               run the call.
 * Errors: SWA_ERR_STATE if c->n == 0; SWA_ERR_INVALID_ARG if the workspace is
 * needed but missing or smaller than required.
 */
swa_status swa_decode(const swa_cache *c, const void *Q, void *O, int G,
                      void *workspace, size_t ws_bytes, void *hip_stream);

/*
 * swa_decode without a workspace, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc).  Same arguments, results and errors as swa_decode; when
 * the decode splits a long window over workgroups, the partial results go to
 * a fixed array inside the library instead: 2 MiB per GPU (each GPU the
 * library runs on holds its own copy until the process ends), enough for
 * B * Hq * nsplit * (d + 2) * 4 bytes of partials (every batch-1 and
 * batch-16 window at d = 128, G = 4, for example).  A call that would need
 * more returns SWA_ERR_UNSUPPORTED with nothing enqueued.  The call
 * allocates nothing and frees nothing.  The stream must belong to the
 * current device (SWA_ERR_INVALID_ARG otherwise).
 * All calls on one GPU share that GPU's array, and each split's partial is
 * written in full before it is read (nothing in it needs clearing): two such
 * calls that can run at the same time on one GPU (different streams) race;
 * calls on one stream do not.
 */
swa_status swa_decode_noalloc(const swa_cache *c, const void *Q, void *O, int G, void *hip_stream);

/*
 * Chunked prefill / multi-query decode against the cache: C new positions
 * n+1 .. n+C (n = c->n) each attend their own S_t -- cached positions (all
 * in the ring, since S_t minus the chunk is a subset of S_n) and the chunk's
 * positions up to t -- and then the chunk is appended (c->n becomes n + C).
 * This serves prompts longer than w a chunk at a time and verifies several
 * draft tokens per step.  Passage: the windowed-softmax equation of the
 * SWA(w,s) section and the cache policy ("KV 缓存") cited above; the
 * result equals rows n+1..n+C of swa_prefill over all n + C positions.
 *   Q, O : [B, C, G * c->Hkv, d]     K_new, V_new : [B, C, c->Hkv, d]
 *   Q, K_new, V_new in c->dt; O in out_dt (c->dt, or SWA_F32 for bf16).
 *   lse  : optional fp32 [B, G * c->Hkv, C], as for swa_prefill.
 * Two launches (the attention, then the append) in general.  A bf16 chunk
 * with bf16 O, no lse and C * G <= 16 whose cache the decode kernel reads
 * without splitting it takes one launch of that kernel instead (chunk rows
 * as extra query columns; it also writes the chunk into the ring); same
 * results, to rounding.
 * Errors as swa_prefill and swa_cache_append; nothing is enqueued and c is
 * untouched on a rejected call.
 */
swa_status swa_prefill_chunk(swa_cache *c, const void *Q, const void *K_new, const void *V_new, void *O,
                             float *lse, int C, int G, swa_dtype out_dt, void *hip_stream);

/*
 * One generation step in one launch: swa_cache_append of one position
 * (K_new, V_new : [B, c->Hkv, d], i.e. [B, 1, Hkv, d]) followed by swa_decode
 * (swa_decode_lsink when sink_logit is not NULL) at the new position, with
 * the same results and cache contents as those two calls.  The new rows are
 * attended from K_new/V_new and written to their slot by the same kernel.
 * c->n is advanced on success.  A bf16 cache runs the fused kernel; an fp32
 * cache runs the two calls; an fp8 cache is SWA_ERR_UNSUPPORTED.
 * Workspace: swa_decode_workspace_bytes(c, G).  Errors as the two calls;
 * nothing is enqueued and c is untouched on a rejected call.
 */
swa_status swa_decode_step(swa_cache *c, const void *K_new, const void *V_new, const void *Q, void *O,
                           const float *sink_logit, int G, void *workspace, size_t ws_bytes, void *hip_stream);

/* Learned-sink variant of swa_decode (see swa_prefill_lsink): sink_logit is
 * device fp32 [G * c->Hkv]; the term joins the final normalisation once,
 * also when the rows are split over workgroups. */
swa_status swa_decode_lsink(const swa_cache *c, const void *Q, void *O, const float *sink_logit, int G,
                            void *workspace, size_t ws_bytes, void *hip_stream);

/*
 * fp8 KV cache: SWA(w,s) combined with KV-cache quantisation (one of the
 * follow-up directions of the paper.rainbus.top summary, limitations and
 * outlook section).  A cache made by swa_cache_init with dt = SWA_FP8_E4M3
 * holds one byte per element in k and v ([B, Hkv, w, d]): the OCP 8-bit
 * floating-point E4M3 code of clamp(x / scale, -448, 448), where x / scale
 * is the correctly rounded fp32 quotient and the code is the nearest E4M3
 * value, ties to the even code.  Reading gives code value * scale.
 *   kv_scale : device fp32 [2, c->Hkv] -- the K scale of each kv-head, then
 *              the V scale.  Positive and finite (not checked: other values
 *              give meaningless results, never a fault).  The same scales must
 *              be passed to every call on one cache.  Read while the stream
 *              runs the call; not retained.
 * Only the two calls below take such a cache; swa_cache_append, swa_decode,
 * swa_decode_lsink and swa_prefill_chunk return SWA_ERR_UNSUPPORTED for it,
 * and these two return SWA_ERR_INVALID_ARG for any other cache.
 */

/* swa_cache_append with quantisation: K_new, V_new are bf16 [B, n_new, Hkv, d]. */
swa_status swa_cache_append_fp8(swa_cache *c, const void *K_new, const void *V_new, int n_new,
                                const float *kv_scale, void *hip_stream);

/* swa_decode over the dequantised cache: Q, O bf16 [B, G * c->Hkv, d].
 * sink_logit: NULL, or device fp32 [G * c->Hkv] as for swa_decode_lsink.
 * Workspace as for swa_decode.  Scores and sums are fp32; K and V enter the
 * bf16 MFMAs as their codes' values (exact in bf16), the K scale joins the
 * softmax scale and the V scale multiplies the output. */
swa_status swa_decode_fp8(const swa_cache *c, const void *Q, void *O, const float *kv_scale,
                          const float *sink_logit, int G, void *workspace, size_t ws_bytes,
                          void *hip_stream);

/*
 * Ragged and paged batches for serving.  The summary's limitations
 * (paper.rainbus.top, limitations and outlook) leave paged KV management and
 * large-batch serving of SWA untested; here they are a storage layout and a
 * batching of the same SWA(w,s) computation: every sequence gets exactly
 * what the calls above give it alone.
 *
 * Varlen prefill: B prompts of different lengths packed along the row axis.
 *   Q, O : [total, Hq, d]      K, V : [total, Hkv, d]
 *   cu_seqlens : device int32 [B + 1]; sequence b is rows cu_seqlens[b] ..
 *                cu_seqlens[b+1] - 1 (cu_seqlens[0] = 0, non-decreasing,
 *                cu_seqlens[B] = total).  Rows outside [0, total) are never
 *                touched, whatever the array holds.
 *   max_len : host int >= the longest sequence (it sizes the grid; blocks
 *             past a sequence's end do nothing).
 *   lse : optional fp32 [Hq, total].
 * dtypes as swa_prefill.
 */
swa_status swa_prefill_varlen(const void *Q, const void *K, const void *V, void *O, float *lse,
                              const int32_t *cu_seqlens, int B, int total, int max_len, int Hq, int G,
                              int d, int w, int s, swa_dtype in_dt, swa_dtype out_dt, void *hip_stream);

/*
 * Paged cache: the dense cache's w slots of each sequence live in pages of
 * `page` slots taken from shared pools, and each sequence has its own
 * position count, kept on the device.
 *   k_pool, v_pool : [num_pages, Hkv, page, d] each, bf16.
 *   block_table : device int32 [B, pages_per_seq], pages_per_seq =
 *                 ceil(w / page): slot j of sequence b (numbered as by
 *                 swa_cache_slot) is row j % page of page
 *                 block_table[b * pages_per_seq + j / page].
 *   n : device int64 [B], positions appended to each sequence so far
 *       (0 = empty).  swa_paged_append advances it on the stream; the
 *       caller may reset an entry (with its pages) to reuse a batch row.
 *   page : a multiple of 32, at most 4096.
 * The caller owns the pools and tables and may change table entries between
 * calls.  Every entry that a call reaches (the pages of slots
 * 0 .. min(n[b], w) - 1 after the call) must name a page in
 * [0, num_pages) not used by another sequence; an entry outside the pool is
 * never dereferenced: its rows are not written and read as zeros (the output
 * is then meaningless, but nothing faults).
 */
typedef struct {
    void *k_pool;
    void *v_pool;
    const int32_t *block_table;
    int64_t *n;
    int B, num_pages, page, pages_per_seq, Hkv, d, w, s;
    swa_dtype dt;
} swa_paged_cache;

/* Fills *c (pages_per_seq computed).  Touches no device memory. */
swa_status swa_paged_cache_init(swa_paged_cache *c, void *k_pool, void *v_pool, const int32_t *block_table,
                                int64_t *n, int B, int num_pages, int page, int Hkv, int d, int w, int s,
                                swa_dtype dt);

/* Appends cu_seqlens[b+1] - cu_seqlens[b] new positions to each sequence b
 * (zero allowed) from K_new, V_new [total, Hkv, d] packed as for
 * swa_prefill_varlen (cu_seqlens[0] = 0, non-decreasing, cu_seqlens[B] =
 * total); as for swa_cache_append, only the rows still attended after the
 * append are written.  Then n[b] grows by that count.  Rows outside
 * [cu_seqlens[0], cu_seqlens[B]) and rows that fall past their sequence's
 * end in a table that is not non-decreasing are never written. */
swa_status swa_paged_append(const swa_paged_cache *c, const void *K_new, const void *V_new,
                            const int32_t *cu_seqlens, int total, void *hip_stream);

/* Decode of every sequence at its own position n[b]: Q, O [B, G * c->Hkv, d]
 * bf16; sequence b attends its min(n[b], w) occupied slots.  A sequence with
 * n[b] == 0 gets O = 0.  sink_logit: NULL or device fp32 [G * c->Hkv] as for
 * swa_decode_lsink.  Workspace: swa_paged_decode_workspace_bytes(c, G). */
swa_status swa_paged_decode(const swa_paged_cache *c, const void *Q, void *O, const float *sink_logit, int G,
                            void *workspace, size_t ws_bytes, void *hip_stream);

size_t swa_paged_decode_workspace_bytes(const swa_paged_cache *c, int G);

/*
 * Chunked prefill against a paged cache: sequence b's C_b = cu_seqlens[b+1] -
 * cu_seqlens[b] new positions n[b]+1 .. n[b]+C_b (zero allowed) each attend
 * their own S_t -- the cached positions, all still in b's pages, and b's
 * chunk rows up to t -- and then every sequence's chunk is appended as by
 * swa_paged_append (n[b] grows by C_b).  swa_prefill_chunk for a batch whose
 * sequences sit at different positions, as a serving loop mixes them.
 * Passage: the windowed-softmax equation and the cache policy cited at
 * swa_prefill_chunk; the result equals rows n[b]+1 .. n[b]+C_b of
 * swa_prefill over sequence b's n[b] + C_b positions.
 *   Q, O : [total, G * c->Hkv, d]   K_new, V_new : [total, c->Hkv, d]
 *   packed as for swa_prefill_varlen (cu_seqlens: device int32 [B + 1],
 *   cu_seqlens[0] = 0, non-decreasing, cu_seqlens[B] = total); Q, K_new,
 *   V_new bf16; O bf16 or, with out_dt = SWA_F32, fp32.
 *   max_chunk : host int >= the longest chunk (it sizes the grid).
 *   lse : optional fp32 [G * c->Hkv, total].
 * Reads n[b] and the block table on the device, so the counts may come from
 * earlier calls still in the stream.  Errors as swa_prefill_varlen and
 * swa_paged_append; nothing is enqueued on a rejected call.
 */
swa_status swa_paged_prefill_chunk(const swa_paged_cache *c, const void *Q, const void *K_new, const void *V_new,
                                   void *O, float *lse, const int32_t *cu_seqlens, int total, int max_chunk, int G,
                                   swa_dtype out_dt, void *hip_stream);

/* Workspace swa_decode needs for this cache and group size, for any n
 * (the split plan is sized for a full window).  0 means none. */
size_t swa_decode_workspace_bytes(const swa_cache *c, int G);

/* 0-based slot of 1-based position p: p-1 for p <= s, else
 * s + ((p-s-1) mod (w-s)).  Returns -1 for p < 1 or invalid (w, s).
 * Passage: the pages fix only that the cache keeps the s sinks and the
 * w - s most recent tokens in constant space (paper.rainbus.top summary, "KV
 * 缓存" and "滑窗注意力 SWA(w, s)"; 163.com article, "研究方法"); this slot
 * map is the ring that realises it: sinks pinned, and a new position
 * overwrites exactly the one that has just left the window.  Pure host
 * function, no device access. */
int64_t swa_cache_slot(int w, int s, int64_t p);

/* |S_t| = min(t, w).  Returns -1 for t < 1 or invalid (w, s).  Passage:
 * the attended set of the paper.rainbus.top summary's SWA(w, s) section
 * (w counts the s sinks) and ai-blog.deepmagic.app, "他們測了什麼" (SWA(64,4):
 * 4 sinks and 60 recent tokens).  Pure host function. */
int64_t swa_attended_count(int w, int s, int64_t t);

/* Message for the last error on the calling thread ("" if none).  Valid until
 * the next libswa call on that thread. */
const char *swa_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* SWA_H */
