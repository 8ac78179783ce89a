// SWA(w,s) decode and cache append on gfx950.
//
// The cache of one (batch, kv-head) is a w x d block: s pinned sink slots and
// a (w - s)-slot ring.  After n appends its occupied slots 0..min(n,w)-1 hold
// exactly the positions the query at position n attends (the first s tokens
// plus the most recent w - s; paper.rainbus.top summary of arXiv 2608.28444,
// "滑窗注意力 SWA(w, s)" and "KV 缓存"; ai-blog.deepmagic.app, "他們測了什麼":
// SWA alters only the mask and which cache rows are kept).  A
// softmax does not depend on the order of its terms, so decode reads the
// occupied slots in physical order with no mask and no un-rotation.
//
// Decode is bound by HBM: per step it reads 2*min(n,w)*d elements per
// (batch, kv-head) and does 4*G*d flops per cached row (G query heads share
// each row).  Waves of a workgroup walk interleaved row blocks of the same
// (batch, kv-head) and meet in LDS; long caches are further split over
// workgroups whose partial (max, sum, acc) triples a second kernel merges:
//     O = sum_j e^{m_j-M} acc_j / sum_j e^{m_j-M} l_j.
// bf16 and fp8 caches use the MFMA kernel further down (swa_decode_mfma_kernel,
// which also has the paged and the fused append + decode modes).  An fp32
// cache uses the VALU kernel next: LPR lanes cover one cached row with 16-byte
// loads, so each load instruction of a wave reads 64/LPR whole rows; each lane
// keeps the G query vectors for its d/LPR dims in registers, and the score of
// a row is a partial dot product reduced over the LPR lanes of the row.
#include <mutex>
#include <type_traits>

#include "device_common.h"
#include "swa_internal.h"

namespace swa {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kUnroll = 4;

template <typename T> __device__ __forceinline__ void unpack16(const u32x4 &raw, float *out);
template <> __device__ __forceinline__ void unpack16<bf16>(const u32x4 &raw, float *out)
{
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        out[2 * i] = __uint_as_float(raw[i] << 16);
        out[2 * i + 1] = __uint_as_float(raw[i] & 0xffff0000u);
    }
}
template <> __device__ __forceinline__ void unpack16<float>(const u32x4 &raw, float *out)
{
#pragma unroll
    for (int i = 0; i < 4; ++i) out[i] = __uint_as_float(raw[i]);
}

typedef short shortx4 __attribute__((ext_vector_type(4)));

template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float x) { return (bf16)x; }
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }

// Learned-sink logit of query head hq in the log2 units of the partial maxima
// (-inf when there is none): one more term e^b in the final denominator.
__device__ __forceinline__ float sink_log2(const DecodeParams &p, int hq)
{
    return p.sink_logit ? p.sink_logit[hq] * 1.4426950408889634f : -INFINITY;
}

template <typename T, int D, int G>
__global__ __launch_bounds__(kThreads) void swa_decode_valu_kernel(DecodeParams p)
{
    constexpr int EPL = 16 / (int)sizeof(T);  // elements per lane per row
    constexpr int LPR = D / EPL;              // lanes per cached row
    constexpr int RPI = 64 / LPR;             // rows per load instruction
    constexpr int RW = RPI * kUnroll;         // rows per wave per trip
    constexpr int RG = RW * kWaves;           // rows per workgroup per trip

    __shared__ float sh_acc[kWaves][G][D];
    __shared__ float sh_ml[kWaves][G][2];

    const int sp = blockIdx.x;         // split index
    const int bh = blockIdx.y;         // b * Hkv + kv-head
    const int b = bh / p.Hkv, hkv = bh % p.Hkv;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int r = lane / LPR, c = lane % LPR;

    const int lo = sp * p.rows_per_split;
    const int hi = min(p.nvalid, lo + p.rows_per_split);

    const size_t block = (size_t)bh * p.w * D;
    const T *Kc = (const T *)p.Kc + block + c * EPL;
    const T *Vc = (const T *)p.Vc + block + c * EPL;

    // queries, pre-scaled so scores come out in log2 units
    const float qscale = 1.4426950408889634f * rsqrtf((float)D);
    float q[G][EPL];
#pragma unroll
    for (int g = 0; g < G; ++g) {
        const T *qp = (const T *)p.Q + ((size_t)b * p.Hq + hkv * G + g) * D + c * EPL;
        float tmp[8];
        unpack16<T>(*(const u32x4 *)qp, tmp);
#pragma unroll
        for (int e = 0; e < EPL; ++e) q[g][e] = tmp[e] * qscale;
    }

    float m[G], l[G], acc[G][EPL];
#pragma unroll
    for (int g = 0; g < G; ++g) {
        m[g] = -INFINITY;
        l[g] = 0.f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[g][e] = 0.f;
    }

    for (int row0 = lo + RW * wave; row0 < hi; row0 += RG) {
        u32x4 kr[kUnroll], vr[kUnroll];
        bool ok[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int row = row0 + u * RPI + r;
            ok[u] = row < hi;
            kr[u] = ok[u] ? *(const u32x4 *)(Kc + (size_t)row * D) : u32x4{0, 0, 0, 0};
            vr[u] = ok[u] ? *(const u32x4 *)(Vc + (size_t)row * D) : u32x4{0, 0, 0, 0};
        }
        float sc[kUnroll][G];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            float kf[8];
            unpack16<T>(kr[u], kf);
#pragma unroll
            for (int g = 0; g < G; ++g) {
                float a = 0.f;
#pragma unroll
                for (int e = 0; e < EPL; ++e) a = fmaf(q[g][e], kf[e], a);
#pragma unroll
                for (int x = 1; x < LPR; x <<= 1) a += __shfl_xor(a, x, 64);
                sc[u][g] = ok[u] ? a : -INFINITY;
            }
        }
        float alpha[G], muse[G];
#pragma unroll
        for (int g = 0; g < G; ++g) {
            float mx = sc[0][g];
#pragma unroll
            for (int u = 1; u < kUnroll; ++u) mx = fmaxf(mx, sc[u][g]);
#pragma unroll
            for (int x = LPR; x < 64; x <<= 1) mx = wave_max_xor(mx, x);
            const float mnew = fmaxf(m[g], mx);
            muse[g] = mnew == -INFINITY ? 0.f : mnew;
            alpha[g] = fast_exp2(m[g] - muse[g]);
            m[g] = mnew;
            l[g] *= alpha[g];
#pragma unroll
            for (int e = 0; e < EPL; ++e) acc[g][e] *= alpha[g];
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            float vf[8];
            unpack16<T>(vr[u], vf);
#pragma unroll
            for (int g = 0; g < G; ++g) {
                const float pr = fast_exp2(sc[u][g] - muse[g]);
                l[g] += pr;
#pragma unroll
                for (int e = 0; e < EPL; ++e) acc[g][e] = fmaf(pr, vf[e], acc[g][e]);
            }
        }
    }

    // combine the row groups of this wave (same dims, different rows)
#pragma unroll
    for (int g = 0; g < G; ++g) {
#pragma unroll
        for (int x = LPR; x < 64; x <<= 1) {
            l[g] += __shfl_xor(l[g], x, 64);
#pragma unroll
            for (int e = 0; e < EPL; ++e) acc[g][e] += __shfl_xor(acc[g][e], x, 64);
        }
    }
    if (r == 0) {
#pragma unroll
        for (int g = 0; g < G; ++g)
#pragma unroll
            for (int e = 0; e < EPL; ++e) sh_acc[wave][g][c * EPL + e] = acc[g][e];
    }
    if (lane == 0) {
#pragma unroll
        for (int g = 0; g < G; ++g) {
            sh_ml[wave][g][0] = m[g];
            sh_ml[wave][g][1] = l[g];
        }
    }
    __syncthreads();

    // combine the waves; one thread per (head, dim)
    for (int idx = tid; idx < G * D; idx += kThreads) {
        const int g = idx / D, dim = idx % D;
        const int hq = hkv * G + g;
        const float sl2 = p.nsplit == 1 ? sink_log2(p, hq) : -INFINITY;  // the sink joins the final sum only
        float M = sl2;
#pragma unroll
        for (int wv = 0; wv < kWaves; ++wv) M = fmaxf(M, sh_ml[wv][g][0]);
        float Ls = fast_exp2(sl2 - M), A = 0.f;  // exp2(-inf) = 0 without a sink
#pragma unroll
        for (int wv = 0; wv < kWaves; ++wv) {
            const float f = fast_exp2(sh_ml[wv][g][0] - M);
            Ls = fmaf(f, sh_ml[wv][g][1], Ls);
            A = fmaf(f, sh_acc[wv][g][dim], A);
        }
        if (p.nsplit == 1) {
            ((T *)p.O)[((size_t)b * p.Hq + hq) * D + dim] = from_f32<T>(A / Ls);
        } else {
            float *part = p.part + (((size_t)b * p.Hq + hq) * p.nsplit + sp) * (D + 2);
            part[dim] = A;
            if (dim == 0) {
                part[D] = M;
                part[D + 1] = Ls;
            }
        }
    }
}


// ---------------------------------------------------------------------------
// bf16 decode on the matrix cores.  A wave takes a task's cache rows in
// chunks of 32 and, per chunk:
//   S^T (32 keys x 16 columns) = K Q^T   : 2 x d/32 MFMA 16x16x32; the G query
//       heads of the kv-head are columns 0..G-1 (the rest are zero).  K comes
//       straight from global memory in MFMA operand layout: lane l reads key
//       l%16 (+16 for the second half), dims 8*(l/16) + 32*kk .. +8 (fp8: the
//       dims are taken in another order, so that one 16-byte load feeds two
//       steps; see kdim0).
//   online softmax per head (column), fp32, lazy rescale as in prefill.
//   O^T (d x 16) += V^T P^T              : d/16 MFMAs; V is copied to a
//       wave-private LDS tile and read back transposed (ds_read_b64_tr_b16),
//       P^T comes from the S^T accumulators.
// Cache rows at or past the task's end read as zero (buffer range) and are
// masked to -inf.  Waves of one task meet in LDS at the end; tasks split over
// several workgroups leave (max, sum, acc) partials for the merge kernel.
constexpr int kChunk = kDecodeChunk;

template <int D> struct McLayout {
    static constexpr int KK = D / 32;                   // QK contraction steps
    static constexpr int DT = D / 16;                   // PV dim tiles
    static constexpr int VROW = D * 2 + 32;             // bytes per V row in LDS (padded)
    static constexpr int VBYTES = kChunk * VROW;        // per wave
};

// Cache elements: bf16, or OCP E4M3 codes (fp8: one byte each).  fp8 values
// are exact in bf16, so the fp8 path converts on load and runs the same
// MFMAs; the per-kv-head K scale joins the softmax scale and the V scale
// multiplies O where it is written.
typedef unsigned char fp8;

template <int D, typename CT> struct ChunkRegs {
    static constexpr int VL = kChunk * D * (int)sizeof(CT) / 16 / 64;  // 16-B V loads per lane
    // K operands as loaded: 8 bf16, or 8 codes (converted just before use)
    using KRaw = std::conditional_t<sizeof(CT) == 2, bf16x8, u32x2>;
    KRaw k[2][McLayout<D>::KK];
    u32x4 v[VL];
};

// Eight E4M3 codes (two dwords, lowest byte first) to bf16 (exact): the
// scaled conversion with scale 1.0 is a plain conversion, one instruction
// per two codes (it equals v_cvt_pk_f32_fp8 followed by rounding to bf16 on
// every pair of codes).
__device__ __forceinline__ bf16x8 fp8x8_to_bf16(uint32_t lo, uint32_t hi)
{
    const bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false);
    const bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true);
    const bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false);
    const bf16x2 e = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true);
    return bf16x8{a[0], a[1], b[0], b[1], c[0], c[1], e[0], e[1]};
}

// PG: paged cache (p.pg) -- each 32-row chunk is read from the page its
// first slot maps to (pages hold a multiple of 32 rows, so a chunk never
// straddles two), and sequence b attends min(n[b], w) slots.
// FU: fused append + decode -- slot p.new_slot takes the new position's rows
// p.Kn, p.Vn: the chunk holding it reads them in place of the slot's old
// contents, and the one wave of the grid that processes that chunk for a
// (b, kv-head) writes them into the slot.  Other waves that happen to load the
// slot while it is written discard what they read, so the append needs no
// ordering against the reads.
// NWV: waves per workgroup, 4 (tasks of 1, 2 or 4 waves), 8 (one task of
// 8 waves, for few (b, kv-head) pairs: twice the waves in flight and half the
// chunks per wave) or 16 (one task of 16 waves, a chunk each, for windows of
// up to 16 chunks at small batch: the waves meet in LDS instead of splitting
// the window over workgroups and merging in a second launch).
// MQ (multi-query decode, bf16 cache, one task per workgroup, no splits):
// the MFMA columns are chunk rows x heads instead of heads alone; each row
// attends the cache slots still in its window and the chunk's rows up to
// itself, and the workgroup writes the chunk's rows into their slots at the end.
template <int D, int G, typename CT, bool PG = false, bool FU = false, int NWV = 4, bool MQ = false>
__global__ __launch_bounds__(64 * NWV, NWV == 4 ? 3 : 1) void swa_decode_mfma_kernel(DecodeParams p)
{
    constexpr int kWaves = NWV;
    using Lay = McLayout<D>;
    using Regs = ChunkRegs<D, CT>;
    constexpr int ES = sizeof(CT);
    constexpr float kLazy = 8.f;
    constexpr int NCOL = MQ ? 16 : G;  // MFMA columns that can hold a query row
    static_assert(!MQ || (ES == 2 && !PG && !FU), "multi-query decode: bf16, unpaged, no fused step");
    // With 16 waves the per-wave V tiles fill most of the LDS; each wave then
    // leaves its accumulators in its own tile (which only it uses) once its
    // chunks are done, instead of in an area of their own.  (Also for MQ: 16
    // columns of accumulators per wave.)
    constexpr bool kAccInTile = NWV == 16 || MQ;
    static_assert(!kAccInTile || NCOL * D * 4 <= Lay::VBYTES, "accumulators must fit a wave's V tile");
    __shared__ __align__(16) unsigned char vbuf[kWaves][Lay::VBYTES];
    __shared__ float sh_acc_own[kAccInTile ? 1 : kWaves][kAccInTile ? 1 : G][kAccInTile ? 1 : D];
    __shared__ float sh_ml[kWaves][NCOL][2];
    // MQ: the chunk's K rows (16 rows, row-major) and V rows (32 rows in the
    // V tile layout, rows past the chunk zero)
    __shared__ __align__(16) unsigned char mq_k[MQ ? 16 * D * 2 : 16];
    __shared__ __align__(16) unsigned char mq_v[MQ ? kChunk * Lay::VROW : 16];
    auto acc_at = [&](int wv, int g, int dim) -> float & {
        if constexpr (kAccInTile) return ((float *)vbuf[wv])[g * D + dim];
        else return sh_acc_own[wv][g][dim];
    };

    // Every kernel argument the first cache loads depend on is requested at
    // once; left to itself the compiler fetched them in four rounds, each
    // waiting on the one before (the index arithmetic between them needs the
    // earlier ones).
    asm volatile("" ::"s"(p.Kc), "s"(p.Vc), "s"(p.Q), "s"(p.O), "s"(p.part), "s"(p.sink_logit), "s"(p.B), "s"(p.Hkv),
                 "s"(p.nsplit), "s"(p.rows_per_split), "s"(p.nvalid), "s"(p.pairs_per_wg), "s"(p.w), "s"(p.Hq));
    if constexpr (FU || MQ) asm volatile("" ::"s"(p.Kn), "s"(p.Vn), "s"(p.new_slot));
    if constexpr (MQ) asm volatile("" ::"s"(p.mq_c), "s"(p.s), "s"(p.ring_head), "s"(p.n0));
    if constexpr (ES == 1) asm volatile("" ::"s"(p.kv_scale));
    if constexpr (PG)
        asm volatile("" ::"s"(p.pg.Kp), "s"(p.pg.Vp), "s"(p.pg.block_table), "s"(p.pg.n), "s"(p.pg.num_pages),
                     "s"(p.pg.page), "s"(p.pg.pages_per_seq));
    // Waves per task, a power of two (4-wave workgroups hold 1, 2 or 4 tasks,
    // larger ones one), so the wave-to-task split takes shifts; the task index
    // is divided only when there are splits or the kv-head count is not a
    // power of two (a run-time division is ~25 scalar and vector instructions
    // on the path to the first load).
    const int P = NWV == 4 ? p.pairs_per_wg : 1;
    const int wlog = NWV == 4 ? (P == 4 ? 0 : P == 2 ? 1 : 2) : (NWV == 8 ? 3 : 4), wpt = 1 << wlog;
    // The wave index is uniform across the wave; saying so keeps the buffer
    // descriptors below in scalar registers.
    const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int r16 = lane & 15, g4 = lane >> 4;
    const int ntasks = p.B * p.Hkv * p.nsplit;
    const int task = blockIdx.x * P + (wave >> wlog), sub = wave & (wpt - 1);
    const bool active = task < ntasks;
    int pair = active ? task : 0, sp = 0;
    if (p.nsplit != 1) {
        const int t = pair;
        pair = t / p.nsplit;
        sp = t - pair * p.nsplit;
    }
    int b, hkv;
    if ((p.Hkv & (p.Hkv - 1)) == 0) {
        b = pair >> __builtin_ctz(p.Hkv);
        hkv = pair & (p.Hkv - 1);
    } else {
        b = pair / p.Hkv;
        hkv = pair - b * p.Hkv;
    }
    const int lo = sp * p.rows_per_split;
    int nv = p.nvalid;
    if constexpr (PG) {
        const int64_t n = p.pg.n[b];
        nv = n < 0 ? 0 : (n < p.w ? (int)n : p.w);
    }
    const int hi = active ? max(lo, min(nv, lo + p.rows_per_split)) : lo;
    const int nchunks = (hi - lo + kChunk - 1) / kChunk;
    const int nmine = sub < nchunks ? (nchunks - sub + wpt - 1) >> wlog : 0;

    const size_t block = (size_t)pair * p.w * D;  // elements
    auto rk = make_rsrc((const CT *)p.Kc + block, hi * D * ES);
    auto rv = make_rsrc((const CT *)p.Vc + block, hi * D * ES);

    // Q^T operand: lane (column r16, group g4) holds head r16's dims 8*g4 + 32*kk.
    // Columns r16 >= G repeat the group's first head; their scores, sums and
    // accumulators are computed but never stored.  (Masking them would make
    // the cache loads below wait for Q.)
    // First dim of contraction step kk for this lane.  bf16: 8*g4 + 32*kk.
    // fp8: 16*g4 + 64*(kk/2) + 8*(kk%2), so that steps kk and kk+1 take one
    // 16-byte load of 16 codes (the sum over d does not depend on the order).
    auto kdim0 = [&](int kk) { return ES == 2 ? 8 * g4 + 32 * kk : 16 * g4 + 64 * (kk / 2) + 8 * (kk % 2); };
    // MQ: column r16 < C*G is chunk row r16 / G, head r16 % G (the columns
    // past C*G repeat column 0, like the columns past G otherwise).
    const int ncol = MQ ? p.mq_c * G : G;
    const int qcol = r16 < ncol ? r16 : 0;
    const int crow = MQ ? qcol / G : 0;  // this lane's chunk row
    bf16x8 qf[Lay::KK];
    {
        const int hq = hkv * G + (MQ ? qcol % G : qcol);
        const bf16 *qrow = (const bf16 *)p.Q + ((size_t)(MQ ? b * p.mq_c + crow : b) * p.Hq + hq) * D;
#pragma unroll
        for (int kk = 0; kk < Lay::KK; ++kk) qf[kk] = *(const bf16x8 *)(qrow + kdim0(kk));
    }

    // log2(e)/sqrt(d), times the K dequantisation scale of an fp8 cache
    const float c = 1.4426950408889634f * rsqrtf((float)D) * (ES == 1 ? p.kv_scale[hkv] : 1.f);
    // the same threshold in raw score units, kLazy * sqrt(D) * ln 2 (divided
    // by the K scale of an fp8 cache); it only decides when the max is raised
    static_assert(D == 64 || D == 128, "head dims 64 and 128");
    constexpr float kLazyRaw = kLazy * (D == 64 ? 8.f : 11.313708498984761f) * 0.6931471805599453f;
    const float lazy_raw = ES == 1 ? kLazyRaw * __builtin_amdgcn_rcpf(p.kv_scale[hkv]) : kLazyRaw;
    float m = -INFINITY, l = 0.f;
    floatx4 oacc[Lay::DT];
#pragma unroll
    for (int dt = 0; dt < Lay::DT; ++dt) oacc[dt] = floatx4{0.f, 0.f, 0.f, 0.f};

    unsigned char *vw = vbuf[wave];
    auto row_of = [&](int i) { return lo + kChunk * (sub + wpt * i); };
    auto load = [&](int i, Regs &r) {
        const int row0 = row_of(i);
        int rb = 0;  // row the descriptors start at: the task's block, or this chunk's page row
        if constexpr (PG) {
            // this chunk's page; an entry outside the pool reads as zeros
            const int pi = p.pg.block_table[(size_t)b * p.pg.pages_per_seq + row0 / p.pg.page];
            const bool ok = pi >= 0 && pi < p.pg.num_pages;
            const size_t base = ((size_t)(ok ? pi : 0) * p.Hkv + hkv) * p.pg.page * D + (size_t)(row0 % p.pg.page) * D;
            const int bytes = ok ? min(hi - row0, kChunk) * D * ES : 0;
            rk = make_rsrc((const CT *)p.pg.Kp + base, bytes);
            rv = make_rsrc((const CT *)p.pg.Vp + base, bytes);
            rb = row0;
        }
#pragma unroll
        for (int hf = 0; hf < 2; ++hf)
#pragma unroll
            for (int kk = 0; kk < Lay::KK; ++kk) {
                const int off = ((row0 - rb + 16 * hf + r16) * D + kdim0(kk)) * ES;
                // Cache rows are non-temporal loads (read once per step):
                // bf16 26.1 -> 23.6 us at batch 64, SWA(512,4); fp8 15.2 ->
                // 14.3 us there once its K loads were 16 bytes wide (with
                // 8-byte K loads the hint had cost 16.1 -> 18.7 us).
                if constexpr (ES == 2) {
                    r.k[hf][kk] = __builtin_bit_cast(bf16x8, buffer_load16_nt(rk, off));
                } else if (kk % 2 == 0) {
                    const u32x4 x = buffer_load16_nt(rk, off);
                    r.k[hf][kk] = u32x2{x[0], x[1]};
                    r.k[hf][kk + 1] = u32x2{x[2], x[3]};
                }
            }
#pragma unroll
        for (int j = 0; j < Regs::VL; ++j) {
            const int q = lane + 64 * j, row = q / (D * ES / 16), col = q % (D * ES / 16);
            r.v[j] = buffer_load16_nt(rv, (row0 - rb + row) * D * ES + col * 16);
        }
        if constexpr (FU) {
            const int tr = p.new_slot - row0;  // the new row's place in this chunk
            if (tr >= 0 && tr < kChunk) {       // uniform
                const size_t nrow = (size_t)pair * D;
                const auto rkn = make_rsrc((const bf16 *)p.Kn + nrow, D * 2);
                const auto rvn = make_rsrc((const bf16 *)p.Vn + nrow, D * 2);
                constexpr int RPJ = 64 / (D / 8);  // V rows per load step
                const u32x4 nv = buffer_load16(rvn, (lane % (D / 8)) * 16);
#pragma unroll
                for (int kk = 0; kk < Lay::KK; ++kk) {
                    const bf16x8 nk = __builtin_bit_cast(bf16x8, buffer_load16(rkn, (8 * g4 + 32 * kk) * 2));
#pragma unroll
                    for (int hf = 0; hf < 2; ++hf)
                        if (hf == tr / 16) r.k[hf][kk] = r16 == tr % 16 ? nk : r.k[hf][kk];
                    // the slot takes the new K row: lanes 0, 16, 32, 48 write its four 8-dim groups
                    if (r16 == 0)
                        *(bf16x8 *)((bf16 *)p.Kc + block + (size_t)p.new_slot * D + 8 * g4 + 32 * kk) = nk;
                }
#pragma unroll
                for (int j = 0; j < Regs::VL; ++j)
                    if (j == tr / RPJ) r.v[j] = lane / (D / 8) == tr % RPJ ? nv : r.v[j];
                if (lane < D / 8) *(u32x4 *)((bf16 *)p.Vc + block + (size_t)p.new_slot * D + lane * 8) = nv;
            }
        }
        // Every load of the chunk is issued before any of them is used: left
        // alone, the scheduler starts the QK MFMAs (which need K only) ahead of
        // the V loads, and each chunk then waits for two memory round trips.
        __builtin_amdgcn_sched_barrier(0);
    };
    // MQ: a ring slot holds the position `age` steps before n0; chunk row
    // crow (position n0 + crow + 1) attends it while age <= R - 2 - crow, and
    // every sink slot.  Otherwise every occupied slot.
    const int R = p.w - p.s;
    auto keep_slot = [&](int key) {
        if constexpr (MQ) {
            int age = p.ring_head - (key - p.s);
            age += age < 0 ? R : 0;
            return key < hi && (key < p.s || age <= R - 2 - crow);
        } else {
            return key < hi;
        }
    };
    // One chunk of 32 keys: S^T from the K fragments kget(hf, kk), the keys
    // this lane's column attends (keep(e), e = the key's row in the chunk),
    // the online softmax, then O^T += V^T P^T with V read from the LDS tile
    // vt (vput() stages it there first).
    auto run_chunk = [&](auto &&kget, auto &&keep, auto &&vput, const unsigned char *vt) {
        floatx4 sacc[2];
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
            sacc[hf] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < Lay::KK; ++kk) sacc[hf] = mma16x16x32(kget(hf, kk), qf[kk], sacc[hf]);
        }
        float sc[8];
#pragma unroll
        for (int hf = 0; hf < 2; ++hf)
#pragma unroll
            for (int i4 = 0; i4 < 4; ++i4) sc[4 * hf + i4] = keep(16 * hf + 4 * g4 + i4) ? sacc[hf][i4] : -INFINITY;
        float mx = fmaxf(fmaxf(sc[0], sc[1]), sc[2]);
        mx = fmaxf(fmaxf(mx, sc[3]), sc[4]);
        mx = fmaxf(fmaxf(mx, sc[5]), sc[6]);
        mx = fmaxf(mx, sc[7]);
        mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
        mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
        const bool raise = mx > m + lazy_raw;
        if (__builtin_amdgcn_ballot_w64(raise)) {
            const float mnew = raise ? mx : m;
            const float alpha = raise ? fast_exp2((m - mnew) * c) : 1.f;
            l *= alpha;
#pragma unroll
            for (int dt = 0; dt < Lay::DT; ++dt) oacc[dt] *= alpha;
            m = mnew;
        }
        const float mc = (m == -INFINITY ? 0.f : m) * c;
        float pv[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            pv[e] = fast_exp2(fmaf(sc[e], c, -mc));
            l += pv[e];
        }
        const bf16x8 pf = to_frag<bf16x8>(pv);
        vput();
        // V^T operand for dim tile dt: lane group g4 takes keys 4*g4..+3 and
        // 16+4*g4..+3 (the key order of the S^T accumulators), dim 16*dt + r16.
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        typedef __attribute__((address_space(3))) shortx4 lds_shortx4;
        const unsigned char *va = vt + (4 * g4 + (r16 >> 2)) * Lay::VROW + (4 * (r16 & 3)) * 2;
#pragma unroll
        for (int dt = 0; dt < Lay::DT; ++dt) {
            const unsigned char *a = va + 32 * dt;
            const shortx4 lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_shortx4 *)a);
            const shortx4 hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_shortx4 *)(a + 16 * Lay::VROW));
            typedef short shortx8 __attribute__((ext_vector_type(8)));
            const shortx8 vv = {lo4[0], lo4[1], lo4[2], lo4[3], hi4[0], hi4[1], hi4[2], hi4[3]};
            oacc[dt] = mma16x16x32(__builtin_bit_cast(bf16x8, vv), pf, oacc[dt]);
        }
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
    };
    auto process = [&](int i, const Regs &r) {
        const int row0 = row_of(i);
        run_chunk(
            [&](int hf, int kk) {
                if constexpr (ES == 2) return r.k[hf][kk];
                else return fp8x8_to_bf16(r.k[hf][kk][0], r.k[hf][kk][1]);
            },
            [&](int e) { return keep_slot(row0 + e); },
            [&] {
                // V into the wave's LDS tile only now, so that the scores above need
                // only the K loads (issued first) and run while V is still arriving.
#pragma unroll
                for (int j = 0; j < Regs::VL; ++j) {
                    const int q = lane + 64 * j, row = q / (D * ES / 16), col = q % (D * ES / 16);
                    if constexpr (ES == 2) {
                        *(u32x4 *)(vw + row * Lay::VROW + col * 16) = r.v[j];
                    } else {
                        // 16 codes: dims 16*col .. 16*col+15
                        *(bf16x8 *)(vw + row * Lay::VROW + col * 32) = fp8x8_to_bf16(r.v[j][0], r.v[j][1]);
                        *(bf16x8 *)(vw + row * Lay::VROW + col * 32 + 16) = fp8x8_to_bf16(r.v[j][2], r.v[j][3]);
                    }
                }
            },
            vw);
    };

    // the V dequantisation scale of an fp8 cache, requested before the cache
    // rows so that its latency is hidden
    const float sv = ES == 1 ? p.kv_scale[p.Hkv + hkv] : 1.f;

    // MQ: the chunk's rows go to LDS (mq_k, mq_v) in 16-byte pieces spread
    // over the workgroup's threads, requested before the first cache chunk
    // and stored once they land; rows past the chunk read as zeros.
    constexpr int KPC = D * 2 / 16;                         // pieces per row
    constexpr int NPC = MQ ? (16 + kChunk) * KPC : 0;       // K rows 0..15, V rows 0..31
    constexpr int PPL = (NPC + 64 * NWV - 1) / (64 * NWV);  // pieces per lane
    u32x4 npc[PPL > 0 ? PPL : 1];
    auto piece_at = [&](int k, int &row, int &col, bool &isv) {
        const int q = tid + 64 * NWV * k;
        isv = q >= 16 * KPC;
        row = (isv ? q - 16 * KPC : q) / KPC;
        col = q % KPC;
        return q < NPC;
    };
    if constexpr (MQ) {
        const size_t cbase = ((size_t)b * p.mq_c * p.Hkv + hkv) * D;  // row 0 of this (b, kv-head)'s chunk rows
        const int cbytes = ((p.mq_c - 1) * p.Hkv + 1) * D * 2;
        const auto rkc = make_rsrc((const bf16 *)p.Kn + cbase, cbytes);
        const auto rvc = make_rsrc((const bf16 *)p.Vn + cbase, cbytes);
#pragma unroll
        for (int k = 0; k < PPL; ++k) {
            int row, col;
            bool isv;
            if (piece_at(k, row, col, isv)) npc[k] = buffer_load16(isv ? rvc : rkc, row * p.Hkv * D * 2 + col * 16);
        }
    }
    auto store_pieces = [&] {
        if constexpr (MQ) {
#pragma unroll
            for (int k = 0; k < PPL; ++k) {
                int row, col;
                bool isv;
                if (piece_at(k, row, col, isv))
                    *(u32x4 *)(isv ? mq_v + row * Lay::VROW + col * 16 : mq_k + row * D * 2 + col * 16) = npc[k];
            }
        }
    };

    // MQ: once the chunk's rows are in LDS (a barrier), the task's last wave
    // (the one with the fewest cache chunks) attends them as one more chunk
    // of keys: row e is attended by chunk row crow when e <= crow and it is
    // in crow's window or a sink.  With 4 or 8 waves this runs while the
    // first cache chunk's loads are in flight.
    auto own_keys = [&] {
        if constexpr (MQ) {
            __syncthreads();
            if (active && sub == wpt - 1) {
                const int C = p.mq_c;
                run_chunk(
                    [&](int hf, int kk) {
                        return hf == 0 ? *(const bf16x8 *)(mq_k + (r16 * D + 8 * g4 + 32 * kk) * 2) : bf16x8{};
                    },
                    [&](int e) { return e < C && e <= crow && (crow - e < R || p.n0 + e + 1 <= p.s); }, [] {}, mq_v);
            }
        }
    };

    // One chunk in flight per wave: with every wave of the grid streaming at
    // once, a deeper prefetch only lengthens the memory queues, and the
    // workgroups dispatched last then wait longest for their first data.
    if constexpr (MQ && NWV == 16) {
        // At most one cache chunk per wave; the chunk's own keys come after it
        // (holding the first chunk's loads across them spills at the 128
        // registers of 16 waves; so did running them through the same
        // instructions as the cache chunk, a second pass of one loop).
        if (nmine > 0) {
            Regs A;
            load(0, A);
            store_pieces();
            process(0, A);
        } else {
            store_pieces();
        }
        own_keys();
    } else if constexpr (MQ) {
        Regs A;
        if (nmine > 0) load(0, A);
        store_pieces();
        own_keys();
        if (nmine > 0) process(0, A);
        for (int i = 1; i < nmine; ++i) {
            Regs A2;
            load(i, A2);
            process(i, A2);
        }
    } else if constexpr (NWV == 16) {
        // the plan gives 16-wave workgroups at most one chunk per wave
        if (nmine > 0) {
            Regs A;
            load(0, A);
            process(0, A);
        }
    } else if constexpr (NWV == 8 && ES == 2) {
        // When the chunks do not divide evenly (18 per pair at SWA(576,4)),
        // the waves with one more request that last chunk together with their
        // first, so their extra round trip is not left for the end of the
        // launch (that layer 15.45 -> 15.17 us per fused step; every wave
        // doing so: 15.70; the fp8 cache's kernel, with less register room,
        // lost 1.6 % and keeps the plain loop).
        const bool extra = nmine >= 2 && nmine > (nchunks >> wlog);
        Regs X;
        if (extra) load(nmine - 1, X);
        for (int i = 0; i < (extra ? nmine - 1 : nmine); ++i) {
            Regs A;
            load(i, A);
            process(i, A);
        }
        if (extra) process(nmine - 1, X);
    } else {
        for (int i = 0; i < nmine; ++i) {
            Regs A;
            load(i, A);
            process(i, A);
        }
    }

    // per-column sum over the four lane groups
    l += __shfl_xor(l, 16, 64);
    l += __shfl_xor(l, 32, 64);
    if (active && r16 < ncol) {
#pragma unroll
        for (int dt = 0; dt < Lay::DT; ++dt)
#pragma unroll
            for (int i4 = 0; i4 < 4; ++i4) acc_at(wave, r16, 16 * dt + 4 * g4 + i4) = oacc[dt][i4];
        if (g4 == 0) {
            sh_ml[wave][r16][0] = m == -INFINITY ? -INFINITY : m * c;  // log2 units
            sh_ml[wave][r16][1] = l;
        }
    }
    __syncthreads();

    // combine the waves of each task; the task's threads split (head, dim).
    // The waves per task are a compile-time count here, so each thread's LDS
    // reads (every wave's max, sum and accumulator) are issued together
    // instead of one dependent read per loop turn: this runs after the last
    // cache rows have landed, when nothing else hides its latency.
    if (!active) return;
    const int t0 = wave & ~(wpt - 1);  // first wave of this task
    auto combine = [&](auto wc) {
        constexpr int W = decltype(wc)::value;  // waves per task
        constexpr int NT = 64 * W;              // threads per task
#pragma unroll
        for (int it = 0; it < (NCOL * D + NT - 1) / NT; ++it) {
            const int idx = (wave - t0) * 64 + lane + NT * it;
            if (idx < ncol * D) {
                const int gq = idx / D, dim = idx % D;  // column, dim
                const int hq = hkv * G + (MQ ? gq % G : gq);
                const float sl2 = p.nsplit == 1 ? sink_log2(p, hq) : -INFINITY;  // the sink joins the final sum only
                float mw[W], lw[W], aw[W];
#pragma unroll
                for (int k = 0; k < W; ++k) {
                    mw[k] = sh_ml[t0 + k][gq][0];
                    lw[k] = sh_ml[t0 + k][gq][1];
                    aw[k] = acc_at(t0 + k, gq, dim);
                }
                float M = sl2;
#pragma unroll
                for (int k = 0; k < W; ++k) M = fmaxf(M, mw[k]);
                float Ls = fast_exp2(sl2 - M), A = 0.f;  // exp2(-inf) = 0 without a sink
#pragma unroll
                for (int k = 0; k < W; ++k) {
                    const float f = fast_exp2(mw[k] - M);  // empty wave: exp2(-inf) = 0
                    Ls = fmaf(f, lw[k], Ls);
                    A = fmaf(f, aw[k], A);
                }
                if (M == -INFINITY) A = Ls = 0.f;  // no rows and no sink term (an empty sequence)
                if (p.nsplit == 1) {
                    const size_t orow = MQ ? (size_t)b * p.mq_c + gq / G : (size_t)b;  // MQ: O is [B, C, Hq, d]
                    ((bf16 *)p.O)[(orow * p.Hq + hq) * D + dim] = Ls > 0.f ? (bf16)(A / Ls * sv) : (bf16)0.f;
                } else {
                    float *part = p.part + (((size_t)b * p.Hq + hq) * p.nsplit + sp) * (D + 2);
                    part[dim] = A;
                    if (dim == 0) {
                        part[D] = M;
                        part[D + 1] = Ls;
                    }
                }
            }
        }
    };
    if constexpr (NWV == 4) {
        if (wpt == 4) combine(std::integral_constant<int, 4>{});
        else if (wpt == 2) combine(std::integral_constant<int, 2>{});
        else combine(std::integral_constant<int, 1>{});
    } else {
        combine(std::integral_constant<int, NWV>{});  // one task per workgroup
    }
    if constexpr (MQ) {
        // The chunk's rows into their slots.  Every wave of the workgroup has
        // read this (b, kv-head)'s cache (the barrier above), and no other
        // workgroup reads it.  A row whose position a later chunk row evicts
        // is skipped: of positions p > s only the last R stay.
        constexpr int KPC = D * 2 / 16;
        const int C = p.mq_c;
        for (int q = tid; q < 2 * C * KPC; q += 64 * NWV) {
            const bool isv = q >= C * KPC;
            const int rq = isv ? q - C * KPC : q, row = rq / KPC, col = rq % KPC;
            const int64_t pos = p.n0 + row + 1;
            if (pos > p.s && pos <= p.n0 + C - R) continue;
            const int64_t slot = pos <= p.s ? pos - 1 : p.s + (pos - p.s - 1) % R;
            const bf16 *src = (const bf16 *)(isv ? p.Vn : p.Kn) + (((size_t)b * C + row) * p.Hkv + hkv) * D;
            bf16 *dst = (bf16 *)(isv ? p.Vc : p.Kc) + block + (size_t)slot * D;
            *(u32x4 *)((unsigned char *)dst + col * 16) = *(const u32x4 *)((const unsigned char *)src + col * 16);
        }
    }
}

// Merge of split partials: one workgroup per (b, query head), one thread per dim.
template <typename T, int D>
__global__ __launch_bounds__(D) void swa_decode_merge_kernel(DecodeParams p)
{
    const int bq = blockIdx.x, dim = threadIdx.x;
    const float *part = p.part + (size_t)bq * p.nsplit * (D + 2);
    const float sl2 = sink_log2(p, bq % p.Hq);
    float M = sl2;
    for (int j = 0; j < p.nsplit; ++j) M = fmaxf(M, part[j * (D + 2) + D]);
    float Ls = fast_exp2(sl2 - M), A = 0.f;  // exp2(-inf) = 0 without a sink
    for (int j = 0; j < p.nsplit; ++j) {
        const float *pj = part + j * (D + 2);
        const float f = fast_exp2(pj[D] - M);
        Ls = fmaf(f, pj[D + 1], Ls);
        A = fmaf(f, pj[dim], A);
    }
    // an fp8 cache's V dequantisation scale, for the kv-head query head bq % Hq reads
    const float sv = p.kv_scale ? p.kv_scale[p.Hkv + (bq % p.Hq) / (p.Hq / p.Hkv)] : 1.f;
    // an empty sequence (no rows, no sink term) gives 0
    ((T *)p.O)[(size_t)bq * D + dim] = from_f32<T>(M == -INFINITY || !(Ls > 0.f) ? 0.f : A / Ls * sv);
}

// Append: copy the surviving new rows into their slots.  One thread per
// 16-byte chunk of a (survivor, b, kv-head) row, K and V together.
// Quantise eight bf16 values to the E4M3 codes of clamp(x / scale, +-448):
// a correctly rounded fp32 division, then the hardware's nearest-even
// conversion (the OCP E4M3 encoding).
__device__ __forceinline__ uint2 bf16x8_to_fp8(const u32x4 &raw, float scale)
{
    float x[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        x[2 * i] = __uint_as_float(raw[i] << 16);
        x[2 * i + 1] = __uint_as_float(raw[i] & 0xffff0000u);
    }
    uint32_t w[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        float q[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) q[i] = fminf(fmaxf(__fdiv_rn(x[4 * h + i], scale), -448.f), 448.f);
        int v = __builtin_amdgcn_cvt_pk_fp8_f32(q[0], q[1], 0, false);
        v = __builtin_amdgcn_cvt_pk_fp8_f32(q[2], q[3], v, true);
        w[h] = (uint32_t)v;
    }
    return uint2{w[0], w[1]};
}

// T: element type of the new rows; CT: of the cache (T, or fp8 from bf16).
template <typename T, int D, typename CT>
__global__ __launch_bounds__(kThreads) void swa_append_kernel(AppendParams p)
{
    // One workgroup column per (b, kv-head) (blockIdx.x), the threads of the
    // columns taking the survivors' 16-byte chunks.  Survivor j is the j-th
    // new sink position (its slot is the position - 1) or, past the sinks,
    // one of the last w - s positions, whose ring slots follow each other
    // from slot2 and wrap once.
    constexpr int CPR = D * (int)sizeof(T) / 16;  // 16-byte chunks of a new row
    const int bh = blockIdx.x;
    const int b = bh / p.Hkv, hkv = bh - b * p.Hkv;
    const int total = (p.n1 + p.n2) * CPR;
    for (int u = blockIdx.y * kThreads + threadIdx.x; u < total; u += gridDim.y * kThreads) {
        const int chunk = u % CPR, j = u / CPR;
        int src_row, slot;
        if (j < p.n1) {
            src_row = p.src1 + j;
            slot = p.slot1 + j;
        } else {
            src_row = p.src2 + (j - p.n1);
            slot = p.slot2 + (j - p.n1);
            if (slot >= p.w) slot -= p.w - p.s;
        }
        const size_t src = (((size_t)b * p.n_new + src_row) * p.Hkv + hkv) * D;
        const size_t dst = ((size_t)bh * p.w + slot) * D;
        const u32x4 *ks = (const u32x4 *)((const T *)p.Kn + src) + chunk;
        const u32x4 *vs = (const u32x4 *)((const T *)p.Vn + src) + chunk;
        if constexpr (sizeof(CT) == sizeof(T)) {
            *((u32x4 *)((T *)p.Kc + dst) + chunk) = *ks;
            *((u32x4 *)((T *)p.Vc + dst) + chunk) = *vs;
        } else {
            // 8 new elements -> 8 codes
            *((uint2 *)((CT *)p.Kc + dst) + chunk) = bf16x8_to_fp8(*ks, p.kv_scale[hkv]);
            *((uint2 *)((CT *)p.Vc + dst) + chunk) = bf16x8_to_fp8(*vs, p.kv_scale[p.Hkv + hkv]);
        }
    }
}

// Paged append: token u of the packed new rows belongs to the sequence b
// with cu[b] <= u < cu[b+1] and is position n[b] + 1 + (u - cu[b]); it is
// written only if it is still attended after the whole append (a member of
// S_N, N = n[b] + its count), to slot(position) in that slot's page.  One
// thread per 16-byte chunk of a (token, kv-head) row, K and V together.
// Entries of the block table outside the pool are skipped (never written).
template <typename T, int D>
__global__ __launch_bounds__(kThreads) void swa_paged_append_kernel(PagedAppendParams p)
{
    constexpr int CPR = D * (int)sizeof(T) / 16;
    const int64_t total = (int64_t)p.total * p.Hkv * CPR;
    for (int64_t u = (int64_t)blockIdx.x * kThreads + threadIdx.x; u < total;
         u += (int64_t)gridDim.x * kThreads) {
        const int chunk = (int)(u % CPR);
        const int64_t rest = u / CPR;
        const int hkv = (int)(rest % p.Hkv);
        const int tok = (int)(rest / p.Hkv);
        // Rows outside [cu[0], cu[B]) belong to no sequence: never written
        // (cu[0] = 0 and cu[B] = total when the table is well formed).
        if (tok < p.cu_seqlens[0] || tok >= p.cu_seqlens[p.B]) continue;
        // sequence of this token: the last b with cu[b] <= tok
        int lo = 0, hi = p.B;  // invariant: cu[lo] <= tok < cu[hi]
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (p.cu_seqlens[mid] <= tok) lo = mid;
            else hi = mid;
        }
        const int b = lo;
        const int64_t n0 = p.c.n[b];
        const int64_t cnt = p.cu_seqlens[b + 1] - p.cu_seqlens[b];
        const int64_t pos = n0 + 1 + (tok - p.cu_seqlens[b]);
        const int64_t N = n0 + cnt;
        // a row past its sequence's end (cu not non-decreasing) or a negative
        // count n0: no slot to write
        if (tok >= p.cu_seqlens[b + 1] || pos < 1) continue;
        if (!(pos <= p.s || pos > N - (p.w - p.s))) continue;  // evicted within this append
        const int64_t slot = pos <= p.s ? pos - 1 : p.s + (pos - p.s - 1) % (p.w - p.s);
        const int pi = p.c.block_table[(size_t)b * p.c.pages_per_seq + slot / p.c.page];
        if (pi < 0 || pi >= p.c.num_pages) continue;
        const size_t dst = (((size_t)pi * p.Hkv + hkv) * p.c.page + slot % p.c.page) * D;
        const size_t src = ((size_t)tok * p.Hkv + hkv) * D;
        *((u32x4 *)((T *)p.c.Kp + dst) + chunk) = *((const u32x4 *)((const T *)p.Kn + src) + chunk);
        *((u32x4 *)((T *)p.c.Vp + dst) + chunk) = *((const u32x4 *)((const T *)p.Vn + src) + chunk);
    }
}

// n[b] += number of new rows of sequence b (after the append has read n).
__global__ __launch_bounds__(kThreads) void swa_paged_advance_kernel(int64_t *n, const int32_t *cu, int B)
{
    const int b = blockIdx.x * kThreads + threadIdx.x;
    if (b < B) n[b] += cu[b + 1] - cu[b];
}

// T: element type of Q and O; CT: of the cache (T, or fp8 with bf16 Q and O);
// PG: paged bf16 cache.
template <typename T, int D, int G, typename CT = T, bool PG = false, bool FU = false, bool MQ = false>
hipError_t launch_decode_t(const DecodeParams &p, hipStream_t st)
{
    if constexpr (MQ) {
        // one task per workgroup, no splits, 4, 8 or 16 waves; C * G <= 16
        if (p.nsplit != 1 || p.pairs_per_wg != 1 || p.mq_c < 1 || p.mq_c * G > 16) return hipErrorInvalidValue;
        const unsigned wgs = (unsigned)((long long)p.B * p.Hkv);
        if (p.waves_per_wg == 16)
            hipLaunchKernelGGL((swa_decode_mfma_kernel<D, G, bf16, false, false, 16, true>), dim3(wgs), dim3(1024), 0, st,
                               p);
        else if (p.waves_per_wg == 8)
            hipLaunchKernelGGL((swa_decode_mfma_kernel<D, G, bf16, false, false, 8, true>), dim3(wgs), dim3(512), 0, st, p);
        else if (p.waves_per_wg == 4)
            hipLaunchKernelGGL((swa_decode_mfma_kernel<D, G, bf16, false, false, 4, true>), dim3(wgs), dim3(kThreads), 0,
                               st, p);
        else
            return hipErrorInvalidValue;
        return hipGetLastError();
    } else if constexpr (std::is_same_v<T, bf16>) {
        // the kernel splits a workgroup's waves into tasks with shifts
        const int P = p.pairs_per_wg;
        if (p.waves_per_wg == 4 ? (P != 1 && P != 2 && P != 4) : P != 1) return hipErrorInvalidValue;
        const long long tasks = (long long)p.B * p.Hkv * p.nsplit;
        const unsigned wgs = (unsigned)((tasks + p.pairs_per_wg - 1) / p.pairs_per_wg);
        if (p.waves_per_wg == 16) {
            if constexpr (sizeof(CT) == 2)
                hipLaunchKernelGGL((swa_decode_mfma_kernel<D, G, CT, PG, FU, 16>), dim3(wgs), dim3(1024), 0, st, p);
            else
                return hipErrorInvalidValue;  // the plan gives fp8 caches no 16-wave workgroups
        } else if (p.waves_per_wg == 8)
            hipLaunchKernelGGL((swa_decode_mfma_kernel<D, G, CT, PG, FU, 8>), dim3(wgs), dim3(512), 0, st, p);
        else
            hipLaunchKernelGGL((swa_decode_mfma_kernel<D, G, CT, PG, FU, 4>), dim3(wgs), dim3(kThreads), 0, st, p);
    } else {
        dim3 grid((unsigned)p.nsplit, (unsigned)(p.B * p.Hkv));
        hipLaunchKernelGGL((swa_decode_valu_kernel<T, D, G>), grid, dim3(kThreads), 0, st, p);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || p.nsplit == 1) return e;
    hipLaunchKernelGGL((swa_decode_merge_kernel<T, D>), dim3((unsigned)(p.B * p.Hq)), dim3(D), 0, st, p);
    return hipGetLastError();
}

template <typename T, int D, typename CT = T, bool PG = false, bool FU = false, bool MQ = false>
hipError_t launch_decode_g(int G, const DecodeParams &p, hipStream_t st)
{
    switch (G) {
    case 1: return launch_decode_t<T, D, 1, CT, PG, FU, MQ>(p, st);
    case 2: return launch_decode_t<T, D, 2, CT, PG, FU, MQ>(p, st);
    case 4: return launch_decode_t<T, D, 4, CT, PG, FU, MQ>(p, st);
    case 8: return launch_decode_t<T, D, 8, CT, PG, FU, MQ>(p, st);
    default: return hipErrorInvalidValue;
    }
}

template <typename T, int D, typename CT = T> hipError_t launch_append_t(const AppendParams &p, hipStream_t st)
{
    constexpr int CPR = D * (int)sizeof(T) / 16;
    AppendParams q = p;
    const int64_t n1 = p.b1 >= p.a1 ? p.b1 - p.a1 + 1 : 0;
    const int64_t n2 = p.b2 >= p.a2 ? p.b2 - p.a2 + 1 : 0;
    // survivors are new rows: sinks in slots below s, and at most w - s ring
    // positions past the sinks
    if (n1 && (p.a1 - p.n_before - 1 < 0 || p.b1 - p.n_before > p.n_new || p.a1 < 1 || p.b1 > p.s))
        return hipErrorInvalidValue;
    if (n2 && (p.a2 - p.n_before - 1 < 0 || p.b2 - p.n_before > p.n_new || p.a2 <= p.s || n2 > p.w - p.s))
        return hipErrorInvalidValue;
    const long long bh = (long long)p.B * p.Hkv;
    if (n1 + n2 == 0 || bh == 0) return hipSuccess;
    if (bh > 0x7fffffffLL || (n1 + n2) * CPR > 0x7fffffffLL) return hipErrorInvalidValue;
    q.n1 = (int)n1;
    q.n2 = (int)n2;
    q.src1 = (int)(p.a1 - p.n_before - 1);
    q.src2 = (int)(p.a2 - p.n_before - 1);
    q.slot1 = (int)(p.a1 - 1);
    q.slot2 = n2 ? (int)(p.s + (p.a2 - p.s - 1) % (p.w - p.s)) : 0;
    const long long cols = ((n1 + n2) * CPR + kThreads - 1) / kThreads;
    const unsigned gy = (unsigned)(cols < 65535 ? cols : 65535);
    hipLaunchKernelGGL((swa_append_kernel<T, D, CT>), dim3((unsigned)bh, gy), dim3(kThreads), 0, st, q);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(Dt dt, int d, int G, const DecodeParams &p, hipStream_t st)
{
    if (dt == Dt::FP8)
        return d == 128 ? launch_decode_g<bf16, 128, fp8>(G, p, st) : launch_decode_g<bf16, 64, fp8>(G, p, st);
    if (dt == Dt::BF16) return d == 128 ? launch_decode_g<bf16, 128>(G, p, st) : launch_decode_g<bf16, 64>(G, p, st);
    return d == 128 ? launch_decode_g<float, 128>(G, p, st) : launch_decode_g<float, 64>(G, p, st);
}

template <typename T, int D> hipError_t launch_paged_append_t(const PagedAppendParams &p, hipStream_t st)
{
    constexpr int CPR = D * (int)sizeof(T) / 16;
    const int64_t total = (int64_t)p.total * p.Hkv * CPR;
    if (total > 0) {
        int64_t blocks = (total + kThreads - 1) / kThreads;
        if (blocks > 65536) blocks = 65536;
        hipLaunchKernelGGL((swa_paged_append_kernel<T, D>), dim3((unsigned)blocks), dim3(kThreads), 0, st, p);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(swa_paged_advance_kernel, dim3((unsigned)((p.B + kThreads - 1) / kThreads)), dim3(kThreads),
                       0, st, p.c.n, p.cu_seqlens, p.B);
    return hipGetLastError();
}

hipError_t launch_paged_append(Dt dt, int d, const PagedAppendParams &p, hipStream_t st)
{
    if (dt == Dt::BF16) return d == 128 ? launch_paged_append_t<bf16, 128>(p, st) : launch_paged_append_t<bf16, 64>(p, st);
    return d == 128 ? launch_paged_append_t<float, 128>(p, st) : launch_paged_append_t<float, 64>(p, st);
}

// Fixed scratch for callers that cannot allocate (swa_decode_noalloc): the
// split partials of one decode call live here instead of in a caller
// workspace.  Each GPU holds its own copy of the array for the life of the
// process.  In host code `scratch` names a host-side stand-in, never a device
// address: the address a kernel gets is the one hipGetSymbolAddress returns
// with that device current, looked up once per device and kept.
static __device__ __align__(256) unsigned char scratch[kDecodeScratchBytes];

hipError_t decode_scratch(int device, void **ptr)
{
    static std::mutex mu;
    static void *addr[kMaxDevices] = {};
    if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[device]) {
        void *a = nullptr;
        const hipError_t e = hipGetSymbolAddress(&a, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        addr[device] = a;
    }
    *ptr = addr[device];
    return hipSuccess;
}

hipError_t launch_decode_step(int d, int G, const DecodeParams &p, hipStream_t st)
{
    return d == 128 ? launch_decode_g<bf16, 128, bf16, false, true>(G, p, st)
                    : launch_decode_g<bf16, 64, bf16, false, true>(G, p, st);
}

hipError_t launch_decode_mq(int d, int G, const DecodeParams &p, hipStream_t st)
{
    return d == 128 ? launch_decode_g<bf16, 128, bf16, false, false, true>(G, p, st)
                    : launch_decode_g<bf16, 64, bf16, false, false, true>(G, p, st);
}

hipError_t launch_decode_paged(int d, int G, const DecodeParams &p, hipStream_t st)
{
    return d == 128 ? launch_decode_g<bf16, 128, bf16, true>(G, p, st) : launch_decode_g<bf16, 64, bf16, true>(G, p, st);
}

hipError_t launch_append(Dt dt, int d, const AppendParams &p, hipStream_t st)
{
    // Dt::FP8: bf16 new rows quantised into an E4M3 cache
    if (dt == Dt::FP8)
        return d == 128 ? launch_append_t<bf16, 128, fp8>(p, st) : launch_append_t<bf16, 64, fp8>(p, st);
    if (dt == Dt::BF16) return d == 128 ? launch_append_t<bf16, 128>(p, st) : launch_append_t<bf16, 64>(p, st);
    return d == 128 ? launch_append_t<float, 128>(p, st) : launch_append_t<float, 64>(p, st);
}

}  // namespace swa
