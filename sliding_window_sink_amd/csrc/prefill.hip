// SWA(w,s) prefill on gfx950.
//
// Every query row t (0-based here) attends the keys
//     j <= t  and  (j < s  or  j > t - (w - s))
// i.e. the first s tokens plus the most recent w - s (paper.rainbus.top summary
// of arXiv 2608.28444, "滑窗注意力 SWA(w, s)" and method steps, step 2), with the
// softmax normalised over exactly that set (the windowed-softmax equation of
// the same section).  Keys outside the set contribute exactly zero: they are
// either in tiles this kernel never visits or masked to -inf before exp.
//
// Work decomposition
//   One workgroup = 4 waves = one (batch, kv-head) and a block of BQ = 128/G
//   query positions for all G query heads sharing that kv-head: 128 packed
//   (head, position) rows, 32 per wave (one 32-row MFMA tile).  K/V tiles of
//   32 keys are staged through LDS once and read by all G heads.  The tiles
//   visited are the sink tiles covering [0, s) and the window band of the
//   block (once the band starts past the first tile, one tile holds the s sink
//   rows and the first 32 - s band rows); everything else is skipped, so the
//   work per row is O(w), not O(t).
//
// Trips: bf16 tiles are taken two at a time (64 keys per trip, fp32 one at a
// time); the tiles of a trip share one softmax step and one barrier.
// Per 32-key tile, per wave (v_mfma_f32_32x32x16_bf16):
//   S^T (32 keys x 32 rows) = K Q^T   : d/16 MFMAs, K from LDS, Q in VGPRs.
//       Lane l holds column l%32 (its query row): keys 8j + 4*(l/32) + i.
//   online softmax in fp32            : row max over the lane's 16 scores per
//       tile of the trip and the partner lane l^32 (one shuffle per trip);
//       exp2 with 1/sqrt(d)*log2(e)
//       folded into one FMA.  The running max is raised only when a row's
//       tile max exceeds it by more than 2^8 in exp2 units (then the
//       accumulators are rescaled); otherwise p <= 256 and nothing is rescaled.
//       Numerator and denominator use the same shift, so this is exact.
//       Row sums: each lane adds the p values it feeds the PV MFMA (bf16:
//       the rounded ones, with dot-product instructions); the two lanes of a
//       row are added at the end.
//   O^T (d x 32 rows) += V^T P^T      : 2 * d/32 MFMAs, V^T from LDS, P^T
//       straight from the S^T accumulators: k-step ks takes elements
//       8ks..8ks+7, i.e. keys 16ks + 8*(e/4) + 4*(l/32) + e%4.  bf16: V is
//       stored row-major and read with transposing loads in that key order;
//       fp32: V^T is written to LDS with its keys in that order.
#include "device_common.h"
#include "swa_internal.h"

#include <type_traits>

namespace swa {
namespace {

constexpr int kThreads = 256;
constexpr int kKB = 32;       // keys per LDS tile
constexpr int kRowsWG = 128;  // packed (head, position) rows per workgroup

// LDS layout of one tile.  K: 32 rows of d elements, row-major, 16 B of
// padding per row.  V: for bf16, 32 rows of d elements row-major with 64 B of
// padding, read with transposing loads; for fp32, transposed on the way in
// (d rows of 32 keys, 16-B chunks XOR-swizzled).  A stage holds the tiles of
// one trip (two for bf16, one for fp32, whose tiles are twice the size), and
// there are two stages.
// The V padding: a transposing read of half a wave touches 4 rows, 2 column
// halves and 4 8-byte columns; with rows d*2 + 64 bytes apart (16 or 48
// banks mod 64) those land on 64 distinct banks.  With 32 B of padding the
// rows were 8 banks apart and the reads two-way conflicted: 89 % of the
// kernel's LDS bank conflicts, which the padding removes (the kernel's time
// stays within 1 %).
template <typename T, int D> struct PrefillLds {
    static constexpr int ES = sizeof(T);
    static constexpr int KROW = D * ES + 16;  // bytes per K row
    static constexpr int VROW = sizeof(T) == 2 ? D * ES + 64 : kKB * ES;
    static constexpr int KTILE = kKB * KROW;
    static constexpr int VTILE = sizeof(T) == 2 ? kKB * VROW : D * VROW;
    static constexpr int STAGE = KTILE + VTILE;      // one tile's K and V
    static constexpr int TPT = sizeof(T) == 2 ? 2 : 1;  // tiles per trip (one softmax step)
    static constexpr int PSTAGE = TPT * STAGE;       // one trip's tiles
    static constexpr int BYTES = 2 * PSTAGE;
    static constexpr int CPR = D * ES / 16;  // 16-byte chunks per global row
};

// fp32 path: position of key k (0..31 of the tile) in the PV contraction
// order; within each half of 16 keys, bits 2 and 3 of the key index swap.
__device__ __forceinline__ int pv_index(int k)
{
    return (k & ~12) | ((k & 4) << 1) | ((k & 8) >> 1);
}

// fp32 V^T rows are 128 B (8 chunks of 16 B); the chunk index is XORed with
// the row's low bits so that consecutive rows spread over the banks.
template <typename T> __device__ __forceinline__ int vt_swizzle(int dim);
template <> __device__ __forceinline__ int vt_swizzle<float>(int dim) { return dim & 7; }

template <typename T, int D> __device__ __forceinline__ int vt_offset(int dim, int kp)
{
    using Lds = PrefillLds<T, D>;
    const int byte = kp * (int)sizeof(T);
    const int chunk = (byte >> 4) ^ vt_swizzle<T>(dim);
    return dim * Lds::VROW + (chunk << 4) + (byte & 15);
}

// Global -> register staging of one K/V tile, and register -> LDS stores.
template <typename T, int D> struct TileStager;

// Tile loads go through buffer descriptors that end at the last row of the
// sequence, so rows past it read as zero without a test; the descriptor base
// moves per tile in scalar registers and each thread's byte offset inside a
// tile never changes.
template <int D> struct TileStager<bf16, D> {
    using Lds = PrefillLds<bf16, D>;
    static constexpr int NC = kKB * Lds::CPR / kThreads;  // 16-B chunks per thread, K and V each
    static_assert(NC >= 1, "tile too small for the workgroup");
    u32x4 k[NC], v[NC];

    __device__ __forceinline__ void load(const bf16 *Kg, const bf16 *Vg, int row_bytes, int key0, int L,
                                         int tid)
    {
        const size_t base = (size_t)key0 * row_bytes;
        const int nbytes = (L - 1 - key0) * row_bytes + D * 2;
        const auto rk = make_rsrc((const char *)Kg + base, nbytes);
        const auto rv = make_rsrc((const char *)Vg + base, nbytes);
#pragma unroll
        for (int u = 0; u < NC; ++u) {
            const int ci = tid + kThreads * u, row = ci / Lds::CPR, col = ci % Lds::CPR;
            const int off = row * row_bytes + col * 16;
            k[u] = buffer_load16(rk, off);
            v[u] = buffer_load16(rv, off);
        }
    }

    // The packed first tile: rows 0..s-1 are keys 0..s-1 (the sinks), rows
    // s..31 are keys band_lo .. band_lo + 31 - s.
    __device__ __forceinline__ void load_packed(const bf16 *Kg, const bf16 *Vg, int row_bytes, int L, int tid,
                                                int s, int band_lo)
    {
        const int nbytes = (L - 1) * row_bytes + D * 2;
        const auto rk = make_rsrc(Kg, nbytes);
        const auto rv = make_rsrc(Vg, nbytes);
#pragma unroll
        for (int u = 0; u < NC; ++u) {
            const int ci = tid + kThreads * u, row = ci / Lds::CPR, col = ci % Lds::CPR;
            const int key = row < s ? row : band_lo + row - s;
            const int off = key * row_bytes + col * 16;
            k[u] = buffer_load16(rk, off);
            v[u] = buffer_load16(rv, off);
        }
    }

    __device__ __forceinline__ void store(unsigned char *stage, int tid) const
    {
#pragma unroll
        for (int u = 0; u < NC; ++u) {
            const int ci = tid + kThreads * u, row = ci / Lds::CPR, col = ci % Lds::CPR;
            *(u32x4 *)(stage + row * Lds::KROW + col * 16) = k[u];
            *(u32x4 *)(stage + Lds::KTILE + row * Lds::VROW + col * 16) = v[u];
        }
    }
};

template <int D> struct TileStager<float, D> {
    using Lds = PrefillLds<float, D>;
    static constexpr int NK = kKB * Lds::CPR / kThreads;
    static constexpr int NV = kKB * (D / 4) / kThreads;
    u32x4 k[NK];
    u32x4 v[NV];

    __device__ __forceinline__ void load(const float *Kg, const float *Vg, int row_bytes, int key0, int L,
                                         int tid)
    {
        const size_t base = (size_t)key0 * row_bytes;
        const int nbytes = (L - 1 - key0) * row_bytes + D * 4;
        const auto rk = make_rsrc((const char *)Kg + base, nbytes);
        const auto rv = make_rsrc((const char *)Vg + base, nbytes);
#pragma unroll
        for (int u = 0; u < NK; ++u) {
            const int ci = tid + kThreads * u, row = ci / Lds::CPR, col = ci % Lds::CPR;
            k[u] = buffer_load16(rk, row * row_bytes + col * 16);
        }
#pragma unroll
        for (int u = 0; u < NV; ++u) {
            const int ci = tid + kThreads * u, key = ci / (D / 4), c4 = ci % (D / 4);
            v[u] = buffer_load16(rv, key * row_bytes + c4 * 16);
        }
    }

    // The packed first tile (rows 0..s-1: the sinks; rows s..31: keys band_lo..).
    __device__ __forceinline__ void load_packed(const float *Kg, const float *Vg, int row_bytes, int L, int tid,
                                                int s, int band_lo)
    {
        const int nbytes = (L - 1) * row_bytes + D * 4;
        const auto rk = make_rsrc(Kg, nbytes);
        const auto rv = make_rsrc(Vg, nbytes);
#pragma unroll
        for (int u = 0; u < NK; ++u) {
            const int ci = tid + kThreads * u, row = ci / Lds::CPR, col = ci % Lds::CPR;
            const int key = row < s ? row : band_lo + row - s;
            k[u] = buffer_load16(rk, key * row_bytes + col * 16);
        }
#pragma unroll
        for (int u = 0; u < NV; ++u) {
            const int ci = tid + kThreads * u, row = ci / (D / 4), c4 = ci % (D / 4);
            const int key = row < s ? row : band_lo + row - s;
            v[u] = buffer_load16(rv, key * row_bytes + c4 * 16);
        }
    }

    __device__ __forceinline__ void store(unsigned char *stage, int tid) const
    {
#pragma unroll
        for (int u = 0; u < NK; ++u) {
            const int ci = tid + kThreads * u, row = ci / Lds::CPR, col = ci % Lds::CPR;
            *(u32x4 *)(stage + row * Lds::KROW + col * 16) = k[u];
        }
        unsigned char *vt = stage + Lds::KTILE;
#pragma unroll
        for (int u = 0; u < NV; ++u) {
            const int ci = tid + kThreads * u, key = ci / (D / 4), c4 = ci % (D / 4);
            const int kp = pv_index(key);
#pragma unroll
            for (int e = 0; e < 4; ++e) *(uint32_t *)(vt + vt_offset<float, D>(4 * c4 + e, kp)) = v[u][e];
        }
    }
};

// Bits a..b-1 of a 32-bit word (a, b in [0, 32]).
__device__ __forceinline__ uint32_t bit_range(int a, int b)
{
    const uint32_t hi = b >= 32 ? 0xffffffffu : ((1u << max(b, 0)) - 1u);
    const uint32_t lo = a >= 32 ? 0xffffffffu : ((1u << max(a, 0)) - 1u);
    return b > a ? (hi & ~lo) : 0u;
}

// A operand of O^T += V^T P^T for one 32-dim tile and 16-key contraction step.
// bf16: two transposing LDS reads.  Within each group of 16 lanes,
// ds_read_b64_tr_b16 hands lane 4a+b element b of the 4 values addressed by
// lane 4j+a, as its element j.  Lane l addresses V row kb + (l%16)/4, dims
// d0 + 4*(l%4), so it receives keys kb..kb+3 of dim d0 + l%16; with
// kb = 16ks + 8q + 4*(l/32) for read q this is element 4q+j <-> key
// 16ks + 8q + 4*(l/32) + j, the key order of the S^T accumulators.
typedef short shortx4 __attribute__((ext_vector_type(4)));
template <typename T, int D> struct VFrag;
template <int D> struct VFrag<bf16, D> {
    static __device__ __forceinline__ bf16x8 load(const unsigned char *vt, int dt, int ks, int lane)
    {
        using Lds = PrefillLds<bf16, D>;
        const int d0 = 32 * dt + 16 * ((lane >> 4) & 1);
        const int row = 16 * ks + 4 * (lane >> 5) + ((lane & 15) >> 2);
        const unsigned char *a = vt + row * Lds::VROW + (d0 + 4 * (lane & 3)) * 2;
        typedef __attribute__((address_space(3))) shortx4 lds_shortx4;
        const shortx4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_shortx4 *)(a));
        const shortx4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_shortx4 *)(a + 8 * Lds::VROW));
        typedef short shortx8 __attribute__((ext_vector_type(8)));
        const shortx8 r = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        return __builtin_bit_cast(bf16x8, r);
    }
};
// fp32: V^T rows in LDS, PV positions 16ks + 8*(l/32) .. +7.
template <int D> struct VFrag<float, D> {
    static __device__ __forceinline__ floatx8 load(const unsigned char *vt, int dt, int ks, int lane)
    {
        const int dim = 32 * dt + (lane & 31), kp0 = 16 * ks + 8 * (lane >> 5);
        const floatx4 a = *(const floatx4 *)(vt + vt_offset<float, D>(dim, kp0));
        const floatx4 b = *(const floatx4 *)(vt + vt_offset<float, D>(dim, kp0 + 4));
        return floatx8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
    }
};

// Row sums: the lane's share of a row's p, summed as the PV MFMA takes them
// (bf16: the rounded values, two per dot-product instruction with a vector
// of ones; both products are exact and the sum is in fp32).
__device__ __forceinline__ float add_row_part(const bf16x8 &pf, float acc)
{
    const bf16x2 one = {(bf16)1.f, (bf16)1.f};
#pragma unroll
    for (int i = 0; i < 4; ++i) acc = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{pf[2 * i], pf[2 * i + 1]}, one, acc, false);
    return acc;
}
__device__ __forceinline__ float add_row_part(const floatx8 &pf, float acc)
{
#pragma unroll
    for (int e = 0; e < 8; ++e) acc += pf[e];
    return acc;
}

template <typename T> __device__ __forceinline__ void store4(T *dst, float a, float b, float c, float d);
template <> __device__ __forceinline__ void store4<bf16>(bf16 *dst, float a, float b, float c, float d)
{
    *(bf16x4 *)dst = bf16x4{(bf16)a, (bf16)b, (bf16)c, (bf16)d};
}
template <> __device__ __forceinline__ void store4<float>(float *dst, float a, float b, float c, float d)
{
    *(floatx4 *)dst = floatx4{a, b, c, d};
}

// T: input (and MFMA operand) type; TO: output type.
// VL (varlen mode): B sequences of different lengths packed along the row
// axis; the grid covers the longest (p.L) and blocks past a sequence's end
// exit at once.
// CK (chunk mode): the rows are the positions n+1..n+L that follow a cache of
// n positions; the key tiles are first the cache tiles holding slots the
// block attends (in slot order, 32 per tile), then the chunk's own sink and
// band tiles.
// PG (with CK and VL): the cache is paged (p.pg) and each sequence follows
// its own n[b]; its chunk rows are its varlen rows.
template <typename T, typename TO, int D, int G, bool CK, bool VL = false, bool PG = false>
__global__ __launch_bounds__(kThreads, (std::is_same_v<T, float> && D == 128 ? 1 : 2)) void swa_prefill_kernel(PrefillParams p)
{
    using F = typename Frag<T>::type;
    using Lds = PrefillLds<T, D>;
    constexpr int BQ = kRowsWG / G;  // query positions per workgroup
    constexpr int KS = D / 16;       // 16-deep contraction steps of Q.K
    constexpr int DT = D / 32;       // 32-dim output tiles
    constexpr float kLazy = 8.f;     // rescale only when the max grows by > 2^8
    __shared__ __align__(16) unsigned char smem[Lds::BYTES];

    const int Hq = p.Hq, Hkv = p.Hkv, w = p.w, s = p.s;
    const int nqb = (p.L + BQ - 1) / BQ;
    const int total = nqb * p.B * Hkv;
    const int lid = xcd_remap((int)blockIdx.x, total);
    const int qb = lid % nqb, bh = lid / nqb;
    const int b = bh / Hkv, hkv = bh % Hkv;
    const int q0 = qb * BQ;
    // this sequence's rows: L of them from packed row rbase
    int L = p.L;
    size_t rbase = (size_t)b * p.L;
    if constexpr (VL) {
        const int c0 = p.cu_seqlens[b], c1 = min(p.cu_seqlens[b + 1], p.total);
        L = c1 > c0 && c0 >= 0 ? c1 - c0 : 0;
        rbase = (size_t)max(c0, 0);
        if (q0 >= L) return;  // uniform: the whole workgroup leaves before any barrier
    }
    const int qlast = min(q0 + BQ, L) - 1;
    // The cache a chunk follows: one position count n for the batch, set by
    // the host; or, for a paged cache, sequence b's own n[b].
    int c_nvalid = p.nvalid, c_sinks = p.sinks_in, c_head = p.ring_head, c_full = p.ring_full, c_any = p.ring_any;
    int c_sk = p.sk;
    if constexpr (PG) {
        const int64_t n = max((int64_t)0, p.pg.n[b]);
        c_nvalid = (int)min(n, (int64_t)w);
        c_sinks = (int)min(n, (int64_t)s);
        c_any = n > s;
        c_head = n > s ? (int)((n - s - 1) % (w - s)) : 0;
        c_full = n - s >= w - s;
        c_sk = (int)max((int64_t)0, min((int64_t)s - n, (int64_t)L));
    }

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int r32 = lane & 31, grp = lane >> 5;

    const T *Qg = (const T *)p.Q;
    const size_t kv_stride = (size_t)Hkv * D;
    const int row_bytes = Hkv * D * (int)sizeof(T);
    const T *Kg = (const T *)p.K + rbase * kv_stride + (size_t)hkv * D;
    const T *Vg = (const T *)p.V + rbase * kv_stride + (size_t)hkv * D;

    // The query row whose column of S^T / O^T this lane holds.
    const int pr = 32 * wave + r32;
    const int gq = pr / BQ, pos = q0 + pr % BQ;
    const bool rvalid = pos < L;
    const int trow = rvalid ? pos : L - 1;
    const int hq = hkv * G + gq;
    // Q and O go through LDS, each wave staging its own 32 rows, so that the
    // global accesses cover whole rows (QC lanes per row) rather than 16-32
    // bytes of each of 32 rows per instruction: that alone took the kernel's
    // load/store phases from 3.6 to about 6 TB/s.  Rows are 16-byte chunks,
    // XOR-swizzled by row so that the fragment reads spread over the banks.
    constexpr int QC = D * (int)sizeof(T) / 16;  // 16-B chunks per Q row
    constexpr int QN = 32 * QC / 64;             // 16-B loads per lane for the wave's 32 rows
    // global row of packed row r of this wave (rows past the end read row L-1,
    // never stored)
    auto grow = [&](int r) {
        const int prr = 32 * wave + r;
        const int pq = min(q0 + prr % BQ, L - 1);
        return ((rbase + pq) * Hq + hkv * G + prr / BQ) * D;
    };
    u32x4 qraw[QN];
#pragma unroll
    for (int n = 0; n < QN; ++n) {
        const int r = n * (64 / QC) + lane / QC, c = lane % QC;
        qraw[n] = *(const u32x4 *)((const unsigned char *)(Qg + grow(r)) + c * 16);
    }
    F qf[KS];

    // Key tiles: the sink tiles [0, ns) and the band [band_t0, kt_hi], in
    // the index space of K (for a chunk: sinks are the chunk rows whose
    // position is at most s, and the band reaches R = w - s rows back).
    const int R = w - s;
    const int sk = CK ? c_sk : s;
    const int band_lo = max(sk, q0 - R + 1);  // smallest band key of any row here
    const int ns = (min(sk, qlast + 1) + kKB - 1) / kKB;
    const int kt_hi = qlast / kKB;
    const int band_t0 = max(band_lo / kKB, ns);
    const int nband = band_lo <= qlast ? max(0, kt_hi - band_t0 + 1) : 0;
    // Cache tiles, visited first: only those holding a slot that some row of
    // this block attends.  Every row attends the sink slots [0, sinks_in);
    // row trow reaches ring offsets [h + trow + 2 - R, h] and, once the ring
    // is full, [h + trow + 2, R) (see cache_bits below), so the block's first
    // row reaches furthest.  The three slot ranges come in increasing order;
    // each range's tiles start past the tiles listed before it, so a tile
    // shared by two ranges is listed once.  (Plain scalars: arrays here
    // would be given a per-thread copy in LDS.)
    int ct0 = 0, cn0 = 0, ct1 = 0, cn1 = 0, ct2 = 0, cn2 = 0;
    if constexpr (CK) {
        const int h = c_head, r0 = q0 + 2;
        const int hi0 = c_sinks;
        const int lo1 = s + max(0, h + r0 - R), hi1 = c_any ? s + h + 1 : 0;
        const int lo2 = s + h + r0, hi2 = c_full ? w : 0;
        int next = 0;  // first tile not yet listed
        if (hi0 > 0) {
            cn0 = (hi0 - 1) / kKB + 1;
            next = cn0;
        }
        if (lo1 < hi1) {
            ct1 = max(next, lo1 / kKB);
            cn1 = max(0, (hi1 - 1) / kKB + 1 - ct1);
            next = ct1 + cn1;
        }
        if (lo2 < hi2) {
            ct2 = max(next, lo2 / kKB);
            cn2 = max(0, (hi2 - 1) / kKB + 1 - ct2);
        }
    }
    const int nct = cn0 + cn1 + cn2;
    // slot of the first row of cache tile i (i < nct)
    auto cache_slot0 = [&](int i) {
        const int t = i < cn0 ? ct0 + i : i < cn0 + cn1 ? ct1 + i - cn0 : ct2 + i - cn0 - cn1;
        return t * kKB;
    };
    // Packed first tile: when the band starts past the first tile, tile 0
    // holds the s sink rows and then the first kKB - s band rows, and the band
    // continues from there, so the sinks need no tile of their own.
    const bool pack = !CK && s > 0 && s < kKB && band_lo >= kKB && band_lo <= qlast;
    const int ntiles = pack ? (s + qlast - band_lo + 1 + kKB - 1) / kKB : nct + ns + nband;
    // keys every row of the block attends without a per-element test: the
    // sinks [0, sk) and [full_lo, q0]; when full_lo == sk (the last row's
    // band reaches back to the sinks) that is every key up to q0
    const int full_lo = max(sk, qlast - R + 1);
    const T *Kcb = nullptr, *Vcb = nullptr;  // this (batch, kv-head)'s cache block
    if constexpr (CK && !PG) {
        Kcb = (const T *)p.Kc + (size_t)bh * w * D;
        Vcb = (const T *)p.Vc + (size_t)bh * w * D;
    }

    const float c = 1.4426950408889634f * rsqrtf((float)D);  // log2(e)/sqrt(d)
    const float lazy_raw = kLazy / c;                          // threshold in raw score units
    float m = -INFINITY;
    // this lane's share of its row's sum of p (the row's keys of a tile are
    // split between lanes l and l^32; the halves are added at the end)
    float lsum = 0.f, lsum2 = 0.f;
    floatx16 oacc[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[dt][i] = 0.f;
    if (p.sink_logit) {
        // Learned sink: e^b in the denominator with no value.  Start the
        // running max at b (in raw score units, b*sqrt(d)) with the row sum
        // e^(b - b) = 1; the online softmax then carries the term exactly.
        const float bl = p.sink_logit[hq];
        if (bl > -INFINITY) {
            m = bl * sqrtf((float)D);
            lsum = grp == 0 ? 1.f : 0.f;  // e^(b - b), counted once per row
        }
    }

    // first key (in K's index space) of chunk tile i, i counted after the
    // cache tiles (packed mode: tile i >= 1 starts kKB*i - s keys into the band)
    auto tile_key = [&](int i) {
        if (pack) return i == 0 ? 0 : band_lo + kKB * i - s;
        return (i < ns ? i : band_t0 + (i - ns)) * kKB;
    };
    // Tile i's rows: cache slots for i < nct, else rows of K / V.  Uniform
    // selects, so one load path serves both.
    // (The packed tile 0 is fetched once, before the loop; a re-fetch of tile
    // 0 past the last tile loads other rows, but it is never stored.)
    auto fetch = [&](TileStager<T, D> &st, int i) {
        const bool cache = CK && i < nct;
        const T *kc = Kcb, *vc = Vcb;
        int c0 = cache ? cache_slot0(i) : 0, crows = c_nvalid;
        if constexpr (PG) {
            // the tile's 32 slots sit in one page (pages hold a multiple of
            // 32): rows from that page's row c0 % page; a table entry outside
            // the pool reads as zero rows
            const int pi = cache ? p.pg.block_table[(size_t)b * p.pg.pages_per_seq + c0 / p.pg.page] : -1;
            const bool ok = pi >= 0 && pi < p.pg.num_pages;
            const size_t row0 = ((size_t)(ok ? pi : 0) * Hkv + hkv) * p.pg.page + c0 % p.pg.page;
            kc = (const T *)p.pg.Kp + row0 * D;
            vc = (const T *)p.pg.Vp + row0 * D;
            crows = ok ? min(kKB, c_nvalid - c0) : 0;
            c0 = 0;
        }
        st.load(cache ? kc : Kg, cache ? vc : Vg, cache ? D * (int)sizeof(T) : row_bytes,
                cache ? c0 : tile_key(i - nct), cache ? crows : L, tid);
    };
    // Slots of a cache tile that chunk row `row` attends, as bits.  The row is
    // at position t = n + row + 1, d = t - n = row + 1 positions past the
    // cache.  Sinks: slots [0, min(s, n)).  Ring (r = slot - s): position n
    // sits at r = h and the ring holds consecutive positions backwards from
    // there, wrapping; position p is attended when p > t - R, which keeps
    // r in [h + d - R + 1, h] and, once the ring is full, r in [h + d + 1, R).
    // Both ring ranges shrink as d grows, so a slot the block's last row
    // attends is attended by every row of the block.
    auto cache_bits = [&](int slot0, int row) {
        const int dd = row + 1, h = c_head;
        uint32_t ok = bit_range(-slot0, c_sinks - slot0);
        if (c_any) {
            ok |= bit_range(s + max(0, h + dd - R + 1) - slot0, s + h + 1 - slot0);
            if (c_full) ok |= bit_range(s + h + dd + 1 - slot0, w - slot0);
        }
        return ok;
    };

    // One trip: S^T, softmax and O^T for the NT tiles it0, it0+1, .. held in
    // LDS at `stage`.  The tiles share one softmax step (one row max across
    // the lane pair, one rescale test), so its fixed costs, the barrier and
    // the drain between the S^T and O^T products are paid once per NT tiles.
    auto compute = [&](int it0, const unsigned char *stage, auto ntc, auto &&mid) {
        constexpr int NT = decltype(ntc)::value;

        // S^T = K Q^T, one accumulator per tile.  The first tile's K fragments
        // are all requested before its first MFMA (the LDS latency is paid
        // once); each later tile's fragments are requested between the MFMAs
        // of the tile before, one per MFMA.
        auto kfrag = [&](int h, int kk) {
            return load_frag<F>(stage + h * Lds::STAGE + r32 * Lds::KROW + (8 * grp + 16 * kk) * (int)sizeof(T));
        };
        // fp32 fragments are twice the registers: there the tile's K
        // fragments are requested two steps ahead of their MFMAs instead of
        // all at once (all at once spilled at d = 128).
        constexpr int KPRE = std::is_same_v<T, float> ? 2 : KS;  // fragments requested up front
        F kf[2][KS];
#pragma unroll
        for (int kk = 0; kk < KPRE; ++kk) kf[0][kk] = kfrag(0, kk);
        __builtin_amdgcn_sched_barrier(0);
        floatx16 sacc[NT];
#pragma unroll
        for (int h = 0; h < NT; ++h) {
#pragma unroll
            for (int i = 0; i < 16; ++i) sacc[h][i] = 0.f;
#pragma unroll
            for (int kk = 0; kk < KS; ++kk) {
                if (h == 0 && kk + KPRE < KS) kf[0][kk + KPRE] = kfrag(0, kk + KPRE);
                sacc[h] = mma32x32x16(kf[h & 1][kk], qf[kk], sacc[h]);
                if (h + 1 < NT) kf[(h + 1) & 1][kk] = kfrag(h + 1, kk);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        // the next trip's tiles go to LDS, and the loads of the one after are
        // issued, while the S^T products drain
        mid();
        __builtin_amdgcn_sched_barrier(0);

        float sc[16 * NT];
        float mx = -INFINITY;
#pragma unroll
        for (int h = 0; h < NT; ++h) {
            float *sh = sc + 16 * h;
#pragma unroll
            for (int i = 0; i < 16; ++i) sh[i] = sacc[h][i];
            const int it = it0 + h;
            const bool ctile = CK && it < nct;
            const int key0 = ctile ? cache_slot0(it) : tile_key(it - nct);
            const bool ptile = pack && it == 0;
            // a cache tile needs no per-element test when the block's last
            // row attends all of its slots (most ring tiles behind a full ring)
            const bool full = ctile ? cache_bits(key0, qlast) == 0xffffffffu
                                    : !ptile && (key0 + kKB - 1 <= q0) &&
                                          ((key0 + kKB <= sk) || (key0 >= full_lo) || (full_lo == sk));
            if (!full) {
                // Keys of this tile the row attends, as bits: the sinks
                // [0, min(sk, t+1)) and the band [max(sk, t-R+1), t]; or, for a
                // cache tile, the slots cache_bits gives; or, for the packed tile,
                // the sinks in rows 0..s-1 and band keys band_lo + (row - s).
                const int t = trow - key0;
                const uint32_t ok = ctile ? cache_bits(key0, trow)
                                    : ptile ? bit_range(0, min(s, trow + 1)) |
                                                  bit_range(s + max(band_lo, trow - R + 1) - band_lo,
                                                            s + trow + 1 - band_lo)
                                            : bit_range(-key0, min(sk, trow + 1) - key0) |
                                                  bit_range(max(sk, trow - R + 1) - key0, t + 1);
                const uint32_t mine = ok >> (4 * grp);
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    // all ones where the key is attended (its bit, sign-extended)
                    const uint32_t keep = (uint32_t)((int32_t)(mine << (31 - (8 * (e >> 2) + (e & 3)))) >> 31);
                    sh[e] = __uint_as_float((__float_as_uint(sh[e]) & keep) | (0xff800000u & ~keep));
                }
            }
            // a tree of three-input maxima (depth 3 instead of a chain of 8)
            const float m0 = fmaxf(fmaxf(sh[0], sh[1]), sh[2]), m1 = fmaxf(fmaxf(sh[3], sh[4]), sh[5]);
            const float m2 = fmaxf(fmaxf(sh[6], sh[7]), sh[8]), m3 = fmaxf(fmaxf(sh[9], sh[10]), sh[11]);
            const float m4 = fmaxf(fmaxf(sh[12], sh[13]), sh[14]);
            mx = fmaxf(mx, fmaxf(fmaxf(fmaxf(m0, m1), m2), fmaxf(fmaxf(m3, m4), sh[15])));
        }
        {
            // lanes l and l^32 hold the same query row's other keys
            const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
            mx = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
        }

        const bool raise = mx > m + lazy_raw;  // true on the first finite max
        if (__builtin_amdgcn_ballot_w64(raise)) {
            const float mnew = raise ? mx : m;
            const float alpha = raise ? fast_exp2((m - mnew) * c) : 1.f;  // m = -inf gives 0
            lsum *= alpha;
            lsum2 *= alpha;
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) oacc[dt] *= alpha;
            m = mnew;
        }
        const float mc = (m == -INFINITY ? 0.f : m) * c;
        float pv[16 * NT];
#pragma unroll
        for (int e = 0; e < 16 * NT; ++e) pv[e] = fast_exp2(fmaf(sc[e], c, -mc));

        // O^T += V^T P^T, two 16-key contraction steps per tile
#pragma unroll
        for (int h = 0; h < NT; ++h) {
            const unsigned char *vt = stage + h * Lds::STAGE + Lds::KTILE;
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                float pk[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) pk[e] = pv[16 * h + 8 * ks + e];
                const F pf = to_frag<F>(pk);
                if (ks == 0) lsum = add_row_part(pf, lsum);
                else lsum2 = add_row_part(pf, lsum2);
#pragma unroll
                for (int dt = 0; dt < DT; ++dt) {
                    const F vf = VFrag<T, D>::load(vt, dt, ks, lane);
                    oacc[dt] = mma32x32x16(vf, pf, oacc[dt]);
                }
            }
        }
    };

    // One register staging set holds the next trip's tiles: in trip j, once
    // its S^T products are issued, they go to the LDS stage trip j-1 used and
    // the tiles of trip j+2 are requested at once, so global loads have a
    // whole trip to land and the stores and load issue fill the wait for the
    // S^T results (before: at the end of the trip, in front of the barrier;
    // +1.5 % at w = 512, +2.5 % on a 128-workgroup grid, -1 % at w = 128).
    // Within a trip, a tile index past the last tile re-reads the last tile
    // (such rows are stored but never read); trips wholly past the end are
    // not fetched: a wave cannot end while its loads are in flight, so a
    // useless fetch at the last trips held every workgroup for one more
    // memory round trip (1-3 % of the launch).
    constexpr int TPT = Lds::TPT;
    TileStager<T, D> st[TPT];
    auto fetch_trip = [&](int j) {
#pragma unroll
        for (int h = 0; h < TPT; ++h) fetch(st[h], max(0, min(TPT * j + h, ntiles - 1)));
    };
    auto store_trip = [&](int j) {
#pragma unroll
        for (int h = 0; h < TPT; ++h) st[h].store(smem + (j & 1) * Lds::PSTAGE + h * Lds::STAGE, tid);
    };
    if (pack)
        st[0].load_packed(Kg, Vg, row_bytes, L, tid, s, band_lo);
    else
        fetch(st[0], 0);
#pragma unroll
    for (int h = 1; h < TPT; ++h) fetch(st[h], max(0, min(h, ntiles - 1)));
    {
        // this wave's Q rows into LDS, then its fragments out of it
        unsigned char *qw = smem + wave * 32 * QC * 16;
#pragma unroll
        for (int n = 0; n < QN; ++n) {
            const int r = n * (64 / QC) + lane / QC, c = lane % QC;
            *(u32x4 *)(qw + r * QC * 16 + ((c ^ (r % QC)) * 16)) = qraw[n];
        }
        constexpr int FC = 8 * (int)sizeof(T) / 16;  // 16-B chunks per fragment
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) {
            const int c0 = (8 * grp + 16 * kk) * (int)sizeof(T) / 16;
            u32x4 part[FC];
#pragma unroll
            for (int t = 0; t < FC; ++t)
                part[t] = *(const u32x4 *)(qw + r32 * QC * 16 + (((c0 + t) ^ (r32 % QC)) * 16));
            qf[kk] = __builtin_bit_cast(F, part);
        }
    }
    __syncthreads();  // every wave has its Q fragments before tile 0 overwrites the rows
    if (ntiles > 0) {
        store_trip(0);
        // Retire every load issued so far (Q fragments, trip 0): otherwise the
        // compiler cannot tell the Q registers are ready and waits for all
        // outstanding loads -- the prefetches included -- on every trip.
        __builtin_amdgcn_s_waitcnt(0);
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) asm volatile("" : "+v"(qf[kk]));
        if (TPT < ntiles) fetch_trip(1);
    }
    __syncthreads();
    // Trips of TPT tiles, then a possible single tile.
    const int nfull = ntiles / TPT;
    int j = 0;
    for (; j < nfull; ++j) {
        compute(TPT * j, smem + (j & 1) * Lds::PSTAGE, std::integral_constant<int, TPT>{}, [&] {
            store_trip(j + 1);
            if (TPT * (j + 2) < ntiles) fetch_trip(j + 2);
        });
        __syncthreads();
    }
    if (TPT * j < ntiles) {
        compute(TPT * j, smem + (j & 1) * Lds::PSTAGE, std::integral_constant<int, 1>{}, [] {});
        __syncthreads();
    }

    lsum += lsum2;
    const auto lsw = __builtin_amdgcn_permlane32_swap(__float_as_uint(lsum), __float_as_uint(lsum), false, false);
    const float lt = __uint_as_float(lsw[0]) + __uint_as_float(lsw[1]);
    const float inv = 1.f / lt;
    constexpr int OC = D * (int)sizeof(TO) / 16;  // 16-B chunks per O row
    if constexpr (4 * 32 * OC * 16 <= Lds::BYTES) {
        // O rows through LDS (the stages are free: every wave has passed the
        // last trip's barrier), then whole rows to global memory
        unsigned char *ow = smem + wave * 32 * OC * 16;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int byte = (32 * dt + 8 * j + 4 * grp) * (int)sizeof(TO);
                store4<TO>((TO *)(ow + r32 * OC * 16 + (((byte / 16) ^ (r32 % OC)) * 16) + byte % 16),
                           oacc[dt][4 * j] * inv, oacc[dt][4 * j + 1] * inv, oacc[dt][4 * j + 2] * inv,
                           oacc[dt][4 * j + 3] * inv);
            }
#pragma unroll
        for (int n = 0; n < 32 * OC / 64; ++n) {
            const int r = n * (64 / OC) + lane / OC, c = lane % OC;
            const u32x4 v = *(const u32x4 *)(ow + r * OC * 16 + ((c ^ (r % OC)) * 16));
            // non-temporal: O is written once and not read back by this
            // kernel, so its lines should not push K/V tiles (re-read by
            // neighbouring blocks) out of L2.  Measured: +8.5 % at w = 128,
            // +4 % at 256, +1.7 % at 512, +15 % on a batch-32 512-token prompt.
            if (q0 + (32 * wave + r) % BQ < L)
                __builtin_nontemporal_store(v, (u32x4 *)((unsigned char *)((TO *)p.O + grow(r)) + c * 16));
        }
    } else if (rvalid) {
        TO *orow = (TO *)p.O + ((rbase + trow) * Hq + hq) * D;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                store4<TO>(orow + 32 * dt + 8 * j + 4 * grp, oacc[dt][4 * j] * inv, oacc[dt][4 * j + 1] * inv,
                          oacc[dt][4 * j + 2] * inv, oacc[dt][4 * j + 3] * inv);
    }
    if (rvalid && p.lse && grp == 0) {
        const size_t li = VL ? (size_t)hq * p.total + rbase + trow : ((size_t)b * Hq + hq) * L + trow;
        p.lse[li] = m * rsqrtf((float)D) + logf(lt);
    }
}

template <typename T, typename TO, int D, int G, bool CK, bool VL, bool PG>
hipError_t launch_t(const PrefillParams &p, hipStream_t st)
{
    constexpr int BQ = kRowsWG / G;
    const long long nqb = (p.L + BQ - 1) / BQ;
    const long long total = nqb * p.B * p.Hkv;
    if (total <= 0) return hipSuccess;
    if (total > 0x7fffffffLL) return hipErrorInvalidValue;
    hipLaunchKernelGGL((swa_prefill_kernel<T, TO, D, G, CK, VL, PG>), dim3((unsigned)total), dim3(kThreads), 0, st, p);
    return hipGetLastError();
}

template <typename T, typename TO, int D, bool CK, bool VL, bool PG>
hipError_t launch_g(int G, const PrefillParams &p, hipStream_t st)
{
    switch (G) {
    case 1: return launch_t<T, TO, D, 1, CK, VL, PG>(p, st);
    case 2: return launch_t<T, TO, D, 2, CK, VL, PG>(p, st);
    case 4: return launch_t<T, TO, D, 4, CK, VL, PG>(p, st);
    case 8: return launch_t<T, TO, D, 8, CK, VL, PG>(p, st);
    default: return hipErrorInvalidValue;
    }
}

template <typename T, typename TO, bool CK, bool VL, bool PG>
hipError_t launch_d(int d, int G, const PrefillParams &p, hipStream_t st)
{
    return d == 128 ? launch_g<T, TO, 128, CK, VL, PG>(G, p, st) : launch_g<T, TO, 64, CK, VL, PG>(G, p, st);
}

template <bool CK, bool VL = false> hipError_t launch_dt(Dt in, Dt out, int d, int G, const PrefillParams &p, hipStream_t st)
{
    if (in == Dt::BF16)
        return out == Dt::BF16 ? launch_d<bf16, bf16, CK, VL, false>(d, G, p, st)
                               : launch_d<bf16, float, CK, VL, false>(d, G, p, st);
    if (out != Dt::F32) return hipErrorInvalidValue;
    return launch_d<float, float, CK, VL, false>(d, G, p, st);
}

}  // namespace

hipError_t launch_prefill(Dt in, Dt out, int d, int G, const PrefillParams &p, hipStream_t st)
{
    return launch_dt<false>(in, out, d, G, p, st);
}

hipError_t launch_prefill_chunk(Dt in, Dt out, int d, int G, const PrefillParams &p, hipStream_t st)
{
    return launch_dt<true>(in, out, d, G, p, st);
}

hipError_t launch_prefill_varlen(Dt in, Dt out, int d, int G, const PrefillParams &p, hipStream_t st)
{
    return launch_dt<false, true>(in, out, d, G, p, st);
}

hipError_t launch_prefill_chunk_paged(Dt out, int d, int G, const PrefillParams &p, hipStream_t st)
{
    // paged caches are bf16; O is bf16 or fp32
    return out == Dt::BF16 ? launch_d<bf16, bf16, true, true, true>(d, G, p, st)
                           : launch_d<bf16, float, true, true, true>(d, G, p, st);
}

}  // namespace swa
