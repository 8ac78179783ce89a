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
//   query positions for all G query heads sharing that kv-head, i.e. 128
//   packed (head, position) rows; each wave owns 32 rows as two 16-row MFMA
//   tiles.  K/V tiles of 32 keys are staged through LDS once and read by all
//   G heads.  The key tiles visited are the sink tiles [0, s) and the window
//   band of the block; everything else is skipped, so work per row is
//   O(w), not O(t).
//
// Per 32-key tile and 16-row tile, with S^T = K Q^T so the query row is the
// MFMA column (lane % 16) and stays in one lane group:
//   S^T (32 keys x 16 rows) : 2 x (d/32) MFMA 16x16x32, K from LDS, Q in VGPRs
//   online softmax in fp32 : row max across the 4 lane groups (2 shuffles),
//                            exp2 with the 1/sqrt(d)*log2(e) scale folded in
//   O^T (d x 16 rows) += V^T P^T : d/16 MFMAs, V^T from LDS, P^T straight from
//                            the S^T accumulators (no shuffle).
// The key order inside the PV contraction is permuted to match the S^T
// accumulator layout; V^T is written to LDS in that order.
#include "device_common.h"
#include "swa_internal.h"

namespace swa {
namespace {

constexpr int kThreads = 256;
constexpr int kKB = 32;       // keys per LDS tile
constexpr int kRowsWG = 128;  // packed (head, position) rows per workgroup

template <typename T, int D> struct PrefillLds {
    static constexpr int ES = sizeof(T);
    static constexpr int KROW = D * ES + 16;  // bytes per K row (16 B pad: conflict-free reads)
    static constexpr int VROW = kKB * ES;     // bytes per V^T row (chunks XOR-swizzled)
    static constexpr int KTILE = kKB * KROW;
    static constexpr int VTILE = D * VROW;
    static constexpr int STAGE = KTILE + VTILE;
    static constexpr int BYTES = 2 * STAGE;
    static constexpr int CPR = D * ES / 16;  // 16-byte chunks per global row
};

// Position of key k (0..31 within the tile) inside the PV contraction.  The
// S^T accumulator of lane group g holds keys 4g..4g+3 (first 16-key half) and
// 16+4g..16+4g+3 (second half); as the PV operand those 8 values are
// contraction indices 8g..8g+7.
__device__ __forceinline__ int pv_index(int k)
{
    const int half = k >> 4, g = (k >> 2) & 3, i = k & 3;
    return 8 * g + 4 * half + i;
}

template <typename T> __device__ __forceinline__ int vt_swizzle(int dim);
// bf16: 4 chunks of 16 B per 64-B row, two rows per 32 banks.
template <> __device__ __forceinline__ int vt_swizzle<bf16>(int dim) { return ((dim >> 1) ^ (dim >> 3)) & 3; }
// fp32: 8 chunks per 128-B row.
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

template <int D> struct TileStager<bf16, D> {
    using Lds = PrefillLds<bf16, D>;
    static constexpr int NK = kKB * Lds::CPR / kThreads;       // 16-B K chunks per thread
    static constexpr int NVU = 16 * Lds::CPR;                  // (key pair, chunk) units
    u32x4 k[NK > 0 ? NK : 1];
    u32x4 v0, v1;

    __device__ __forceinline__ void load(const bf16 *Kg, const bf16 *Vg, size_t row_stride, int key0,
                                         int L, int tid)
    {
#pragma unroll
        for (int u = 0; u < NK; ++u) {
            const int ci = tid + kThreads * u, row = ci / Lds::CPR, col = ci % Lds::CPR;
            const int pos = key0 + row;
            k[u] = pos < L ? *(const u32x4 *)(Kg + (size_t)pos * row_stride + col * 8) : u32x4{0, 0, 0, 0};
        }
        if (tid < NVU) {
            const int j = tid / Lds::CPR, c = tid % Lds::CPR;
            const int p0 = key0 + 2 * j, p1 = p0 + 1;
            v0 = p0 < L ? *(const u32x4 *)(Vg + (size_t)p0 * row_stride + c * 8) : u32x4{0, 0, 0, 0};
            v1 = p1 < L ? *(const u32x4 *)(Vg + (size_t)p1 * row_stride + c * 8) : u32x4{0, 0, 0, 0};
        }
    }

    __device__ __forceinline__ void store(unsigned char *stage, int tid) const
    {
#pragma unroll
        for (int u = 0; u < NK; ++u) {
            const int ci = tid + kThreads * u, row = ci / Lds::CPR, col = ci % Lds::CPR;
            *(u32x4 *)(stage + row * Lds::KROW + col * 16) = k[u];
        }
        if (tid < NVU) {
            const int j = tid / Lds::CPR, c = tid % Lds::CPR;
            unsigned char *vt = stage + Lds::KTILE;
            const int kp = pv_index(2 * j);  // keys 2j and 2j+1 are adjacent in PV order
            uint32_t pk[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const uint32_t a = v0[e >> 1], b = v1[e >> 1];
                pk[e] = (e & 1) ? ((a >> 16) | (b & 0xffff0000u)) : ((a & 0xffffu) | (b << 16));
            }
            // Lanes whose chunk index has bit 2 set write the dims of each pair
            // in swapped order, which halves the LDS bank collisions.
            const int flip = (c >> 2) & 1;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int ee = e ^ flip;
                const uint32_t val = flip ? pk[e ^ 1] : pk[e];
                *(uint32_t *)(vt + vt_offset<bf16, D>(8 * c + ee, kp)) = val;
            }
        }
    }
};

template <int D> struct TileStager<float, D> {
    using Lds = PrefillLds<float, D>;
    static constexpr int NK = kKB * Lds::CPR / kThreads;
    static constexpr int NV = kKB * (D / 4) / kThreads;
    u32x4 k[NK];
    u32x4 v[NV];

    __device__ __forceinline__ void load(const float *Kg, const float *Vg, size_t row_stride, int key0,
                                         int L, int tid)
    {
#pragma unroll
        for (int u = 0; u < NK; ++u) {
            const int ci = tid + kThreads * u, row = ci / Lds::CPR, col = ci % Lds::CPR;
            const int pos = key0 + row;
            k[u] = pos < L ? *(const u32x4 *)(Kg + (size_t)pos * row_stride + col * 4) : u32x4{0, 0, 0, 0};
        }
#pragma unroll
        for (int u = 0; u < NV; ++u) {
            const int ci = tid + kThreads * u, key = ci / (D / 4), c4 = ci % (D / 4);
            const int pos = key0 + key;
            v[u] = pos < L ? *(const u32x4 *)(Vg + (size_t)pos * row_stride + c4 * 4) : u32x4{0, 0, 0, 0};
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

template <typename T, int D> __device__ __forceinline__ typename Frag<T>::type load_vt_frag(const unsigned char *vt, int dim, int grp);
template <> __device__ __forceinline__ bf16x8 load_vt_frag<bf16, 64>(const unsigned char *vt, int dim, int grp)
{
    return *(const bf16x8 *)(vt + vt_offset<bf16, 64>(dim, 8 * grp));
}
template <> __device__ __forceinline__ bf16x8 load_vt_frag<bf16, 128>(const unsigned char *vt, int dim, int grp)
{
    return *(const bf16x8 *)(vt + vt_offset<bf16, 128>(dim, 8 * grp));
}
template <int D> __device__ __forceinline__ floatx8 load_vt_frag_f32(const unsigned char *vt, int dim, int grp)
{
    const floatx4 a = *(const floatx4 *)(vt + vt_offset<float, D>(dim, 8 * grp));
    const floatx4 b = *(const floatx4 *)(vt + vt_offset<float, D>(dim, 8 * grp + 4));
    return floatx8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}
template <> __device__ __forceinline__ floatx8 load_vt_frag<float, 64>(const unsigned char *vt, int dim, int grp)
{
    return load_vt_frag_f32<64>(vt, dim, grp);
}
template <> __device__ __forceinline__ floatx8 load_vt_frag<float, 128>(const unsigned char *vt, int dim, int grp)
{
    return load_vt_frag_f32<128>(vt, dim, grp);
}

template <typename T> __device__ __forceinline__ void store4(T *dst, floatx4 v, float inv);
template <> __device__ __forceinline__ void store4<bf16>(bf16 *dst, floatx4 v, float inv)
{
    bf16x4 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) r[i] = (bf16)(v[i] * inv);
    *(bf16x4 *)dst = r;
}
template <> __device__ __forceinline__ void store4<float>(float *dst, floatx4 v, float inv)
{
    *(floatx4 *)dst = floatx4{v[0] * inv, v[1] * inv, v[2] * inv, v[3] * inv};
}

template <typename T, int D, int G>
__global__ __launch_bounds__(kThreads) void swa_prefill_kernel(PrefillParams p)
{
    using F = typename Frag<T>::type;
    using Lds = PrefillLds<T, D>;
    constexpr int BQ = kRowsWG / G;  // query positions per workgroup
    constexpr int KS = D / 32;       // 32-deep contraction steps of Q.K
    constexpr int DT = D / 16;       // 16-dim output tiles
    __shared__ __align__(16) unsigned char smem[Lds::BYTES];

    const int L = p.L, Hq = p.Hq, Hkv = p.Hkv, w = p.w, s = p.s;
    const int nqb = (L + BQ - 1) / BQ;
    const int total = nqb * p.B * Hkv;
    const int lid = xcd_remap((int)blockIdx.x, total);
    const int qb = lid % nqb, bh = lid / nqb;
    const int b = bh / Hkv, hkv = bh % Hkv;
    const int q0 = qb * BQ;
    const int qlast = min(q0 + BQ, L) - 1;

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int r16 = lane & 15, grp = lane >> 4;

    const T *Qg = (const T *)p.Q;
    const size_t kv_stride = (size_t)Hkv * D;
    const T *Kg = (const T *)p.K + (size_t)b * L * kv_stride + (size_t)hkv * D;
    const T *Vg = (const T *)p.V + (size_t)b * L * kv_stride + (size_t)hkv * D;

    // The two rows (one per 16-row tile) whose query, softmax state and
    // output column this lane holds.
    int trow[2], hq[2];
    bool rvalid[2];
    F qf[2][KS];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
        const int pr = 32 * wave + 16 * rt + r16;
        const int g = pr / BQ, pos = q0 + pr % BQ;
        rvalid[rt] = pos < L;
        trow[rt] = rvalid[rt] ? pos : L - 1;
        hq[rt] = hkv * G + g;
        const T *qrow = Qg + (((size_t)b * L + trow[rt]) * Hq + hq[rt]) * D;
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) {
            if (rvalid[rt]) qf[rt][kk] = load_frag<F>(qrow + 8 * grp + 32 * kk);
            else qf[rt][kk] = F{};
        }
    }

    // Key tiles: the sink tiles [0, ns) and the band [band_t0, kt_hi].
    const int band_lo = max(s, q0 - (w - s) + 1);  // smallest band key of any row here
    const int ns = (min(s, qlast + 1) + kKB - 1) / kKB;
    const int kt_hi = qlast / kKB;
    const int band_t0 = max(band_lo / kKB, ns);
    const int nband = band_lo <= qlast ? max(0, kt_hi - band_t0 + 1) : 0;
    const int ntiles = ns + nband;
    // keys every row of the block may see without a per-element test
    const int full_lo = max(s, qlast - (w - s) + 1);

    const float c = 1.4426950408889634f * rsqrtf((float)D);  // log2(e)/sqrt(d)
    float m[2] = {-INFINITY, -INFINITY}, l[2] = {0.f, 0.f};
    floatx4 oacc[2][DT];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) oacc[rt][dt] = floatx4{0.f, 0.f, 0.f, 0.f};

    TileStager<T, D> stg;
    auto tile_key = [&](int i) { return (i < ns ? i : band_t0 + (i - ns)) * kKB; };

    if (ntiles > 0) {
        stg.load(Kg, Vg, kv_stride, tile_key(0), L, tid);
        stg.store(smem, tid);
    }
    __syncthreads();

    for (int it = 0; it < ntiles; ++it) {
        const int key0 = tile_key(it);
        if (it + 1 < ntiles) stg.load(Kg, Vg, kv_stride, tile_key(it + 1), L, tid);

        const unsigned char *kt = smem + (it & 1) * Lds::STAGE;
        const unsigned char *vt = kt + Lds::KTILE;

        // S^T = K Q^T for both 16-key halves and both row tiles
        floatx4 sacc[2][2];
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) sacc[rt][hf] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int hf = 0; hf < 2; ++hf)
#pragma unroll
            for (int kk = 0; kk < KS; ++kk) {
                const F kf = load_frag<F>(kt + (16 * hf + r16) * Lds::KROW + (8 * grp + 32 * kk) * (int)sizeof(T));
#pragma unroll
                for (int rt = 0; rt < 2; ++rt) sacc[rt][hf] = mma16x16x32(kf, qf[rt][kk], sacc[rt][hf]);
            }

        const bool full = (key0 + kKB - 1 <= q0) && ((key0 + kKB <= s) || (key0 >= full_lo));
        F pf[2];
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
            float sc[8];
#pragma unroll
            for (int hf = 0; hf < 2; ++hf)
#pragma unroll
                for (int i = 0; i < 4; ++i) sc[4 * hf + i] = sacc[rt][hf][i];
            if (!full) {
                const int t = trow[rt];
#pragma unroll
                for (int hf = 0; hf < 2; ++hf)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int j = key0 + 16 * hf + 4 * grp + i;
                        // Branch-free on purpose: with short-circuit && / || the
                        // compiler (ROCm 7.2 clang, gfx950) dropped the window-edge
                        // test for the first element.
                        const bool ok = (j <= t) & ((j < s) | (j > t - (w - s)));
                        sc[4 * hf + i] = ok ? sc[4 * hf + i] : -INFINITY;
                    }
            }
            float mx = sc[0];
#pragma unroll
            for (int j = 1; j < 8; ++j) mx = fmaxf(mx, sc[j]);
            mx = wave_max_xor(mx, 16);
            mx = wave_max_xor(mx, 32);
            const float mnew = fmaxf(m[rt], mx);
            const float muse = mnew == -INFINITY ? 0.f : mnew;
            const float alpha = fast_exp2((m[rt] - muse) * c);
            const float mc = muse * c;
            float pv[8], rs = 0.f;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                pv[j] = fast_exp2(fmaf(sc[j], c, -mc));
                rs += pv[j];
            }
            l[rt] = fmaf(l[rt], alpha, rs);
            m[rt] = mnew;
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) oacc[rt][dt] *= alpha;
            pf[rt] = to_frag<F>(pv);
        }

        // O^T += V^T P^T
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
            const F vf = load_vt_frag<T, D>(vt, 16 * dt + r16, grp);
#pragma unroll
            for (int rt = 0; rt < 2; ++rt) oacc[rt][dt] = mma16x16x32(vf, pf[rt], oacc[rt][dt]);
        }

        if (it + 1 < ntiles) stg.store(smem + ((it + 1) & 1) * Lds::STAGE, tid);
        __syncthreads();
    }

    T *Og = (T *)p.O;
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
        float lt = l[rt];
        lt += __shfl_xor(lt, 16, 64);
        lt += __shfl_xor(lt, 32, 64);
        if (!rvalid[rt]) continue;
        const float inv = 1.f / lt;
        T *orow = Og + (((size_t)b * L + trow[rt]) * Hq + hq[rt]) * D;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) store4<T>(orow + 16 * dt + 4 * grp, oacc[rt][dt], inv);
        if (p.lse && grp == 0)
            p.lse[((size_t)b * Hq + hq[rt]) * L + trow[rt]] = m[rt] * rsqrtf((float)D) + logf(lt);
    }
}

template <typename T, int D, int G> hipError_t launch_t(const PrefillParams &p, hipStream_t st)
{
    constexpr int BQ = kRowsWG / G;
    const long long nqb = (p.L + BQ - 1) / BQ;
    const long long total = nqb * p.B * p.Hkv;
    if (total <= 0) return hipSuccess;
    if (total > 0x7fffffffLL) return hipErrorInvalidValue;
    hipLaunchKernelGGL((swa_prefill_kernel<T, D, G>), dim3((unsigned)total), dim3(kThreads), 0, st, p);
    return hipGetLastError();
}

template <typename T, int D> hipError_t launch_g(int G, const PrefillParams &p, hipStream_t st)
{
    switch (G) {
    case 1: return launch_t<T, D, 1>(p, st);
    case 2: return launch_t<T, D, 2>(p, st);
    case 4: return launch_t<T, D, 4>(p, st);
    case 8: return launch_t<T, D, 8>(p, st);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_prefill(Dt dt, int d, int G, const PrefillParams &p, hipStream_t st)
{
    if (dt == Dt::BF16) return d == 128 ? launch_g<bf16, 128>(G, p, st) : launch_g<bf16, 64>(G, p, st);
    return d == 128 ? launch_g<float, 128>(G, p, st) : launch_g<float, 64>(G, p, st);
}

}  // namespace swa
