// SWA(w,s) decode and cache append on gfx950.
//
// The cache of one (batch, kv-head) is a w x d block: s pinned sink slots and
// a (w - s)-slot ring.  After n appends its occupied slots 0..min(n,w)-1 hold
// exactly the positions the query at position n attends (the first s tokens
// plus the most recent w - s; paper.rainbus.top summary of arXiv 2608.28444,
// "滑窗注意力 SWA(w, s)" and "KV 缓存"; ai-blog.deepmagic.app, "他們測了什麼",
// where SWA is "a change of mask and of the KV-cache eviction policy").  A
// softmax does not depend on the order of its terms, so decode reads the
// occupied slots in physical order with no mask and no un-rotation.
//
// Decode is bound by HBM: per step it reads 2*min(n,w)*d elements per
// (batch, kv-head) and does 4*G*d flops per cached row (G query heads share
// each row).  Layout per wave: LPR lanes cover one cached row with 16-byte
// loads (LPR = 16 for bf16, d = 128), so each load instruction of a wave reads
// 64/LPR whole rows -- fully coalesced.  Each lane keeps the G query vectors
// for its d/LPR dims in registers; the score of a row is a partial dot product
// per lane reduced over the LPR lanes of the row.  The online softmax runs per
// chunk of rows with a wave-wide running max per head.  Waves of a workgroup
// walk interleaved row blocks of the same (batch, kv-head) and meet in LDS;
// long caches are further split over workgroups whose partial (max, sum, acc)
// triples a second kernel merges:  O = sum_j e^{m_j-M} acc_j / sum_j e^{m_j-M} l_j.
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

template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float x) { return (bf16)x; }
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }

template <typename T, int D, int G>
__global__ __launch_bounds__(kThreads) void swa_decode_kernel(DecodeParams p)
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
        float M = -INFINITY;
#pragma unroll
        for (int wv = 0; wv < kWaves; ++wv) M = fmaxf(M, sh_ml[wv][g][0]);
        float Ls = 0.f, A = 0.f;
#pragma unroll
        for (int wv = 0; wv < kWaves; ++wv) {
            const float f = fast_exp2(sh_ml[wv][g][0] - M);
            Ls = fmaf(f, sh_ml[wv][g][1], Ls);
            A = fmaf(f, sh_acc[wv][g][dim], A);
        }
        const int hq = hkv * G + g;
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

// Merge of split partials: one workgroup per (b, query head), one thread per dim.
template <typename T, int D>
__global__ __launch_bounds__(D) void swa_decode_merge_kernel(DecodeParams p)
{
    const int bq = blockIdx.x, dim = threadIdx.x;
    const float *part = p.part + (size_t)bq * p.nsplit * (D + 2);
    float M = -INFINITY;
    for (int j = 0; j < p.nsplit; ++j) M = fmaxf(M, part[j * (D + 2) + D]);
    float Ls = 0.f, A = 0.f;
    for (int j = 0; j < p.nsplit; ++j) {
        const float *pj = part + j * (D + 2);
        const float f = fast_exp2(pj[D] - M);
        Ls = fmaf(f, pj[D + 1], Ls);
        A = fmaf(f, pj[dim], A);
    }
    ((T *)p.O)[(size_t)bq * D + dim] = from_f32<T>(A / Ls);
}

// Append: copy the surviving new rows into their slots.  One thread per
// 16-byte chunk of a (survivor, b, kv-head) row, K and V together.
template <typename T, int D>
__global__ __launch_bounds__(kThreads) void swa_append_kernel(AppendParams p)
{
    constexpr int CPR = D * (int)sizeof(T) / 16;
    const int64_t n1 = p.b1 >= p.a1 ? p.b1 - p.a1 + 1 : 0;
    const int64_t n2 = p.b2 >= p.a2 ? p.b2 - p.a2 + 1 : 0;
    const int64_t total = (n1 + n2) * p.B * p.Hkv * CPR;
    for (int64_t u = (int64_t)blockIdx.x * kThreads + threadIdx.x; u < total;
         u += (int64_t)gridDim.x * kThreads) {
        const int chunk = (int)(u % CPR);
        int64_t rest = u / CPR;
        const int hkv = (int)(rest % p.Hkv);
        rest /= p.Hkv;
        const int b = (int)(rest % p.B);
        const int64_t j = rest / p.B;
        const int64_t pos = j < n1 ? p.a1 + j : p.a2 + (j - n1);
        const int64_t src_row = pos - p.n_before - 1;
        const int64_t slot = pos <= p.s ? pos - 1 : p.s + (pos - p.s - 1) % (p.w - p.s);
        const size_t src = (((size_t)b * p.n_new + src_row) * p.Hkv + hkv) * D;
        const size_t dst = (((size_t)b * p.Hkv + hkv) * p.w + slot) * D;
        const u32x4 *ks = (const u32x4 *)((const T *)p.Kn + src) + chunk;
        const u32x4 *vs = (const u32x4 *)((const T *)p.Vn + src) + chunk;
        *((u32x4 *)((T *)p.Kc + dst) + chunk) = *ks;
        *((u32x4 *)((T *)p.Vc + dst) + chunk) = *vs;
    }
}

template <typename T, int D, int G> hipError_t launch_decode_t(const DecodeParams &p, hipStream_t st)
{
    dim3 grid((unsigned)p.nsplit, (unsigned)(p.B * p.Hkv));
    hipLaunchKernelGGL((swa_decode_kernel<T, D, G>), grid, dim3(kThreads), 0, st, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || p.nsplit == 1) return e;
    hipLaunchKernelGGL((swa_decode_merge_kernel<T, D>), dim3((unsigned)(p.B * p.Hq)), dim3(D), 0, st, p);
    return hipGetLastError();
}

template <typename T, int D> hipError_t launch_decode_g(int G, const DecodeParams &p, hipStream_t st)
{
    switch (G) {
    case 1: return launch_decode_t<T, D, 1>(p, st);
    case 2: return launch_decode_t<T, D, 2>(p, st);
    case 4: return launch_decode_t<T, D, 4>(p, st);
    case 8: return launch_decode_t<T, D, 8>(p, st);
    default: return hipErrorInvalidValue;
    }
}

template <typename T, int D> hipError_t launch_append_t(const AppendParams &p, hipStream_t st)
{
    constexpr int CPR = D * (int)sizeof(T) / 16;
    const int64_t n1 = p.b1 >= p.a1 ? p.b1 - p.a1 + 1 : 0;
    const int64_t n2 = p.b2 >= p.a2 ? p.b2 - p.a2 + 1 : 0;
    const int64_t total = (n1 + n2) * p.B * p.Hkv * CPR;
    if (total <= 0) return hipSuccess;
    int64_t blocks = (total + kThreads - 1) / kThreads;
    if (blocks > 65536) blocks = 65536;
    hipLaunchKernelGGL((swa_append_kernel<T, D>), dim3((unsigned)blocks), dim3(kThreads), 0, st, p);
    return hipGetLastError();
}

}  // namespace

void decode_plan(int B, int Hkv, int nvalid, int *nsplit, int *rows_per_split, int *max_splits)
{
    const long long pairs = (long long)B * Hkv;
    int ns = 1;
    if (nvalid > 1024 && pairs < 1024) {
        const long long by_rows = (nvalid + 511) / 512;
        long long cap = 2048 / pairs;
        if (cap < 1) cap = 1;
        ns = (int)(by_rows < cap ? by_rows : cap);
    }
    *max_splits = ns;  // non-decreasing in nvalid, and >= the rounded count below
    int rps = (nvalid + ns - 1) / ns;
    rps = (rps + 127) / 128 * 128;
    if (rps < 128) rps = 128;
    ns = (nvalid + rps - 1) / rps;
    if (ns < 1) ns = 1;
    *nsplit = ns;
    *rows_per_split = rps;
}

hipError_t launch_decode(Dt dt, int d, int G, const DecodeParams &p, hipStream_t st)
{
    if (dt == Dt::BF16) return d == 128 ? launch_decode_g<bf16, 128>(G, p, st) : launch_decode_g<bf16, 64>(G, p, st);
    return d == 128 ? launch_decode_g<float, 128>(G, p, st) : launch_decode_g<float, 64>(G, p, st);
}

hipError_t launch_append(Dt dt, int d, const AppendParams &p, hipStream_t st)
{
    if (dt == Dt::BF16) return d == 128 ? launch_append_t<bf16, 128>(p, st) : launch_append_t<bf16, 64>(p, st);
    return d == 128 ? launch_append_t<float, 128>(p, st) : launch_append_t<float, 64>(p, st);
}

}  // namespace swa
