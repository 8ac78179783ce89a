// Host-only stand-ins for the HIP kernel launchers and the three HIP runtime
// calls the C ABI makes, for a CPU build of api.cpp + plan.cpp under
// AddressSanitizer / UndefinedBehaviorSanitizer.  Every launcher checks the
// parameters the host side hands it (ranges, plans, pointers) instead of
// launching; nothing here touches the (fake) device addresses.
#include <stdio.h>
#include <stdlib.h>

#include "swa_internal.h"

#define REQUIRE(c)                                                                  \
    do {                                                                            \
        if (!(c)) {                                                                 \
            fprintf(stderr, "stub check failed: %s (%s:%d)\n", #c, __FILE__, __LINE__); \
            abort();                                                                \
        }                                                                           \
    } while (0)

int g_launches = 0;

extern "C" {
const char *hipGetErrorString(hipError_t) { return "stubbed HIP error"; }
hipError_t hipGetDevice(int *d)
{
    *d = 0;
    return hipSuccess;
}
hipError_t hipStreamGetDevice(hipStream_t, hipDevice_t *d)
{
    *d = 0;
    return hipSuccess;
}
}

namespace swa {

static void check_prefill(Dt in, Dt out, int d, int G, const PrefillParams &p)
{
    REQUIRE(in == Dt::BF16 || in == Dt::F32);
    REQUIRE(out == in || (in == Dt::BF16 && out == Dt::F32));
    REQUIRE(d == 64 || d == 128);
    REQUIRE(G == 1 || G == 2 || G == 4 || G == 8);
    REQUIRE(p.Q && p.K && p.V && p.O);
    REQUIRE(p.B >= 1 && p.L >= 1 && p.Hq == G * p.Hkv);
    REQUIRE(p.w > p.s && p.s >= 0);
    ++g_launches;
}

hipError_t launch_prefill(Dt in, Dt out, int d, int G, const PrefillParams &p, hipStream_t)
{
    check_prefill(in, out, d, G, p);
    REQUIRE(!p.cu_seqlens && !p.Kc);
    return hipSuccess;
}

hipError_t launch_prefill_varlen(Dt in, Dt out, int d, int G, const PrefillParams &p, hipStream_t)
{
    check_prefill(in, out, d, G, p);
    REQUIRE(p.cu_seqlens && p.total >= p.L && p.total >= 1);
    return hipSuccess;
}

hipError_t launch_prefill_chunk(Dt in, Dt out, int d, int G, const PrefillParams &p, hipStream_t)
{
    check_prefill(in, out, d, G, p);
    REQUIRE(p.Kc && p.Vc);
    REQUIRE(p.nvalid >= 0 && p.nvalid <= p.w);
    REQUIRE(p.sinks_in >= 0 && p.sinks_in <= p.s && p.sinks_in <= p.nvalid);
    REQUIRE(p.sk >= 0 && p.sk <= p.L && p.sk <= p.s);
    REQUIRE(p.ring_head >= 0 && (p.ring_head < p.w - p.s || !p.ring_any));
    return hipSuccess;
}

hipError_t launch_prefill_chunk_paged(Dt out, int d, int G, const PrefillParams &p, hipStream_t)
{
    check_prefill(Dt::BF16, out, d, G, p);
    REQUIRE(p.cu_seqlens && p.total >= p.L && p.total >= 1 && !p.Kc && !p.Vc);
    REQUIRE(p.pg.Kp && p.pg.Vp && p.pg.block_table && p.pg.n);
    REQUIRE(p.pg.num_pages >= 1 && p.pg.page >= kDecodeChunk && p.pg.page % kDecodeChunk == 0);
    REQUIRE(p.pg.pages_per_seq == (p.w + p.pg.page - 1) / p.pg.page);
    return hipSuccess;
}

hipError_t launch_append(Dt dt, int d, const AppendParams &p, hipStream_t)
{
    REQUIRE(d == 64 || d == 128);
    REQUIRE(p.Kn && p.Vn && p.Kc && p.Vc && p.n_new >= 1);
    REQUIRE((dt == Dt::FP8) == (p.kv_scale != nullptr));
    const int64_t n = p.n_before, N = n + p.n_new;
    // survivors: inside the new positions, attended after the append, in
    // distinct slots (at most w of them)
    int64_t count = 0;
    if (p.b1 >= p.a1) {
        REQUIRE(p.a1 == n + 1 && p.b1 <= N && p.b1 <= p.s);
        count += p.b1 - p.a1 + 1;
    }
    if (p.b2 >= p.a2) {
        REQUIRE(p.a2 >= n + 1 && p.a2 > p.s && p.b2 == N && p.a2 >= N - (p.w - p.s) + 1);
        count += p.b2 - p.a2 + 1;
    }
    REQUIRE(count <= p.w && count <= p.n_new);
    ++g_launches;
    return hipSuccess;
}

static void check_plan(const DecodeParams &p)
{
    REQUIRE(p.nsplit >= 1 && p.rows_per_split >= kDecodeChunk && p.rows_per_split % kDecodeChunk == 0);
    REQUIRE((long long)p.nsplit * p.rows_per_split >= p.nvalid);
    REQUIRE((long long)(p.nsplit - 1) * p.rows_per_split < p.nvalid || p.nsplit == 1);
    REQUIRE(p.nsplit == 1 || p.part != nullptr);
    REQUIRE(p.pairs_per_wg == 1 || p.pairs_per_wg == 2 || p.pairs_per_wg == 4);
    REQUIRE(p.waves_per_wg == 4 || p.waves_per_wg == 8 || p.waves_per_wg == 16);
    REQUIRE(p.waves_per_wg == 4 || p.pairs_per_wg == 1);
    REQUIRE(p.B >= 1 && p.Hkv >= 1 && p.Hq % p.Hkv == 0 && p.Q && p.O);
}

hipError_t launch_decode(Dt dt, int d, int G, const DecodeParams &p, hipStream_t)
{
    REQUIRE(d == 64 || d == 128);
    REQUIRE(p.Hq == G * p.Hkv);
    REQUIRE(p.nvalid >= 1 && p.nvalid <= p.w && p.Kc && p.Vc);
    REQUIRE((dt == Dt::FP8) == (p.kv_scale != nullptr));
    check_plan(p);
    ++g_launches;
    return hipSuccess;
}

hipError_t launch_decode_step(int d, int G, const DecodeParams &p, hipStream_t st)
{
    REQUIRE(p.Kn && p.Vn && p.new_slot >= 0 && p.new_slot < p.w && p.new_slot < p.nvalid);
    return launch_decode(Dt::BF16, d, G, p, st);
}

hipError_t launch_decode_mq(int d, int G, const DecodeParams &p, hipStream_t)
{
    REQUIRE((d == 64 || d == 128) && p.Hq == G * p.Hkv && p.Kc && p.Vc && p.Q && p.O && p.Kn && p.Vn);
    REQUIRE(p.mq_c >= 1 && p.mq_c * G <= 16 && p.nsplit == 1 && p.pairs_per_wg == 1);
    REQUIRE(p.waves_per_wg == 4 || p.waves_per_wg == 8 || p.waves_per_wg == 16);
    REQUIRE(p.s >= 0 && p.s < p.w && p.n0 >= 0 && p.nvalid == (p.n0 < p.w ? p.n0 : p.w));
    REQUIRE(p.ring_head >= 0 && p.ring_head < p.w - p.s);
    check_plan(p);
    ++g_launches;
    return hipSuccess;
}

hipError_t launch_decode_paged(int d, int G, const DecodeParams &p, hipStream_t)
{
    REQUIRE((d == 64 || d == 128) && p.Hq == G * p.Hkv);
    REQUIRE(p.pg.Kp && p.pg.Vp && p.pg.block_table && p.pg.n);
    REQUIRE(p.pg.page % kDecodeChunk == 0 && p.pg.pages_per_seq * p.pg.page >= p.w);
    check_plan(p);
    ++g_launches;
    return hipSuccess;
}

hipError_t launch_paged_append(Dt dt, int d, const PagedAppendParams &p, hipStream_t)
{
    REQUIRE(dt == Dt::BF16 && (d == 64 || d == 128));
    REQUIRE(p.Kn && p.Vn && p.cu_seqlens && p.total >= 0 && p.c.page % kDecodeChunk == 0);
    ++g_launches;
    return hipSuccess;
}

hipError_t decode_scratch(int device, void **ptr)
{
    REQUIRE(device == 0);
    static unsigned char fake[64] __attribute__((aligned(256)));
    *ptr = fake;  // never dereferenced: launches are stubbed
    return hipSuccess;
}

}  // namespace swa
