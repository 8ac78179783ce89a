// Host-side decode planning: how the cache rows of each (batch, kv-head)
// are split over waves and workgroups.  Plain C++ (no device code), so the
// C ABI's host logic can also be built and sanitised without the GPU
// toolchain.
#include "swa_internal.h"

namespace swa {

void decode_plan(int B, int Hkv, int nvalid, int *nsplit, int *rows_per_split, int *max_splits,
                 int *pairs_per_wg, int *waves_per_wg, bool allow16)
{
    // Aim for about 2048 waves in flight (8 per CU), one 32-row chunk per
    // wave at least.  A task is one (b, kv-head, split); 1, 2 or 4 waves share
    // a task, and a workgroup of 4 waves holds 4, 2 or 1 tasks; between 4 and
    // 8 wanted waves per pair (or more, see below), one task takes a whole
    // 8-wave workgroup.
    // Splits across workgroups (with a merge pass) only when one workgroup per
    // (b, kv-head) would leave the GPU mostly idle.
    const long long pairs = (long long)B * Hkv;
    const long long chunks = (nvalid + kDecodeChunk - 1) / kDecodeChunk;
    long long want = (2048 + pairs - 1) / pairs;
    if (want > chunks) want = chunks;
    if (want < 1) want = 1;
    int ns = 1, P, NW = 4;
    if (want <= 1) P = 4;
    else if (want <= 2) P = 2;
    else {
        P = 1;
        // With 64 or more pairs, up to 16 chunks go to one 8-wave workgroup
        // (two per wave) rather than to splits and a merge pass (batch 16 at
        // SWA(512,4): 12.8 against 13.8 us per fused step); fewer pairs keep
        // the splits, which fill more of the GPU.
        // With fewer pairs and at most 16 chunks each (a window of up to 512
        // rows at batch 1 to 7 with 8 kv-heads), one 16-wave workgroup per
        // pair, a chunk per wave, meeting in LDS: no split and no second
        // launch for the merge, which costs more than it saves on so little
        // data (allow16: not for fp8 caches, whose kernel needs more
        // registers than 16-wave workgroups leave).
        if (want > 8 && chunks <= 16 && pairs < 64 && allow16) NW = 16;
        else if (want > 8 && !(chunks <= 16 && pairs >= 64)) ns = (int)((want + 3) / 4);
        else if (want > 4) NW = 8;
    }
    *waves_per_wg = NW;
    *max_splits = ns;  // non-decreasing in nvalid, and >= the rounded count below
    int rps = (nvalid + ns - 1) / ns;
    rps = (rps + kDecodeChunk - 1) / kDecodeChunk * kDecodeChunk;
    if (rps < kDecodeChunk) rps = kDecodeChunk;
    ns = (nvalid + rps - 1) / rps;
    if (ns < 1) ns = 1;
    *nsplit = ns;
    *rows_per_split = rps;
    *pairs_per_wg = P;
}

}  // namespace swa
