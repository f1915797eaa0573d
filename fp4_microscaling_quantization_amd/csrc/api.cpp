// Version, status strings and host helpers of the libmxq C ABI.
#include <math.h>

#include "mxq.h"

extern "C" const char *mxq_status_string(mxq_status s)
{
    switch (s) {
    case MXQ_OK: return "ok";
    case MXQ_ERR_NULL: return "a required pointer is NULL";
    case MXQ_ERR_SHAPE: return "invalid size (negative, or not a multiple of 32 along the block axis)";
    case MXQ_ERR_ALIGN: return "misaligned pointer or leading dimension";
    case MXQ_ERR_UNSUPPORTED: return "unsupported option or combination";
    case MXQ_ERR_DEVICE: return "HIP launch failed";
    case MXQ_ERR_WORKSPACE: return "workspace missing or too small";
    default: return "unknown status";
    }
}

extern "C" int32_t mxq_abi_version(void) { return MXQ_ABI_VERSION; }

// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As Easy
// as 1, 2, 3", SC'11): ten rounds of two 32x32->64-bit products, the high
// halves xored into the other words with the round key, the key bumped by
// the two Weyl constants after each round.
static void philox_host(uint32_t ctr[4], uint32_t k0, uint32_t k1)
{
    for (int r = 0; r < 10; ++r) {
        const uint64_t p0 = (uint64_t)0xD2511F53u * ctr[0];
        const uint64_t p1 = (uint64_t)0xCD9E8D57u * ctr[2];
        const uint32_t n0 = (uint32_t)(p1 >> 32) ^ ctr[1] ^ k0;
        const uint32_t n2 = (uint32_t)(p0 >> 32) ^ ctr[3] ^ k1;
        ctr[1] = (uint32_t)p1;
        ctr[3] = (uint32_t)p0;
        ctr[0] = n0;
        ctr[2] = n2;
        k0 += 0x9E3779B9u;
        k1 += 0xBB67AE85u;
    }
}

extern "C" uint32_t mxq_rht_sign_mask(uint64_t seed, uint32_t n)
{
    if (n != 16 && n != 32)
        return 0;
    uint32_t ctr[4] = {0u, 0xFFFFFFFFu, 0xFFFFFFFFu, 0xFFFFFFFFu};
    philox_host(ctr, (uint32_t)seed, (uint32_t)(seed >> 32));
    return n == 32 ? ctr[0] : (ctr[0] & 0xFFFFu);
}

// Effective bucket ratio exp(H) / L of a tensor's magnitude-code histogram
// (H its entropy in nats, L the number of levels the grid emits).
extern "C" double mxq_bucket_ratio(const mxq_stats *stats, int32_t grid)
{
    const int L = (grid == MXQ_GRID_E2M1 || grid == MXQ_GRID_E1M2) ? 8
                  : grid == MXQ_GRID_E2M1_MAX4                     ? 7
                  : grid == MXQ_GRID_E2M1_MAX3                     ? 6
                                                                   : 0;
    if (!stats || L == 0)
        return NAN;
    double n = 0.0;
    for (int m = 0; m < L; ++m)
        n += (double)stats->level_count[m];
    if (!(n > 0.0))
        return NAN;
    double h = 0.0;
    for (int m = 0; m < L; ++m) {
        if (stats->level_count[m] == 0)
            continue;
        const double p = (double)stats->level_count[m] / n;
        h -= p * log(p);
    }
    return exp(h) / L;
}
