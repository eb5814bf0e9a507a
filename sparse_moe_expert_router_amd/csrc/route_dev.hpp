// Device helpers of the top-k selection, shared by the router kernels and the expert kernels that
// select a small batch's experts themselves.
#pragma once
#include "moe_common.hpp"

namespace moe {

// Ordered 64-bit key of a logit: a larger logit has a larger key, NaN ranks with -inf, and 0 is
// below every logit (the key of an empty or already selected slot).
__device__ __forceinline__ uint64_t logit_key(double l)
{
    if (l != l) l = -INFINITY;
    if (l == 0.0) l = 0.0;                        // -0 and +0 are the same logit
    const uint64_t b = __builtin_bit_cast(uint64_t, l);
    return (b >> 63) ? ~b : (b | 0x8000000000000000ull);
}

__device__ __forceinline__ double key_logit(uint64_t k)
{
    return __builtin_bit_cast(double, (k >> 63) ? (k & 0x7FFFFFFFFFFFFFFFull) : ~k);
}

// Top-k of one token's E <= 64 * MAXV logits by one whole wave (every lane active).  Lane l holds
// experts l + 64 i.  Each of the k rounds finds the wave maximum of the lanes' best remaining
// keys in 32-bit steps (DPP / permlane butterflies, no LDS): the high words first, then the low
// words among the lanes that tie on them, then the lowest expert index among exact ties.  Only
// the winning lane retires that slot and rescans its own.  Lane j < k writes slot j (softmax over
// the k selected logits = the renormalised top-k weights) and returns its expert id.
template <int MAXV>
__device__ int wave_topk(const double *__restrict__ lrow, int E, int k, int lane,
                         int32_t *__restrict__ idx_out, float *__restrict__ w_out)
{
    uint64_t key[MAXV];
#pragma unroll
    for (int i = 0; i < MAXV; ++i) {                // unconditional loads: one round trip
        const int e = lane + WAVE * i;
        const uint64_t kv = logit_key(lrow[min(e, E - 1)]);
        key[i] = e < E ? kv : 0ull;
    }
    auto best = [&](uint64_t &bk, int &bs) {       // first slot holding the lane's largest key
        bk = key[0];
        bs = 0;
#pragma unroll
        for (int i = 1; i < MAXV; ++i)
            if (key[i] > bk) {
                bk = key[i];
                bs = i;
            }
    };
    uint64_t bk;
    int bs;
    best(bk, bs);
    uint64_t my_key = 0ull, key0 = 0ull;
    int my_e = 0;
    for (int j = 0; j < k; ++j) {
        const uint32_t hi = (uint32_t)(bk >> 32), lo = (uint32_t)bk;
        const uint32_t mhi = wave_max_u32(hi);
        uint64_t hit = __ballot(hi == mhi);
        if (__popcll(hit) > 1) {                   // several lanes share the high word
            const uint32_t mlo = wave_max_u32(hi == mhi ? lo : 0u);
            hit = __ballot(hi == mhi && lo == mlo);
        }
        int win;
        if (__popcll(hit) == 1) {
            win = __ffsll((unsigned long long)hit) - 1;
        } else {                                   // equal logits: the lowest expert index
            const bool tied = ((hit >> lane) & 1ull) != 0ull;
            const uint32_t m = ~wave_max_u32(tied ? ~(uint32_t)(lane + WAVE * bs) : 0u);
            win = __builtin_amdgcn_readfirstlane((int)(m & (WAVE - 1)));
        }
        const int we = min(__builtin_amdgcn_readlane(lane + WAVE * bs, win), E - 1);
        const uint64_t km = (uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)lo, win) |
                            ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)hi, win) << 32);
        if (j == 0) key0 = km;
        if (lane == j) {
            my_key = km;
            my_e = we;
        }
        if (lane == win) {
#pragma unroll
            for (int i = 0; i < MAXV; ++i)
                if (i == bs) key[i] = 0ull;
            best(bk, bs);
        }
    }
    const double l0 = key_logit(key0);
    const double ex = lane < k ? exp(key_logit(my_key) - l0) : 0.0;
    const double z = wave_sum_f64(ex);
    if (lane < k) {
        idx_out[lane] = my_e;
        w_out[lane] = (float)(ex / z);
    }
    return my_e;
}

}  // namespace moe
