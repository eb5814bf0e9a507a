// Device helpers of the top-k selection, shared by the router kernels and the expert kernels that
// select a small batch's experts themselves.
#pragma once
#include "moe_common.hpp"
#include "moe_launch.hpp"

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

// Sort of 64 (key, expert) pairs across a wave (bitonic network, xor partners by DPP and the
// permlane swaps): lane l ends with the l-th best, best = larger key, then lower expert.  Every
// lane active.
__device__ __forceinline__ void wave_sort_desc(uint64_t &key, int &idx, int lane)
{
#pragma unroll
    for (int size = 2; size <= WAVE; size <<= 1) {
#pragma unroll
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            const uint32_t ohi = xor_lane_u32((uint32_t)(key >> 32), stride, lane);
            const uint32_t olo = xor_lane_u32((uint32_t)key, stride, lane);
            const int oi = (int)xor_lane_u32((uint32_t)idx, stride, lane);
            const uint64_t ok = ((uint64_t)ohi << 32) | olo;
            const bool mine_better = (key > ok) | ((key == ok) & (idx < oi));
            // the lower lane of a pair keeps the better one in a descending block (size bit 0)
            const bool keep = (((lane & stride) == 0) == ((lane & size) == 0)) ? mine_better : !mine_better;
            key = keep ? key : ok;
            idx = keep ? idx : oi;
        }
    }
}

// Bitonic merge of a bitonic sequence of 64 (key, expert) pairs into descending order.
__device__ __forceinline__ void wave_merge_desc(uint64_t &key, int &idx, int lane)
{
#pragma unroll
    for (int stride = WAVE >> 1; stride > 0; stride >>= 1) {
        const uint32_t ohi = xor_lane_u32((uint32_t)(key >> 32), stride, lane);
        const uint32_t olo = xor_lane_u32((uint32_t)key, stride, lane);
        const int oi = (int)xor_lane_u32((uint32_t)idx, stride, lane);
        const uint64_t ok = ((uint64_t)ohi << 32) | olo;
        const bool mine_better = (key > ok) | ((key == ok) & (idx < oi));
        const bool keep = ((lane & stride) == 0) ? mine_better : !mine_better;
        key = keep ? key : ok;
        idx = keep ? idx : oi;
    }
}

// a beats b: larger key, or the same key and a lower expert index
__device__ __forceinline__ bool key_beats(uint64_t ka, int ia, uint64_t kb, int ib)
{
    return (ka > kb) | ((ka == kb) & (ia < ib));      // no short circuit: no branch
}


// Top-k of the T tokens for more than 128 experts (MAXV = 4 or 8 keys per lane of a 64-wide share):
// MAXV waves per token each sort 64 of the logits' keys, then the sorted lists are merged pairwise:
// the better of entry i of one list and entry 63 - i of the other, over i < 64, is the best 64 of
// the two (a bitonic sequence), which a bitonic merge sorts.  After log2(MAXV) rounds lane j of the
// token's first wave holds its rank-j expert.  A workgroup of NWV >= MAXV waves takes NWV / MAXV
// tokens per pass; every thread of the workgroup calls it (it holds block barriers).  Writes the
// ids and weights to topk_idx / topk_w (global or LDS) and the ids to s_idx[t k + j]; s_cand holds
// NWV * 64 entries.
template <int MAXV, int NWV = 16>
__device__ void topk_sorted(const double *__restrict__ logits, int T, int k, int E, int wave, int lane,
                            int32_t *topk_idx, float *topk_w, int *s_idx, uint4 *s_cand)
{
    static_assert(NWV >= MAXV && NWV % MAXV == 0, "a token's lists need MAXV waves of the workgroup");
    constexpr int TP = NWV / MAXV;                 // tokens per pass
    const int tp = wave / MAXV, part = wave - tp * MAXV;
    for (int t0 = 0; t0 < T; t0 += TP) {
        const int t = t0 + tp;                     // wave-uniform
        const double *lrow = logits + (size_t)min(t, T - 1) * E;
        const int e = part * WAVE + lane;
        uint64_t key = logit_key(lrow[min(e, E - 1)]);
        if (e >= E) key = 0ull;
        int idx = e;
        if (t < T) wave_sort_desc(key, idx, lane);  // (waves past the last token idle: they
                                                   // share the SIMDs with the working ones)
#pragma unroll
        for (int half = 1; half < MAXV; half <<= 1) {
            s_cand[wave * WAVE + lane] = make_uint4((uint32_t)key, (uint32_t)(key >> 32), (uint32_t)idx, 0u);
            __syncthreads();
            if (t < T && (part & (2 * half - 1)) == 0) {
                const uint4 o = s_cand[(wave + half) * WAVE + (WAVE - 1 - lane)];
                const uint64_t ok = (uint64_t)o.x | ((uint64_t)o.y << 32);
                const bool mine = key_beats(key, idx, ok, (int)o.z);
                key = mine ? key : ok;
                idx = mine ? idx : (int)o.z;
                wave_merge_desc(key, idx, lane);
            }
            __syncthreads();
        }
        if (t < T && part == 0) {                  // softmax over the k best, as wave_topk
            const uint32_t k0lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)key);
            const uint32_t k0hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(key >> 32));
            const double l0 = key_logit((uint64_t)k0lo | ((uint64_t)k0hi << 32));
            const double ex = lane < k ? exp(key_logit(key) - l0) : 0.0;
            const double z = wave_sum_f64(ex);
            if (lane < k) {
                const int sel = min(idx, E - 1);   // (always < E)
                topk_idx[(size_t)t * k + lane] = sel;
                topk_w[(size_t)t * k + lane] = (float)(ex / z);
                s_idx[t * k + lane] = sel;
            }
        }
    }
}


// In-block routing for small batches (T <= 2, T k <= 64, E <= MAX_E), so that the layer needs no
// separate selection and permute step: every expert block selects the top-k of all T tokens from
// the fp64 logits itself (E <= 128: one wave per token, wave_topk; more experts: the sorted lists
// of topk_sorted over the block's NWV waves; the same selection and weights as the router's
// top-k), counts the pairs per expert in LDS, and takes slot s = the s-th selected expert in
// ascending id (then the shared experts), its first permuted row (the pairs of lower experts) and
// its pairs in pair order, exactly the records and orders the permute step writes.  The blocks
// with `writer` set (one per slot) write their slot's record and the perm / inv entries of its
// pairs, slot 0's also the active count and the top-k ids and weights, for the down projection
// and the combine that run afterwards.  Every block repeats the T selections, so this pays while
// T is small: Gemma-shaped decode, tokens/s with it / with the separate small-batch select
// kernel, T = 1 39.0k / 36.6k, T = 2 56.4k / 53.5k, T = 3 63.5k / 64.6k, T = 4 75.3k / 75.9k,
// T = 5 80.6k / 84.5k.  Every thread of the block calls it (it holds block barriers).
struct RouteSlot {
    int e, row0, n_e, tok;                         // e < 0: no expert in this slot
};

template <int NWV>
__device__ RouteSlot route_slot_any(const RouteIn &ri, int T, int k, int slot, bool writer, int li)
{
    static_assert(NWV >= 8, "the sorted selection over 512 experts takes eight waves per token");
    constexpr int PER = MAX_E / WAVE;              // experts per lane in the scans
    static_assert(PER == 8, "the count reads below take 8 experts per lane");
    __shared__ int r_idx[64];
    __shared__ float r_w[64];
    __shared__ __attribute__((aligned(16))) int r_cnt[MAX_E];
    __shared__ int r_info[4];
    __shared__ int r_pair[SLOT_TOKS];
    __shared__ uint4 r_cand[NWV * WAVE];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int E = ri.E, P = T * k;
    for (int i = tid; i < MAX_E; i += NWV * WAVE) r_cnt[i] = 0;
    if (E <= 128) {
        if (wave < T) wave_topk<2>(ri.logits + (size_t)wave * E, E, k, lane, r_idx + wave * k, r_w + wave * k);
    } else if (E <= 256) {
        topk_sorted<4, NWV>(ri.logits, T, k, E, wave, lane, r_idx, r_w, r_idx, r_cand);
    } else {
        topk_sorted<8, NWV>(ri.logits, T, k, E, wave, lane, r_idx, r_w, r_idx, r_cand);
    }
    __syncthreads();
    if (T == 1) {
        // one token: every selected expert holds one pair, so slot s < k is the selected expert
        // of rank s by id, at permuted row s, holding the pair of its position in the top-k list;
        // slots k .. k + S - 1 are the shared experts (rows k ..)
        if (wave == 0) {
            const int id = r_idx[min(lane, k - 1)];
            int below = 0;                           // selected experts with a lower id
            for (int i = 0; i < k; ++i) below += __builtin_amdgcn_readlane(id, i) < id;
            const bool mine = lane < k && below == slot;
            const uint64_t b = __ballot(mine);
            if (lane == 0) {
                int e = -1;
                if (slot < k) e = __builtin_amdgcn_readlane(id, b ? __ffsll((unsigned long long)b) - 1 : 0);
                else if (slot < k + ri.S) e = E + (slot - k);
                r_info[0] = e;
                r_info[1] = slot;
                r_info[2] = 1;
                r_info[3] = k + ri.S;
                r_pair[0] = slot < k ? (b ? __ffsll((unsigned long long)b) - 1 : 0) : 0;
            }
        }
        __syncthreads();
    } else {
    if (tid < P) atomicAdd(&r_cnt[r_idx[tid]], 1);   // (order-free)
    __syncthreads();
    if (wave == 0) {
        // lane owns experts PER lane .. PER lane + PER - 1: scans of the active flags and counts
        int c[PER], la = 0, lc = 0;
        const int4 c0 = reinterpret_cast<const int4 *>(r_cnt)[2 * lane];
        const int4 c1 = reinterpret_cast<const int4 *>(r_cnt)[2 * lane + 1];
        c[0] = c0.x; c[1] = c0.y; c[2] = c0.z; c[3] = c0.w;
        c[4] = c1.x; c[5] = c1.y; c[6] = c1.z; c[7] = c1.w;
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            la += c[i] > 0;
            lc += c[i];
        }
        int ia = la, ic = lc;
#pragma unroll
        for (int off = 1; off < WAVE; off <<= 1) {
            const int oa = __shfl_up(ia, off, WAVE), oc = __shfl_up(ic, off, WAVE);
            if (lane >= off) {
                ia += oa;
                ic += oc;
            }
        }
        const int nact = __shfl(ia, WAVE - 1, WAVE);
        const int pa = ia - la, pc = ic - lc;
        int e = -1, row0 = 0, n_e = 0;
        if (slot < nact) {                           // exactly one lane holds the slot's expert
            const bool mine = pa <= slot && slot < pa + la;
            int me = 0, mr = 0, mn = 0, a = pa, r = pc;
#pragma unroll
            for (int i = 0; i < PER; ++i) {
                const bool hit = c[i] > 0 && a == slot;
                me = hit ? lane * PER + i : me;
                mr = hit ? r : mr;
                mn = hit ? c[i] : mn;
                a += c[i] > 0;
                r += c[i];
            }
            const int src = __ffsll((unsigned long long)__ballot(mine)) - 1;
            e = __shfl(me, src, WAVE);
            row0 = __shfl(mr, src, WAVE);
            n_e = __shfl(mn, src, WAVE);
        } else if (slot < nact + ri.S) {             // shared expert: rows P + sh T + t hold pair t k
            e = E + (slot - nact);
            row0 = P + (slot - nact) * T;
            n_e = T;
        }
        if (e >= 0 && e < E) {
            const bool hit = lane < P && r_idx[min(lane, P - 1)] == e;
            const uint64_t b = __ballot(hit);
            const int m = __popcll(b & ((1ull << lane) - 1ull));
            if (hit) r_pair[m] = lane;
        } else if (e >= E && lane < T) {
            r_pair[lane] = lane * k;
        }
        if (lane == 0) {
            r_info[0] = e;
            r_info[1] = row0;
            r_info[2] = n_e;
            r_info[3] = nact + ri.S;
        }
    }
    __syncthreads();
    }
    RouteSlot rs;
    rs.e = r_info[0];
    rs.row0 = r_info[1];
    rs.n_e = r_info[2];
    rs.tok = li < rs.n_e ? r_pair[min(li, SLOT_TOKS - 1)] / k : 0;
    if (writer && rs.e >= 0) {
        if (tid == 0) ri.slots[(size_t)slot * SLOT_INT4] = make_int4(rs.e, rs.row0, rs.n_e, 0);
        if (tid < SLOT_TOKS)
            reinterpret_cast<int *>(ri.slots + (size_t)slot * SLOT_INT4)[4 + tid] = tid < rs.n_e ? r_pair[tid] / k : 0;
        if (tid < rs.n_e) {
            ri.perm[rs.row0 + tid] = r_pair[tid];
            if (rs.e < E) ri.inv[r_pair[tid]] = rs.row0 + tid;
        }
        if (slot == 0) {
            if (tid == 0) *ri.n_active = r_info[3];
            if (tid < P) {
                ri.topk_idx[tid] = r_idx[tid];
                ri.topk_w[tid] = r_w[tid];
            }
        }
    }
    return rs;
}

}  // namespace moe
