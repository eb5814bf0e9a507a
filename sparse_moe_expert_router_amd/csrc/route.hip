// Router and permute kernels (gfx950).
//
// Router: l[e] = x[t] . W_r[e] + b[e] accumulated in fp64 (every fp32 or bf16 by fp32 product is
// exact in fp64), so the selected experts are the exact-arithmetic ones; softmax over the k
// selected logits gives the renormalised top-k weights (equal to softmax over all E followed by
// renormalisation, the order the Inferentia page's router and the layer definition use).
// Top-k: one wavefront per token, k rounds of a wave-wide (logit desc, index asc) arg-max.
//
// Permute: one workgroup builds the expert histogram (LDS atomics, order-free), the exclusive
// prefix sums and a stable scatter of the pairs into (expert, pair id) order, which is the
// gather the mul_mat_id step of the Gemma-on-a-Xeon page ("Three-part fix") needs on a GPU.
#include "moe_common.hpp"
#include "moe_launch.hpp"

namespace moe {

// One wave per expert row; TT tokens per block row.
template <int XT, int TT>
__global__ __launch_bounds__(256) void router_logits_kernel(const void *__restrict__ x, int T, int d,
                                                            const float *__restrict__ Wr,
                                                            const float *__restrict__ bias, int E,
                                                            double *__restrict__ logits)
{
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int e = blockIdx.x * 4 + wave;
    if (e >= E) return;
    const int t0 = blockIdx.y * TT;
    double acc[TT];
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) acc[tt] = 0.0;
    const float4 *wrow = reinterpret_cast<const float4 *>(Wr + (size_t)e * d);
    const int n4 = d >> 2;
    for (int i = lane; i < n4; i += WAVE) {
        const float4 w = wrow[i];
#pragma unroll
        for (int tt = 0; tt < TT; ++tt) {
            const int t = t0 + tt;
            if (t < T) {
                float xv[4];
                if (XT == X_BF16) {
                    const uint2 b = reinterpret_cast<const uint2 *>(
                        reinterpret_cast<const uint16_t *>(x) + (size_t)t * d)[i];
                    xv[0] = __uint_as_float(b.x << 16);
                    xv[1] = __uint_as_float(b.x & 0xFFFF0000u);
                    xv[2] = __uint_as_float(b.y << 16);
                    xv[3] = __uint_as_float(b.y & 0xFFFF0000u);
                } else {
                    const float4 f = reinterpret_cast<const float4 *>(
                        reinterpret_cast<const float *>(x) + (size_t)t * d)[i];
                    xv[0] = f.x; xv[1] = f.y; xv[2] = f.z; xv[3] = f.w;
                }
                acc[tt] = fma((double)w.x, (double)xv[0], acc[tt]);
                acc[tt] = fma((double)w.y, (double)xv[1], acc[tt]);
                acc[tt] = fma((double)w.z, (double)xv[2], acc[tt]);
                acc[tt] = fma((double)w.w, (double)xv[3], acc[tt]);
            }
        }
    }
    const double b = bias ? (double)bias[e] : 0.0;
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) {
        const double s = wave_sum(acc[tt]);
        const int t = t0 + tt;
        if (lane == 0 && t < T) logits[(size_t)t * E + e] = s + b;
    }
}

// Top-k of one token's E (<= 512) logits by one wave.  Lane j < k writes slot j.
__device__ void wave_topk(const double *__restrict__ lrow, int E, int k, int lane,
                          int32_t *__restrict__ idx_out, float *__restrict__ w_out)
{
    constexpr int MAXV = MAX_E / WAVE;
    double v[MAXV];
    uint32_t taken = 0;
#pragma unroll
    for (int i = 0; i < MAXV; ++i) {
        const int e = lane + WAVE * i;
        double l = e < E ? lrow[e] : -INFINITY;
        if (l != l) l = -INFINITY;  // a NaN logit ranks last
        v[i] = l;
        if (e >= E) taken |= 1u << i;
    }
    double my_l = 0.0;
    int my_e = 0;
    for (int j = 0; j < k; ++j) {
        double bv = -INFINITY;
        int bi = 0x7FFFFFFF;
#pragma unroll
        for (int i = 0; i < MAXV; ++i) {
            const int e = lane + WAVE * i;
            if (!((taken >> i) & 1u) && (v[i] > bv || (v[i] == bv && e < bi))) {
                bv = v[i];
                bi = e;
            }
        }
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) {
            const double ov = __shfl_xor(bv, off, WAVE);
            const int oi = __shfl_xor(bi, off, WAVE);
            if (ov > bv || (ov == bv && oi < bi)) {
                bv = ov;
                bi = oi;
            }
        }
        if (bi >= E) bi = E - 1;  // unreachable for k <= E; keeps the id in range regardless
        if ((bi & (WAVE - 1)) == lane) taken |= 1u << (bi >> 6);
        if (lane == j) {
            my_l = bv;
            my_e = bi;
        }
    }
    const double l0 = __shfl(my_l, 0, WAVE);
    const double ex = lane < k ? exp(my_l - l0) : 0.0;
    const double z = wave_sum(ex);
    if (lane < k) {
        idx_out[lane] = my_e;
        w_out[lane] = (float)(ex / z);
    }
}

__global__ __launch_bounds__(256) void topk_kernel(const double *__restrict__ logits, int T, int E,
                                                   int k, int32_t *__restrict__ topk_idx,
                                                   float *__restrict__ topk_w)
{
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= T) return;
    wave_topk(logits + (size_t)t * E, E, k, threadIdx.x & 63, topk_idx + (size_t)t * k,
              topk_w + (size_t)t * k);
}

// Block-wide exclusive scan of one int per thread (blockDim = 1024).  `tmp` holds 16 ints.
__device__ __forceinline__ int block_excl_scan(int v, int *tmp, int *total)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int incl = v;
#pragma unroll
    for (int off = 1; off < WAVE; off <<= 1) {
        const int o = __shfl_up(incl, off, WAVE);
        if (lane >= off) incl += o;
    }
    if (lane == WAVE - 1) tmp[wave] = incl;
    __syncthreads();
    int pre = 0, tot = 0;
    for (int w = 0; w < 16; ++w) {
        const int s = tmp[w];
        pre += w < wave ? s : 0;
        tot += s;
    }
    __syncthreads();
    *total = tot;
    return pre + incl - v;
}

// Optionally selects the top-k of every token (DO_TOPK, T small), then permutes the P = T*k
// pairs.  One workgroup of 1024 threads.
template <bool DO_TOPK>
__global__ __launch_bounds__(1024) void select_permute_kernel(
    const double *__restrict__ logits, const int32_t *idx_in, int T, int k, int E,
    int32_t *topk_idx, float *__restrict__ topk_w, int32_t *__restrict__ counts,
    int32_t *__restrict__ offsets, int32_t *__restrict__ perm, int32_t *__restrict__ inv,
    int32_t *__restrict__ active, int32_t *__restrict__ n_active, int32_t *__restrict__ tile_off,
    int BM)
{
    __shared__ int s_cnt[MAX_E];
    __shared__ int s_next[MAX_E];
    __shared__ int s_wcnt[16][MAX_E];
    __shared__ int s_tmp[16];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int P = T * k;

    if (DO_TOPK) {
        for (int t = wave; t < T; t += 16)
            wave_topk(logits + (size_t)t * E, E, k, lane, topk_idx + (size_t)t * k,
                      topk_w + (size_t)t * k);
        __threadfence_block();
    }
    const int32_t *idx = DO_TOPK ? topk_idx : idx_in;

    for (int i = tid; i < MAX_E; i += 1024) s_cnt[i] = 0;
    for (int i = tid; i < 16 * MAX_E; i += 1024) (&s_wcnt[0][0])[i] = 0;
    __syncthreads();
    for (int p = tid; p < P; p += 1024) atomicAdd(&s_cnt[clamp_id(idx[p], E)], 1);
    __syncthreads();

    // exclusive scans over experts: pair offsets, active-expert slots, prefill row tiles
    const int c = tid < E ? s_cnt[tid] : 0;
    int tot_c, tot_a, tot_t;
    const int off_c = block_excl_scan(c, s_tmp, &tot_c);
    const int off_a = block_excl_scan(c > 0 ? 1 : 0, s_tmp, &tot_a);
    const int tiles = BM > 0 ? (c + BM - 1) / BM : 0;
    const int off_t = block_excl_scan(tiles, s_tmp, &tot_t);
    if (tid < E) {
        counts[tid] = c;
        offsets[tid] = off_c;
        s_next[tid] = off_c;
        if (c > 0 && active) active[off_a] = tid;
        if (tile_off) tile_off[tid] = off_t;
    }
    if (tid == 0) {
        offsets[E] = tot_c;
        if (n_active) *n_active = tot_a;
        if (tile_off) tile_off[E] = tot_t;
    }
    __syncthreads();

    // stable scatter, 1024 pairs per round
    for (int base = 0; base < P; base += 1024) {
        const int p = base + tid;
        const bool valid = p < P;
        const int e = valid ? clamp_id(idx[p], E) : 0;
        uint64_t m = __ballot(valid);
#pragma unroll
        for (int bit = 0; bit < MAX_E_BITS; ++bit) {
            const bool b = (e >> bit) & 1;
            const uint64_t bal = __ballot(valid && b);
            m &= b ? bal : ~bal;
        }
        const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
        const int rank = __popcll(m & lt);
        if (valid && rank == 0) s_wcnt[wave][e] = __popcll(m);
        __syncthreads();
        if (valid) {
            int pre = 0;
            for (int w = 0; w < wave; ++w) pre += s_wcnt[w][e];
            const int pos = s_next[e] + pre + rank;
            perm[pos] = p;
            inv[p] = pos;
        }
        __syncthreads();
        if (tid < E) {
            int tot = 0;
            for (int w = 0; w < 16; ++w) tot += s_wcnt[w][tid];
            s_next[tid] += tot;
        }
        __syncthreads();
        if (valid && rank == 0) s_wcnt[wave][e] = 0;
        __syncthreads();
    }
}

// ------------------------------------------------------------------------------------------
// Host launchers
// ------------------------------------------------------------------------------------------

hipError_t launch_router_logits(const void *x, int xtype, int T, int d, const float *Wr,
                                const float *bias, int E, double *logits, hipStream_t s)
{
    constexpr int TT = 8;
    dim3 grid((E + 3) / 4, (T + TT - 1) / TT);
    ProfScope ps(K_ROUTER, s);
    if (xtype == X_BF16)
        hipLaunchKernelGGL((router_logits_kernel<X_BF16, TT>), grid, dim3(256), 0, s, x, T, d, Wr,
                           bias, E, logits);
    else
        hipLaunchKernelGGL((router_logits_kernel<X_F32, TT>), grid, dim3(256), 0, s, x, T, d, Wr,
                           bias, E, logits);
    return hipGetLastError();
}

hipError_t launch_topk(const double *logits, int T, int E, int k, int32_t *idx, float *w,
                       hipStream_t s)
{
    ProfScope ps(K_TOPK, s);
    hipLaunchKernelGGL(topk_kernel, dim3((T + 3) / 4), dim3(256), 0, s, logits, T, E, k, idx, w);
    return hipGetLastError();
}

hipError_t launch_select_permute(const double *logits, const int32_t *idx_in, int T, int k, int E,
                                 int32_t *topk_idx, float *topk_w, const PermuteOut &po, int BM,
                                 hipStream_t s)
{
    ProfScope ps(K_PERMUTE, s);
    if (logits)
        hipLaunchKernelGGL((select_permute_kernel<true>), dim3(1), dim3(1024), 0, s, logits,
                           nullptr, T, k, E, topk_idx, topk_w, po.counts, po.offsets, po.perm,
                           po.inv, po.active, po.n_active, po.tile_off, BM);
    else
        hipLaunchKernelGGL((select_permute_kernel<false>), dim3(1), dim3(1024), 0, s, nullptr,
                           idx_in, T, k, E, nullptr, nullptr, po.counts, po.offsets, po.perm,
                           po.inv, po.active, po.n_active, po.tile_off, BM);
    return hipGetLastError();
}

}  // namespace moe
