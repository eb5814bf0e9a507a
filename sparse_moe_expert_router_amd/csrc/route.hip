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

template <int XT>
__device__ __forceinline__ void load_x4(const void *__restrict__ x, size_t off, float *xv)
{
    if (XT == X_BF16) {
        const uint2 b = *reinterpret_cast<const uint2 *>(reinterpret_cast<const uint16_t *>(x) + off);
        xv[0] = __uint_as_float(b.x << 16);
        xv[1] = __uint_as_float(b.x & 0xFFFF0000u);
        xv[2] = __uint_as_float(b.y << 16);
        xv[3] = __uint_as_float(b.y & 0xFFFF0000u);
    } else {
        const float4 f = *reinterpret_cast<const float4 *>(reinterpret_cast<const float *>(x) + off);
        xv[0] = f.x; xv[1] = f.y; xv[2] = f.z; xv[3] = f.w;
    }
}

// Decode router: one block (4 waves) per expert row e and group of TT tokens; the 256 threads
// split the row in 8-float chunks, issue all their loads before the fp64 FMAs, and reduce in a
// fixed order (a tree over the 256 partial sums in LDS).
template <int XT, int TT, int UN>
__global__ __launch_bounds__(256) void router_logits_kernel(const void *__restrict__ x, int T, int d,
                                                            const float *__restrict__ Wr,
                                                            const float *__restrict__ bias, int E,
                                                            double *__restrict__ logits)
{
    __shared__ double red[TT][256];
    const int e = blockIdx.x;
    const int t0 = blockIdx.y * TT;
    const int tid = threadIdx.x;
    const int n8 = d >> 3;
    const int nt = min(TT, T - t0);
    double acc[TT];
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) acc[tt] = 0.0;
    const float4 *wrow = reinterpret_cast<const float4 *>(Wr + (size_t)e * d);
    for (int c0 = tid; c0 < n8; c0 += 256 * UN) {
        float4 w[UN][2];
        float xv[UN][TT][8];
#pragma unroll
        for (int u = 0; u < UN; ++u) {
            const int c = c0 + 256 * u;
            const bool in = c < n8;
            w[u][0] = in ? wrow[2 * c] : make_float4(0.f, 0.f, 0.f, 0.f);
            w[u][1] = in ? wrow[2 * c + 1] : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
            for (int tt = 0; tt < TT; ++tt) {
                if (in && tt < nt) {
                    load_x4<XT>(x, (size_t)(t0 + tt) * d + 8 * (size_t)c, xv[u][tt]);
                    load_x4<XT>(x, (size_t)(t0 + tt) * d + 8 * (size_t)c + 4, xv[u][tt] + 4);
                } else {
#pragma unroll
                    for (int i = 0; i < 8; ++i) xv[u][tt][i] = 0.f;
                }
            }
        }
#pragma unroll
        for (int u = 0; u < UN; ++u)
#pragma unroll
            for (int tt = 0; tt < TT; ++tt) {
                const float wv[8] = {w[u][0].x, w[u][0].y, w[u][0].z, w[u][0].w,
                                     w[u][1].x, w[u][1].y, w[u][1].z, w[u][1].w};
#pragma unroll
                for (int i = 0; i < 8; ++i) acc[tt] = fma((double)wv[i], (double)xv[u][tt][i], acc[tt]);
            }
    }
    // fixed-order reduction of the 256 partial sums of each live token, through LDS
    for (int tt = 0; tt < nt; ++tt) red[tt][tid] = acc[tt];
    __syncthreads();
    for (int half = 128; half >= 1; half >>= 1) {
        if (tid < half)
            for (int tt = 0; tt < nt; ++tt) red[tt][tid] += red[tt][tid + half];
        __syncthreads();
    }
    if (tid < nt) logits[(size_t)(t0 + tid) * E + e] = red[tid][0] + (bias ? (double)bias[e] : 0.0);
}

// Batched router on the fp64 matrix cores: block = 32 tokens x 32 experts, 4 waves as 2 x 2
// tiles of 16 x 16, v_mfma_f64_16x16x4_f64 over K chunks of 64 staged in LDS as fp64 (bf16 / fp32
// inputs convert exactly).  Every product is exact and the sums are fp64, as in the decode router.
typedef __attribute__((__vector_size__(4 * sizeof(double)))) double f64x4;
constexpr int RB = 32, RKC = 64;

template <int XT>
__global__ __launch_bounds__(256) void router_logits_mfma_kernel(const void *__restrict__ x, int T, int d,
                                                                 const float *__restrict__ Wr,
                                                                 const float *__restrict__ bias, int E,
                                                                 double *__restrict__ logits)
{
    __shared__ double xs[RB][RKC + 1];
    __shared__ double wsm[RB][RKC + 1];
    const int t0 = blockIdx.x * RB, e0 = blockIdx.y * RB;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int wt = wave >> 1, we = wave & 1;
    const int li = lane & 15, lg = lane >> 4;
    // loader: thread covers row lr = tid / 8, columns 8 * (tid % 8) .. +7 of the 32 x 64 chunk
    const int lr = tid >> 3, lc = (tid & 7) * 8;
    const bool xrow_ok = t0 + lr < T, wrow_ok = e0 + lr < E;
    f64x4 acc = {0.0, 0.0, 0.0, 0.0};
    float xv[8], wv[8];
    auto gload = [&](int k0) {
        if (xrow_ok) {
            load_x4<XT>(x, (size_t)(t0 + lr) * d + k0 + lc, xv);
            load_x4<XT>(x, (size_t)(t0 + lr) * d + k0 + lc + 4, xv + 4);
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) xv[i] = 0.f;
        }
        if (wrow_ok) {
            const float4 a = *reinterpret_cast<const float4 *>(Wr + (size_t)(e0 + lr) * d + k0 + lc);
            const float4 b = *reinterpret_cast<const float4 *>(Wr + (size_t)(e0 + lr) * d + k0 + lc + 4);
            wv[0] = a.x; wv[1] = a.y; wv[2] = a.z; wv[3] = a.w; wv[4] = b.x; wv[5] = b.y; wv[6] = b.z; wv[7] = b.w;
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) wv[i] = 0.f;
        }
    };
    gload(0);
    for (int k0 = 0; k0 < d; k0 += RKC) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            xs[lr][lc + i] = (double)xv[i];
            wsm[lr][lc + i] = (double)wv[i];
        }
        __syncthreads();
        if (k0 + RKC < d) gload(k0 + RKC);
#pragma unroll
        for (int kk = 0; kk < RKC; kk += 4)
            acc = __builtin_amdgcn_mfma_f64_16x16x4f64(xs[wt * 16 + li][kk + lg], wsm[we * 16 + li][kk + lg],
                                                       acc, 0, 0, 0);
        __syncthreads();
    }
    // the f64 16x16x4 result layout: lane holds C[token lg + 4*i][expert li] of its tile (unlike
    // the fp32 / int32 16x16 shapes, whose register i holds row 4*lg + i)
    const int e = e0 + we * 16 + li;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int t = t0 + wt * 16 + lg + 4 * i;
        if (t < T && e < E) logits[(size_t)t * E + e] = acc[i] + (bias ? (double)bias[e] : 0.0);
    }
}

// Top-k of one token's E (<= 512) logits by one wave.  Lane j < k writes slot j and returns its
// expert id.
__device__ int wave_topk(const double *__restrict__ lrow, int E, int k, int lane,
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
    return my_e;
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

constexpr int SMALL_P = 256;   // up to this many pairs a pair's rank is counted directly

// Optionally selects the top-k of every token (DO_TOPK, T small), then permutes the P = T*k
// pairs.  One workgroup of 1024 threads; one wave does the prefix sums over the experts.
template <bool DO_TOPK>
__global__ __launch_bounds__(1024) void select_permute_kernel(
    const double *__restrict__ logits, const int32_t *idx_in, int T, int k, int E,
    int32_t *topk_idx, float *__restrict__ topk_w, int32_t *__restrict__ counts,
    int32_t *__restrict__ offsets, int32_t *__restrict__ perm, int32_t *__restrict__ inv,
    int4 *__restrict__ slots, int32_t *__restrict__ n_active, int32_t *__restrict__ tile_off,
    int BM)
{
    __shared__ int s_idx[SMALL_P];
    __shared__ int s_cnt[MAX_E];
    __shared__ int s_next[MAX_E];
    __shared__ int s_wcnt[16][MAX_E];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int P = T * k;
    const bool small = P <= SMALL_P;

    if (DO_TOPK) {
        for (int t = wave; t < T; t += 16) {
            const int sel = wave_topk(logits + (size_t)t * E, E, k, lane, topk_idx + (size_t)t * k,
                                      topk_w + (size_t)t * k);
            if (small && lane < k) s_idx[t * k + lane] = sel;
        }
        __threadfence_block();
    }
    const int32_t *idx = DO_TOPK ? topk_idx : idx_in;

    for (int i = tid; i < MAX_E; i += 1024) s_cnt[i] = 0;
    if (!small)
        for (int i = tid; i < 16 * MAX_E; i += 1024) (&s_wcnt[0][0])[i] = 0;
    __syncthreads();
    for (int p = tid; p < P; p += 1024) {
        int e;
        if (DO_TOPK && small) {
            e = s_idx[p];
        } else {
            e = clamp_id(idx[p], E);
            if (small) s_idx[p] = e;
        }
        atomicAdd(&s_cnt[e], 1);
    }
    __syncthreads();

    // exclusive scans over the experts by wave 0: lane owns experts 8*lane .. 8*lane+7
    if (wave == 0) {
        constexpr int PER = MAX_E / WAVE;
        int c[PER], lc = 0, la = 0, lt = 0;
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int e = lane * PER + i;
            c[i] = e < E ? s_cnt[e] : 0;
            lc += c[i];
            la += c[i] > 0;
            lt += BM > 0 ? (c[i] + BM - 1) / BM : 0;
        }
        int ic = lc, ia = la, it = lt;
#pragma unroll
        for (int off = 1; off < WAVE; off <<= 1) {
            const int oc = __shfl_up(ic, off, WAVE), oa = __shfl_up(ia, off, WAVE), ot = __shfl_up(it, off, WAVE);
            if (lane >= off) { ic += oc; ia += oa; it += ot; }
        }
        int pc = ic - lc, pa = ia - la, pt = it - lt;
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int e = lane * PER + i;
            if (e < E) {
                counts[e] = c[i];
                offsets[e] = pc;
                s_next[e] = pc;
                if (c[i] > 0 && slots) slots[pa] = make_int4(e, pc, c[i], 0);
                if (tile_off) tile_off[e] = pt;
            }
            pc += c[i];
            pa += c[i] > 0;
            pt += BM > 0 ? (c[i] + BM - 1) / BM : 0;
        }
        if (lane == WAVE - 1) {
            offsets[E] = ic;
            if (n_active) *n_active = ia;
            if (tile_off) tile_off[E] = it;
        }
    }
    __syncthreads();

    if (small) {
        // stable order: a pair's rank among its expert's pairs = earlier pairs with that expert
        if (tid < P) {
            const int e = s_idx[tid];
            int r = 0;
            for (int q = 0; q < tid; ++q) r += s_idx[q] == e;
            const int pos = s_next[e] + r;
            perm[pos] = tid;
            inv[tid] = pos;
        }
        return;
    }
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
    ProfScope ps(K_ROUTER, s);
    if (T <= 64) {
        const dim3 grid(E, (T + TT - 1) / TT);
        if (xtype == X_BF16)
            hipLaunchKernelGGL((router_logits_kernel<X_BF16, TT, 2>), grid, dim3(256), 0, s, x, T, d,
                               Wr, bias, E, logits);
        else
            hipLaunchKernelGGL((router_logits_kernel<X_F32, TT, 2>), grid, dim3(256), 0, s, x, T, d,
                               Wr, bias, E, logits);
        return hipGetLastError();
    }
    const dim3 grid((T + RB - 1) / RB, (E + RB - 1) / RB);
    if (xtype == X_BF16)
        hipLaunchKernelGGL((router_logits_mfma_kernel<X_BF16>), grid, dim3(256), 0, s, x, T, d, Wr, bias,
                           E, logits);
    else
        hipLaunchKernelGGL((router_logits_mfma_kernel<X_F32>), grid, dim3(256), 0, s, x, T, d, Wr, bias,
                           E, logits);
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
                           po.inv, po.slots, po.n_active, po.tile_off, BM);
    else
        hipLaunchKernelGGL((select_permute_kernel<false>), dim3(1), dim3(1024), 0, s, nullptr,
                           idx_in, T, k, E, nullptr, nullptr, po.counts, po.offsets, po.perm,
                           po.inv, po.slots, po.n_active, po.tile_off, BM);
    return hipGetLastError();
}

}  // namespace moe
