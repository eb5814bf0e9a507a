// Router and permute kernels (gfx950).
//
// Router: l[e] = x[t] . W_r[e] + b[e] accumulated in fp64 (every fp32 or bf16 by fp32 product is
// exact in fp64), so the selected experts are the exact-arithmetic ones; softmax over the k
// selected logits gives the renormalised top-k weights (equal to softmax over all E followed by
// renormalisation, the order the Inferentia page's router and the layer definition use).
// Top-k: one wavefront per token, k rounds of a wave-wide (logit desc, index asc) arg-max over
// ordered 64-bit keys of the logits.
//
// Permute: one workgroup builds the expert histogram (LDS atomics, order-free), the exclusive
// prefix sums and a stable scatter of the pairs into (expert, pair id) order, which is the
// gather the mul_mat_id step of the Gemma-on-a-Xeon page ("Three-part fix") needs on a GPU.
#include "moe_common.hpp"
#include "moe_launch.hpp"
#include "route_dev.hpp"

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

// Decode router: one block (4 waves) per expert row e and group of TT tokens.  Thread c takes
// the 8-float chunks c, c + 256, ... of the row, multiplies them with the same chunks of every
// token in fp64, and the partial sums meet in a fixed order: a butterfly inside each wave, then
// the four wave sums in wave order.
template <int XT>
__device__ __forceinline__ void load_x8f(const void *__restrict__ x, size_t off, float *xv)
{
    if (XT == X_BF16) {
        const uint4 b = *reinterpret_cast<const uint4 *>(reinterpret_cast<const uint16_t *>(x) + off);
        const uint32_t w[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            xv[2 * i] = __uint_as_float(w[i] << 16);
            xv[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
        }
    } else {
        const float4 p = *reinterpret_cast<const float4 *>(reinterpret_cast<const float *>(x) + off);
        const float4 q = *reinterpret_cast<const float4 *>(reinterpret_cast<const float *>(x) + off + 4);
        xv[0] = p.x; xv[1] = p.y; xv[2] = p.z; xv[3] = p.w;
        xv[4] = q.x; xv[5] = q.y; xv[6] = q.z; xv[7] = q.w;
    }
}

template <int XT, int TT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 2))) void router_logits_kernel(const void *__restrict__ x, int T, int d,
                                                            const float *__restrict__ Wr,
                                                            const float *__restrict__ bias, int E,
                                                            double *__restrict__ logits)
{
    __shared__ double red[TT][4];
    const int e = blockIdx.x;
    const int t0 = blockIdx.y * TT;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n8 = d >> 3;
    const int nt = min(TT, T - t0);
    double acc[TT];
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) acc[tt] = 0.0;
    const float4 *wrow = reinterpret_cast<const float4 *>(Wr + (size_t)e * d);
    // two chunks per pass (c and c + 256), all their loads issued together; a second chunk past
    // the row re-reads the last one and is left out by a select, not a branch
    for (int c = tid; c < n8; c += 512) {
        const int c2 = c + 256;
        const bool has2 = c2 < n8;
        const int cc[2] = {c, has2 ? c2 : n8 - 1};
        float wv[2][8], xv[2][TT][8];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const float4 w0 = wrow[2 * cc[h]], w1 = wrow[2 * cc[h] + 1];
            wv[h][0] = w0.x; wv[h][1] = w0.y; wv[h][2] = w0.z; wv[h][3] = w0.w;
            wv[h][4] = w1.x; wv[h][5] = w1.y; wv[h][6] = w1.z; wv[h][7] = w1.w;
            // a token slot past the batch re-reads the last token; its sums are never stored
#pragma unroll
            for (int tt = 0; tt < TT; ++tt)
                load_x8f<XT>(x, (size_t)(t0 + min(tt, nt - 1)) * d + 8 * (size_t)cc[h], xv[h][tt]);
        }
#pragma unroll
        for (int tt = 0; tt < TT; ++tt) {
            double a0 = acc[tt];
#pragma unroll
            for (int i = 0; i < 8; ++i) a0 = fma((double)wv[0][i], (double)xv[0][tt][i], a0);
            double a1 = a0;
#pragma unroll
            for (int i = 0; i < 8; ++i) a1 = fma((double)wv[1][i], (double)xv[1][tt][i], a1);
            acc[tt] = has2 ? a1 : a0;
        }
    }
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) {
        const double v = wave_sum_f64(acc[tt]);
        if (lane == 0) red[tt][wave] = v;
    }
    __syncthreads();
    if (tid < nt)
        logits[(size_t)(t0 + tid) * E + e] = ((red[tid][0] + red[tid][1]) + red[tid][2]) + red[tid][3] +
                                              (bias ? (double)bias[e] : 0.0);
}

// Decode router for narrow rows (d <= 1024): one wave per expert row, RPB = 4 rows per block, so
// a 1024-wide row is two 8-float chunks per lane and the sum needs no LDS: lane l takes chunks
// l, l + 64, l + 128, ... (pairs of them per pass, all loads of a pass issued together), and the
// wave's butterfly gives the row's fp64 sum in a fixed order.
template <int XT, int TT>
__global__ __launch_bounds__(256) void router_logits_rows_kernel(const void *__restrict__ x, int T, int d,
                                                                  const float *__restrict__ Wr,
                                                                  const float *__restrict__ bias, int E,
                                                                  double *__restrict__ logits)
{
    const int lane = threadIdx.x & 63;
    const int e = min(blockIdx.x * 4 + (threadIdx.x >> 6), E - 1);   // rows past E redo row E - 1
    const bool row_ok = blockIdx.x * 4 + (threadIdx.x >> 6) < E;
    const int t0 = blockIdx.y * TT;
    const int n8 = d >> 3;
    const int nt = min(TT, T - t0);
    double acc[TT];
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) acc[tt] = 0.0;
    const float4 *wrow = reinterpret_cast<const float4 *>(Wr + (size_t)e * d);
    for (int c = lane; c < n8; c += 128) {
        const int c2 = c + 64;
        const bool has2 = c2 < n8;
        const int cc[2] = {c, has2 ? c2 : n8 - 1};
        float wv[2][8], xv[2][TT][8];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const float4 w0 = wrow[2 * cc[h]], w1 = wrow[2 * cc[h] + 1];
            wv[h][0] = w0.x; wv[h][1] = w0.y; wv[h][2] = w0.z; wv[h][3] = w0.w;
            wv[h][4] = w1.x; wv[h][5] = w1.y; wv[h][6] = w1.z; wv[h][7] = w1.w;
#pragma unroll
            for (int tt = 0; tt < TT; ++tt)
                load_x8f<XT>(x, (size_t)(t0 + min(tt, nt - 1)) * d + 8 * (size_t)cc[h], xv[h][tt]);
        }
#pragma unroll
        for (int tt = 0; tt < TT; ++tt) {
            double a0 = acc[tt];
#pragma unroll
            for (int i = 0; i < 8; ++i) a0 = fma((double)wv[0][i], (double)xv[0][tt][i], a0);
            double a1 = a0;
#pragma unroll
            for (int i = 0; i < 8; ++i) a1 = fma((double)wv[1][i], (double)xv[1][tt][i], a1);
            acc[tt] = has2 ? a1 : a0;
        }
    }
    const double b = bias ? (double)bias[e] : 0.0;
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) {
        const double v = wave_sum_f64(acc[tt]);
        if (lane == 0 && row_ok && tt < nt) logits[(size_t)(t0 + tt) * E + e] = v + b;
    }
}

// Batched router on the fp64 matrix cores (v_mfma_f64_16x16x4_f64), operands straight from global
// memory: block = 32 tokens x 32 experts (four 16 x 16 tiles), 8 waves; wave w takes the 32-wide
// K chunks c = w, w + 8, w + 16, ... and keeps all four tiles in registers.  In MFMA step s of
// chunk c, lane (i, g) supplies K offset 32c + 8g + s of token row i (A) and of expert row i (B):
// A and B agree on which K each lane and step carries, so the 8 steps add every product of the
// chunk once, and each lane loads its 8 K values as one contiguous piece (16 bytes of bf16 x,
// 32 bytes of fp32 W).  Every product is exact in fp64 and the sums are fp64, as in the decode
// router; the order is fixed: per wave its chunks in order, then the 8 waves' sums in wave order,
// + bias.  Chunk c + 8's loads are issued before chunk c's MFMAs.  Rows past T or E re-read the
// last row (their results are never stored), so no load is conditional.
// A register-only probe sustains one v_mfma_f64_16x16x4_f64 per ~107 cycles per SIMD (4 waves per
// SIMD; ~114 with 2, ~153 with 1): about 47 TFLOP/s over the chip, so at T = 2048, E = 128,
// d = 2816 the 723k MFMAs take ~32 us, which is what this kernel measures (31 - 34 us; the same
// tiles staged through LDS as doubles: 42 us).  16-token blocks (4 waves per SIMD, 35.5 us) and a
// third register stage (32.4 us) measured no better.
typedef __attribute__((__vector_size__(4 * sizeof(double)))) double f64x4;
constexpr int RNW = 8;     // waves per block
constexpr int RRT = 2;     // 16-token row tiles per block
constexpr int RST = 2;     // register stages (chunks in flight per wave)
constexpr int RB = 16 * RRT, REB = 32;

template <int XT>
struct RChunk {
    uint4 x[RRT][XT == X_BF16 ? 1 : 2];   // token rows 16 rt + i: 8 values at 32c + 8g
    uint4 w[2][2];                        // expert rows 16 ct + i: 8 fp32 at 32c + 8g
};

template <int XT>
__global__ __launch_bounds__(64 * RNW) void router_logits_mfma_kernel(const void *__restrict__ x, int T, int d,
                                                                      const float *__restrict__ Wr,
                                                                      const float *__restrict__ bias, int E,
                                                                      double *__restrict__ logits)
{
    __shared__ f64x4 part[RNW][2 * RRT][64];           // each wave's tile sums
    const int t0 = blockIdx.x * RB, e0 = blockIdx.y * REB;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int li = lane & 15, lg = lane >> 4;
    const int NCH = d >> 5;                           // 32-wide K chunks (d is a multiple of 64)
    const uint16_t *xb = reinterpret_cast<const uint16_t *>(x);
    const float *xf = reinterpret_cast<const float *>(x);
    size_t xo[RRT], wo[2];
#pragma unroll
    for (int r = 0; r < RRT; ++r) xo[r] = (size_t)min(t0 + 16 * r + li, T - 1) * d + 8 * lg;
#pragma unroll
    for (int r = 0; r < 2; ++r) wo[r] = (size_t)min(e0 + 16 * r + li, E - 1) * d + 8 * lg;
    auto gload = [&](RChunk<XT> &R, int c) {
        const size_t k0 = (size_t)min(c, NCH - 1) * 32;   // past the end: a re-read, never used
#pragma unroll
        for (int r = 0; r < RRT; ++r) {
            if (XT == X_BF16) {
                R.x[r][0] = *reinterpret_cast<const uint4 *>(xb + xo[r] + k0);
            } else {
                R.x[r][0] = *reinterpret_cast<const uint4 *>(xf + xo[r] + k0);
                R.x[r][XT == X_BF16 ? 0 : 1] = *reinterpret_cast<const uint4 *>(xf + xo[r] + k0 + 4);
            }
        }
#pragma unroll
        for (int r = 0; r < 2; ++r) {
            R.w[r][0] = *reinterpret_cast<const uint4 *>(Wr + wo[r] + k0);
            R.w[r][1] = *reinterpret_cast<const uint4 *>(Wr + wo[r] + k0 + 4);
        }
    };
    auto word = [](const uint4 &v, int q) { return q == 0 ? v.x : q == 1 ? v.y : q == 2 ? v.z : v.w; };
    // value s (0..7) of a lane's 8, as a double (bf16 and fp32 convert exactly)
    auto xval = [&](const RChunk<XT> &R, int r, int s) {
        if (XT == X_BF16) {
            const uint32_t u = word(R.x[r][0], s >> 1);
            return (double)__uint_as_float((s & 1) ? (u & 0xFFFF0000u) : (u << 16));
        } else {
            return (double)__uint_as_float(word(R.x[r][(s >> 2) & (XT == X_BF16 ? 0 : 1)], s & 3));
        }
    };
    auto wval = [&](const RChunk<XT> &R, int r, int s) { return (double)__uint_as_float(word(R.w[r][s >> 2], s & 3)); };
    f64x4 acc[RRT][2];
#pragma unroll
    for (int a = 0; a < RRT; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b) acc[a][b] = f64x4{0.0, 0.0, 0.0, 0.0};
    auto compute = [&](const RChunk<XT> &R) {
#pragma unroll
        for (int s = 0; s < 8; ++s) {
            double av[RRT];
#pragma unroll
            for (int a = 0; a < RRT; ++a) av[a] = xval(R, a, s);
            const double b0 = wval(R, 0, s), b1 = wval(R, 1, s);
#pragma unroll
            for (int a = 0; a < RRT; ++a) {
                acc[a][0] = __builtin_amdgcn_mfma_f64_16x16x4f64(av[a], b0, acc[a][0], 0, 0, 0);
                acc[a][1] = __builtin_amdgcn_mfma_f64_16x16x4f64(av[a], b1, acc[a][1], 0, 0, 0);
            }
        }
    };
    // RST register stages: while chunk c is multiplied, the loads of chunks c + 8 .. c + 8 (RST - 1)
    // are in flight (stage j of a round holds chunk c + 8 j)
    RChunk<XT> R[RST];
#pragma unroll
    for (int j = 0; j + 1 < RST; ++j) gload(R[j], wave + RNW * j);
    for (int c = wave; c < NCH; c += RNW * RST) {
#pragma unroll
        for (int j = 0; j < RST; ++j) {
            if (c + RNW * j < NCH) {
                gload(R[(j + RST - 1) % RST], c + RNW * (j + RST - 1));
                compute(R[j]);
            }
        }
    }
    // the waves' sums, in wave order, + bias
#pragma unroll
    for (int a = 0; a < RRT; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b) part[wave][2 * a + b][lane] = acc[a][b];
    __syncthreads();
    if (wave >= 2 * RRT) return;
    const int tile = wave, wt = tile >> 1, we = tile & 1;
    f64x4 sum = part[0][tile][lane];
#pragma unroll
    for (int w = 1; w < RNW; ++w) sum += part[w][tile][lane];
    // the f64 16x16x4 result layout: lane holds C[token lg + 4*i][expert li] of its tile (unlike
    // the fp32 / int32 16x16 shapes, whose register i holds row 4*lg + i)
    const int e = e0 + we * 16 + li;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int t = t0 + wt * 16 + lg + 4 * i;
        if (t < T && e < E) logits[(size_t)t * E + e] = sum[i] + (bias ? (double)bias[e] : 0.0);
    }
}

template <int MAXV>
__global__ __launch_bounds__(256) void topk_kernel(const double *__restrict__ logits, int T, int E,
                                                   int k, int32_t *__restrict__ topk_idx,
                                                   float *__restrict__ topk_w)
{
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= T) return;                           // whole waves leave together
    wave_topk<MAXV>(logits + (size_t)t * E, E, k, threadIdx.x & 63, topk_idx + (size_t)t * k,
                    topk_w + (size_t)t * k);
}

// Top-k of one token per workgroup for more than 128 experts: MAXV waves sort 64 keys each and
// merge their lists (topk_sorted, a single pass).
template <int MAXV>
__global__ __launch_bounds__(64 * MAXV) void topk_sorted_kernel(const double *__restrict__ logits, int E, int k,
                                                               int32_t *__restrict__ topk_idx,
                                                               float *__restrict__ topk_w)
{
    __shared__ uint4 s_cand[MAXV * WAVE];
    __shared__ int s_idx[MAX_K];
    const size_t t = blockIdx.x;
    topk_sorted<MAXV, MAXV>(logits + t * E, 1, k, E, threadIdx.x >> 6, threadIdx.x & 63, topk_idx + t * k,
                            topk_w + t * k, s_idx, s_cand);
}

constexpr int SEL_P = 64 * MAX_K;     // pairs kept in LDS when the top-k runs in the same kernel

// The BM-row tiles of expert e (cnt pairs from permuted row off, first tile t0): {e, row, rows}.
__device__ __forceinline__ void write_tiles(int4 *tiles, int e, int t0, int off, int cnt, int BM)
{
    for (int t = 0; t * BM < cnt; ++t) tiles[t0 + t] = make_int4(e, off + t * BM, min(BM, cnt - t * BM), 0);
}

// S shared experts after the permute: slot records n_act .. n_act+S-1 = {E + s, P + s T, T, 0}
// with tokens 0 .. 15, the rows P + s T + t of the permuted order (holding pair t k, so that
// row / k is the token t), and with BM > 0 their BM-row tiles from tile t0 on.  Every thread of
// the workgroup calls it; nt threads.
__device__ void write_shared(int tid, int nt, int S, int E, int T, int k, int P, int n_act, int t0, int BM,
                             int4 *__restrict__ slots, int32_t *__restrict__ perm, int4 *__restrict__ tiles)
{
    for (int i = tid; i < S * T; i += nt) perm[P + i] = (i % T) * k;
    if (slots)
        for (int i = tid; i < S * (1 + SLOT_TOKS); i += nt) {
            const int sh = i / (1 + SLOT_TOKS), m = i - sh * (1 + SLOT_TOKS);
            int *rec = reinterpret_cast<int *>(slots + (size_t)(n_act + sh) * SLOT_INT4);
            if (m == 0)
                reinterpret_cast<int4 *>(rec)[0] = make_int4(E + sh, P + sh * T, T, 0);
            else if (m - 1 < T)
                rec[4 + m - 1] = m - 1;
        }
    if (tiles && BM > 0) {
        const int ntl = (T + BM - 1) / BM;
        for (int i = tid; i < S * ntl; i += nt) {
            const int sh = i / ntl, j = i - sh * ntl;
            tiles[t0 + i] = make_int4(E + sh, P + sh * T + j * BM, min(BM, T - j * BM), 0);
        }
    }
}

// Optionally selects the top-k of every token (DO_TOPK, T <= 64, E <= 128), then permutes the
// P = T*k pairs.  One workgroup of 1024 threads: LDS histogram, one-wave exclusive scans over the experts,
// then a stable scatter in rounds of 1024 pairs (a pair's rank among its wave's pairs of the same
// expert comes from ballots over the expert id bits).
template <bool DO_TOPK, int MAXV>
__global__ __launch_bounds__(1024) void select_permute_kernel(
    const double *__restrict__ logits, const int32_t *idx_in, int T, int k, int E,
    int32_t *topk_idx, float *__restrict__ topk_w, int32_t *__restrict__ counts,
    int32_t *__restrict__ offsets, int32_t *__restrict__ perm, int32_t *__restrict__ inv,
    int4 *__restrict__ slots, int32_t *__restrict__ n_active, int32_t *__restrict__ tile_off,
    int4 *__restrict__ tiles, int BM, int S)
{
    __shared__ int s_tot[2];                         // active routed experts, their tiles
    __shared__ int s_idx[DO_TOPK ? SEL_P : 1];
    __shared__ __attribute__((aligned(16))) int s_cnt[MAX_E];
    __shared__ int s_next[MAX_E];
    __shared__ int s_off[MAX_E];
    __shared__ int s_t0[MAX_E];
    __shared__ int s_slot[MAX_E];
    __shared__ int s_wcnt[16][MAX_E];
    static_assert(MAXV <= 2, "more than 128 experts select in topk_sorted_kernel");
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int P = T * k;

    for (int i = tid; i < MAX_E; i += 1024) s_cnt[i] = 0;
    for (int i = tid; i < 16 * MAX_E; i += 1024) (&s_wcnt[0][0])[i] = 0;
    if (DO_TOPK) {
        for (int t = wave; t < T; t += 16) {
            const int sel = wave_topk<MAXV>(logits + (size_t)t * E, E, k, lane, topk_idx + (size_t)t * k,
                                            topk_w + (size_t)t * k);
            if (lane < k) s_idx[t * k + lane] = sel;
        }
    }
    __syncthreads();
    auto expert_of = [&](int p) { return DO_TOPK ? s_idx[p] : clamp_id(idx_in[p], E); };
    for (int p = tid; p < P; p += 1024) atomicAdd(&s_cnt[expert_of(p)], 1);
    __syncthreads();

    // exclusive scans over the experts by wave 0: lane owns experts 8*lane .. 8*lane+7
    if (wave == 0) {
        constexpr int PER = MAX_E / WAVE;
        static_assert(PER == 8, "the count reads below take 8 experts per lane");
        int c[PER], lc = 0, la = 0, lt = 0;
        const int4 c0 = reinterpret_cast<const int4 *>(s_cnt)[2 * lane];       // zero past E
        const int4 c1 = reinterpret_cast<const int4 *>(s_cnt)[2 * lane + 1];
        c[0] = c0.x; c[1] = c0.y; c[2] = c0.z; c[3] = c0.w;
        c[4] = c1.x; c[5] = c1.y; c[6] = c1.z; c[7] = c1.w;
#pragma unroll
        for (int i = 0; i < PER; ++i) {
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
                s_off[e] = pc;
                s_slot[e] = pa;
                if (c[i] > 0 && slots) slots[(size_t)pa * SLOT_INT4] = make_int4(e, pc, c[i], 0);
                if (tile_off) tile_off[e] = pt;
                s_t0[e] = pt;
            }
            pc += c[i];
            pa += c[i] > 0;
            pt += BM > 0 ? (c[i] + BM - 1) / BM : 0;
        }
        if (lane == WAVE - 1) {
            offsets[E] = ic;
            if (n_active) *n_active = ia + S;
            if (tile_off) tile_off[E] = it + (BM > 0 ? S * ((T + BM - 1) / BM) : 0);
            s_tot[0] = ia;
            s_tot[1] = it;
        }
    }
    __syncthreads();
    if (tiles && BM > 0 && tid < E && s_cnt[tid] > 0) write_tiles(tiles, tid, s_t0[tid], s_off[tid], s_cnt[tid], BM);
    if (S > 0) write_shared(tid, 1024, S, E, T, k, T * k, s_tot[0], s_tot[1], BM, slots, perm, tiles);

    const int nbits = 32 - __clz(max(E - 1, 1));
    const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    for (int base = 0; base < P; base += 1024) {
        const int p = base + tid;
        const bool valid = p < P;
        const int e = valid ? expert_of(p) : 0;
        uint64_t m = __ballot(valid);
        for (int bit = 0; bit < nbits; ++bit) {
            const bool b = (e >> bit) & 1;
            const uint64_t bal = __ballot(valid && b);
            m &= b ? bal : ~bal;
        }
        const int rank = __popcll(m & lt);
        if (valid && rank == 0) s_wcnt[wave][e] = __popcll(m);
        __syncthreads();
        if (valid) {
            int pre = 0;
            for (int w = 0; w < wave; ++w) pre += s_wcnt[w][e];
            const int pos = s_next[e] + pre + rank;
            perm[pos] = p;
            inv[p] = pos;
            const int m = pos - s_off[e];             // the pair's place among its expert's pairs
            if (slots && m < SLOT_TOKS)
                reinterpret_cast<int *>(slots + (size_t)s_slot[e] * SLOT_INT4)[4 + m] = p / k;
        }
        if (base + 1024 >= P) break;              // block-uniform: the last round needs no clean-up
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
// Permute of many pairs over many workgroups: per-block expert histograms, one workgroup that
// turns them into per-block starting rows (and the counts, offsets, slot records and M-tile
// prefix), then a stable per-block scatter.  The result is the single-workgroup kernel's.
// ------------------------------------------------------------------------------------------

constexpr int PB = 1024;              // pairs per block
constexpr int PERMUTE_ONE_BLOCK_MAX = 2048;   // more pairs than this use the multi-block permute

__global__ __launch_bounds__(PB) void pair_hist_kernel(const int32_t *__restrict__ idx, int P, int E,
                                                       int32_t *__restrict__ hist)
{
    __shared__ int h[MAX_E];
    const int tid = threadIdx.x;
    for (int i = tid; i < E; i += PB) h[i] = 0;
    __syncthreads();
    const int p = blockIdx.x * PB + tid;
    if (p < P) atomicAdd(&h[clamp_id(idx[p], E)], 1);
    __syncthreads();
    for (int i = tid; i < E; i += PB) hist[(size_t)blockIdx.x * E + i] = h[i];
}


// Scan and scatter in one kernel: block b first sums the per-block histograms itself (expert e's
// total, and its count in blocks before b), scans the totals over the experts (wave 0, 8 experts
// per lane: pair offsets, active slots, M-tiles), and then scatters its pairs as
// follows: a pair's place is base[b][e] = offsets[e] + the count before b, plus the earlier waves'
// pairs of expert e in the block, plus its rank among its own wave's (ballots over the id bits);
// pairs among the first SLOT_TOKS of their expert also record their token in the expert's slot
// record.  Block 0 also writes the counts, offsets, per-expert records, M-tile records, the active
// count and the shared experts' rows.  The histogram is nb x E ints (8 KB at 16 blocks x 128
// experts), read by every block from L2.
__global__ __launch_bounds__(PB) void pair_scan_scatter_kernel(
    const int32_t *__restrict__ idx, int P, int k, int E, int nb, const int32_t *__restrict__ hist, int BM,
    int32_t *__restrict__ counts, int32_t *__restrict__ offsets, int4 *__restrict__ slots,
    int32_t *__restrict__ n_active, int32_t *__restrict__ tile_off, int4 *__restrict__ tiles, int T, int S,
    int32_t *__restrict__ perm, int32_t *__restrict__ inv)
{
    __shared__ __attribute__((aligned(16))) int s_cnt[MAX_E];
    __shared__ int s_off[MAX_E], s_slot[MAX_E], s_t0[MAX_E], s_base[MAX_E];
    __shared__ int s_tot[2];
    __shared__ int s_wcnt[PB / WAVE][MAX_E];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int b = blockIdx.x;
    const bool lead = b == 0;
    for (int i = tid; i < (PB / WAVE) * MAX_E; i += PB) (&s_wcnt[0][0])[i] = 0;
    // this block's pair: its expert and its rank among the wave's pairs of that expert
    const int p = b * PB + tid;
    const bool valid = p < P;
    const int e = valid ? clamp_id(idx[p], E) : 0;
    // column sums, 16 rows at a time (a row past nb re-reads the last, unused)
    constexpr int CB = 16;
    int before = 0;
    if (tid < MAX_E) {
        int run = 0;
        if (tid < E)
            for (int b0 = 0; b0 < nb; b0 += CB) {
                int c[CB];
#pragma unroll
                for (int j = 0; j < CB; ++j) c[j] = hist[(size_t)min(b0 + j, nb - 1) * E + tid];
#pragma unroll
                for (int j = 0; j < CB; ++j) {
                    run += b0 + j < nb ? c[j] : 0;
                    before += b0 + j < b ? c[j] : 0;
                }
            }
        s_cnt[tid] = run;
    }
    const int nbits = 32 - __clz(max(E - 1, 1));
    uint64_t m = __ballot(valid);
    for (int bit = 0; bit < nbits; ++bit) {
        const bool bb = (e >> bit) & 1;
        const uint64_t bal = __ballot(valid && bb);
        m &= bb ? bal : ~bal;
    }
    const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    const int rank = __popcll(m & lt);
    __syncthreads();                                 // totals in, the zeroing done
    if (valid && rank == 0) s_wcnt[wave][e] = __popcll(m);
    if (wave == 0) {
        constexpr int PER = MAX_E / WAVE;
        static_assert(PER == 8, "the count reads below take 8 experts per lane");
        int c[PER], lc = 0, la = 0, lt8 = 0;
        const int4 c0 = reinterpret_cast<const int4 *>(s_cnt)[2 * lane];       // zero past E
        const int4 c1 = reinterpret_cast<const int4 *>(s_cnt)[2 * lane + 1];
        c[0] = c0.x; c[1] = c0.y; c[2] = c0.z; c[3] = c0.w;
        c[4] = c1.x; c[5] = c1.y; c[6] = c1.z; c[7] = c1.w;
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            lc += c[i];
            la += c[i] > 0;
            lt8 += BM > 0 ? (c[i] + BM - 1) / BM : 0;
        }
        int ic = lc, ia = la, it = lt8;
#pragma unroll
        for (int off = 1; off < WAVE; off <<= 1) {
            const int oc = __shfl_up(ic, off, WAVE), oa = __shfl_up(ia, off, WAVE), ot = __shfl_up(it, off, WAVE);
            if (lane >= off) { ic += oc; ia += oa; it += ot; }
        }
        int pc = ic - lc, pa = ia - la, pt = it - lt8;
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int ee = lane * PER + i;
            if (ee < E) {
                s_off[ee] = pc;
                s_slot[ee] = pa;
                s_t0[ee] = pt;
                if (lead) {
                    counts[ee] = c[i];
                    offsets[ee] = pc;
                    if (c[i] > 0 && slots) slots[(size_t)pa * SLOT_INT4] = make_int4(ee, pc, c[i], 0);
                    if (tile_off) tile_off[ee] = pt;
                }
            }
            pc += c[i];
            pa += c[i] > 0;
            pt += BM > 0 ? (c[i] + BM - 1) / BM : 0;
        }
        if (lane == WAVE - 1) {
            if (lead) {
                offsets[E] = ic;
                if (n_active) *n_active = ia + S;
                if (tile_off) tile_off[E] = it + (BM > 0 ? S * ((T + BM - 1) / BM) : 0);
            }
            s_tot[0] = ia;
            s_tot[1] = it;
        }
    }
    __syncthreads();
    if (tid < E) s_base[tid] = s_off[tid] + before;
    if (lead) {
        if (tiles && BM > 0 && tid < E && s_cnt[tid] > 0) write_tiles(tiles, tid, s_t0[tid], s_off[tid], s_cnt[tid], BM);
        if (S > 0) write_shared(tid, PB, S, E, T, k, T * k, s_tot[0], s_tot[1], BM, slots, perm, tiles);
    }
    __syncthreads();
    if (valid) {
        int pre = 0;
        for (int w = 0; w < wave; ++w) pre += s_wcnt[w][e];
        const int pos = s_base[e] + pre + rank;
        perm[pos] = p;
        inv[p] = pos;
        const int mm = pos - s_off[e];
        if (slots && mm < SLOT_TOKS)
            reinterpret_cast<int *>(slots + (size_t)s_slot[e] * SLOT_INT4)[4 + mm] = p / k;
    }
}


// ------------------------------------------------------------------------------------------
// Host launchers
// ------------------------------------------------------------------------------------------

constexpr int ROUTER_ROWS_MAX_D = 1024;   // a wave per expert row up to this width

hipError_t launch_router_logits(const void *x, int xtype, int T, int d, const float *Wr,
                                const float *bias, int E, double *logits, hipStream_t s)
{
    ProfScope ps(K_ROUTER, s);
    if (T <= 64) {
        // tokens per block (a block re-reads its expert row for each group of TT tokens; a slot
        // past the batch re-reads the last token).  Gemma-shaped decode, tokens/s with TT = 1 / 2 /
        // 4 / 8: T = 1 41.3k / 40.9k / 40.3k / 38.8k, T = 2 58.7k / 58.3k / 57.5k / 56.0k, T = 8
        // 105.6k / 106.6k / 106.4k / 105.2k.
#define RL(TT) do {                                                                                          \
        const dim3 grid(E, (T + TT - 1) / TT);                                                              \
        if (xtype == X_BF16)                                                                                \
            hipLaunchKernelGGL((router_logits_kernel<X_BF16, TT>), grid, dim3(256), 0, s, x, T, d, Wr, bias, E, \
                               logits);                                                                     \
        else                                                                                                \
            hipLaunchKernelGGL((router_logits_kernel<X_F32, TT>), grid, dim3(256), 0, s, x, T, d, Wr, bias, E, \
                               logits);                                                                     \
    } while (0)
#define RR(TT) do {                                                                                          \
        const dim3 grid((E + 3) / 4, (T + TT - 1) / TT);                                                    \
        if (xtype == X_BF16)                                                                                \
            hipLaunchKernelGGL((router_logits_rows_kernel<X_BF16, TT>), grid, dim3(256), 0, s, x, T, d, Wr, bias, \
                               E, logits);                                                                  \
        else                                                                                                \
            hipLaunchKernelGGL((router_logits_rows_kernel<X_F32, TT>), grid, dim3(256), 0, s, x, T, d, Wr, bias, \
                               E, logits);                                                                  \
    } while (0)
        if (d <= ROUTER_ROWS_MAX_D) {
            if (T <= 2) RR(1);
            else if (T <= 8) RR(2);
            else RR(8);
        } else {
            if (T <= 2) RL(1);
            else if (T <= 8) RL(2);
            else RL(8);
        }
#undef RL
#undef RR
        return hipGetLastError();
    }
    const dim3 grid((T + RB - 1) / RB, (E + REB - 1) / REB);
    if (xtype == X_BF16)
        hipLaunchKernelGGL((router_logits_mfma_kernel<X_BF16>), grid, dim3(64 * RNW), 0, s, x, T, d, Wr, bias,
                           E, logits);
    else
        hipLaunchKernelGGL((router_logits_mfma_kernel<X_F32>), grid, dim3(64 * RNW), 0, s, x, T, d, Wr, bias,
                           E, logits);
    return hipGetLastError();
}

// slots per lane for E experts (E <= 512)
static int topk_maxv(int E) { return E <= 64 ? 1 : E <= 128 ? 2 : E <= 256 ? 4 : 8; }

static hipError_t launch_topk_sorted(const double *logits, int T, int E, int k, int32_t *idx, float *w,
                                     hipStream_t s)
{
    if (topk_maxv(E) == 4)
        hipLaunchKernelGGL(topk_sorted_kernel<4>, dim3(T), dim3(4 * WAVE), 0, s, logits, E, k, idx, w);
    else
        hipLaunchKernelGGL(topk_sorted_kernel<8>, dim3(T), dim3(8 * WAVE), 0, s, logits, E, k, idx, w);
    return hipGetLastError();
}

hipError_t launch_topk(const double *logits, int T, int E, int k, int32_t *idx, float *w,
                       hipStream_t s)
{
    ProfScope ps(K_TOPK, s);
    if (E > 128) return launch_topk_sorted(logits, T, E, k, idx, w, s);
    const dim3 g((T + 3) / 4), b(256);
    switch (topk_maxv(E)) {
    case 1: hipLaunchKernelGGL((topk_kernel<1>), g, b, 0, s, logits, T, E, k, idx, w); break;
    case 2: hipLaunchKernelGGL((topk_kernel<2>), g, b, 0, s, logits, T, E, k, idx, w); break;
    case 4: hipLaunchKernelGGL((topk_kernel<4>), g, b, 0, s, logits, T, E, k, idx, w); break;
    default: hipLaunchKernelGGL((topk_kernel<8>), g, b, 0, s, logits, T, E, k, idx, w); break;
    }
    return hipGetLastError();
}

int permute_scratch_ints(int P, int E) { return ((P + PB - 1) / PB) * E; }   // per-block histograms

// Selection and permute of a small decode batch (T <= 8, T k <= 64, E <= 128, no prefill tiles) in
// one 8-wave workgroup: wave t selects token t's top-k (wave_topk), the pairs are counted in LDS,
// then wave 0 alone scans the counts (lane l: experts 2l, 2l + 1), writes the per-expert records,
// and places every pair p (lane p) at its expert's offset + its rank among the earlier pairs of
// that expert (ballots over the expert id bits), the offsets coming from the scanning lanes by
// shuffles.  The same outputs as select_permute_kernel with fewer threads and barriers.
__global__ __launch_bounds__(512) void select_small_kernel(const double *__restrict__ logits, int T, int k, int E,
                                                           int32_t *topk_idx, float *__restrict__ topk_w,
                                                           int32_t *__restrict__ counts, int32_t *__restrict__ offsets,
                                                           int32_t *__restrict__ perm, int32_t *__restrict__ inv,
                                                           int4 *__restrict__ slots, int32_t *__restrict__ n_active,
                                                           int S)
{
    __shared__ int s_idx[64];
    __shared__ __attribute__((aligned(16))) int s_cnt[128];
    __shared__ int s_nact;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int P = T * k;
    if (tid < 128) s_cnt[tid] = 0;
    if (wave < T) {
        const int sel = wave_topk<2>(logits + (size_t)wave * E, E, k, lane, topk_idx + (size_t)wave * k,
                                     topk_w + (size_t)wave * k);
        if (lane < k) s_idx[wave * k + lane] = sel;
    }
    __syncthreads();
    if (tid < P) atomicAdd(&s_cnt[s_idx[tid]], 1);   // (order-free)
    __syncthreads();
    if (wave == 0) {
        const int c0 = s_cnt[2 * lane], c1 = s_cnt[2 * lane + 1];
        const int la = (c0 > 0) + (c1 > 0), lc = c0 + c1;
        int ia = la, ic = lc;
#pragma unroll
        for (int off = 1; off < WAVE; off <<= 1) {
            const int oa = __shfl_up(ia, off, WAVE), oc = __shfl_up(ic, off, WAVE);
            if (lane >= off) {
                ia += oa;
                ic += oc;
            }
        }
        const int pa = ia - la, pc = ic - lc;       // active experts and pairs before expert 2 lane
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int e = 2 * lane + i, c = i ? c1 : c0;
            const int off = i ? pc + c0 : pc, sl = i ? pa + (c0 > 0) : pa;
            if (e < E) {
                counts[e] = c;
                offsets[e] = off;
                if (c > 0) slots[(size_t)sl * SLOT_INT4] = make_int4(e, off, c, 0);
            }
        }
        if (lane == WAVE - 1) {
            offsets[E] = ic;
            *n_active = ia + S;
            s_nact = ia;
        }
        // pair p = lane: its rank among the earlier pairs of the same expert
        const bool valid = lane < P;
        const int e = valid ? s_idx[min(lane, P - 1)] : 0;
        uint64_t m = __ballot(valid);
#pragma unroll
        for (int bit = 0; bit < 7; ++bit) {
            const bool b = (e >> bit) & 1;
            const uint64_t bal = __ballot(valid && b);
            m &= b ? bal : ~bal;
        }
        const uint64_t lt = lane == 0 ? 0ull : (~0ull >> (64 - lane));
        const int rank = __popcll(m & lt);
        const int src = e >> 1;
        const int o0 = __shfl(pc, src, WAVE), cs = __shfl(c0, src, WAVE), a0 = __shfl(pa, src, WAVE);
        const int off_e = (e & 1) ? o0 + cs : o0, slot_e = (e & 1) ? a0 + (cs > 0) : a0;
        if (valid) {
            const int pos = off_e + rank;
            perm[pos] = lane;
            inv[lane] = pos;
            if (rank < SLOT_TOKS) reinterpret_cast<int *>(slots + (size_t)slot_e * SLOT_INT4)[4 + rank] = lane / k;
        }
    }
    if (S > 0) {
        __syncthreads();
        write_shared(tid, 512, S, E, T, k, P, s_nact, 0, 0, slots, perm, nullptr);
    }
}

// The same for 128 < E <= 64 MAXV experts (MAXV = 4, 8) and T <= 16 / MAXV tokens: the top-k by
// topk_sorted in one pass of the 16 waves, then as above with wave 0 holding 8 experts per lane;
// the per-expert offsets and slots go through LDS (one more barrier) instead of shuffles.
template <int MAXV>
__global__ __launch_bounds__(1024) void select_small_sorted_kernel(
    const double *__restrict__ logits, int T, int k, int E, int32_t *topk_idx, float *__restrict__ topk_w,
    int32_t *__restrict__ counts, int32_t *__restrict__ offsets, int32_t *__restrict__ perm,
    int32_t *__restrict__ inv, int4 *__restrict__ slots, int32_t *__restrict__ n_active, int S)
{
    constexpr int PER = 8;                           // experts per lane of wave 0 (E <= 512)
    __shared__ int s_idx[64];
    __shared__ __attribute__((aligned(16))) int s_cnt[WAVE * PER];
    __shared__ int s_off[WAVE * PER], s_slot[WAVE * PER];
    __shared__ uint4 s_cand[16 * WAVE];
    __shared__ int s_nact;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int P = T * k;
    if (tid < WAVE * PER) s_cnt[tid] = 0;
    topk_sorted<MAXV>(logits, T, k, E, wave, lane, topk_idx, topk_w, s_idx, s_cand);
    __syncthreads();
    if (tid < P) atomicAdd(&s_cnt[s_idx[tid]], 1);   // (order-free)
    __syncthreads();
    if (wave == 0) {
        int c[PER], lc = 0, la = 0;
        const int4 c0 = reinterpret_cast<const int4 *>(s_cnt)[2 * lane];
        const int4 c1 = reinterpret_cast<const int4 *>(s_cnt)[2 * lane + 1];
        c[0] = c0.x; c[1] = c0.y; c[2] = c0.z; c[3] = c0.w;
        c[4] = c1.x; c[5] = c1.y; c[6] = c1.z; c[7] = c1.w;
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            lc += c[i];
            la += c[i] > 0;
        }
        int ic = lc, ia = la;
#pragma unroll
        for (int off = 1; off < WAVE; off <<= 1) {
            const int oc = __shfl_up(ic, off, WAVE), oa = __shfl_up(ia, off, WAVE);
            if (lane >= off) {
                ic += oc;
                ia += oa;
            }
        }
        int pc = ic - lc, pa = ia - la;
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int e = lane * PER + i;
            if (e < E) {
                counts[e] = c[i];
                offsets[e] = pc;
                s_off[e] = pc;
                s_slot[e] = pa;
                if (c[i] > 0) slots[(size_t)pa * SLOT_INT4] = make_int4(e, pc, c[i], 0);
            }
            pc += c[i];
            pa += c[i] > 0;
        }
        if (lane == WAVE - 1) {
            offsets[E] = ic;
            *n_active = ia + S;
            s_nact = ia;
        }
    }
    __syncthreads();
    if (wave == 0) {                                 // pair p = lane
        const bool valid = lane < P;
        const int e = valid ? s_idx[min(lane, P - 1)] : 0;
        uint64_t m = __ballot(valid);
#pragma unroll
        for (int bit = 0; bit < 9; ++bit) {
            const bool b = (e >> bit) & 1;
            const uint64_t bal = __ballot(valid && b);
            m &= b ? bal : ~bal;
        }
        const uint64_t lt = lane == 0 ? 0ull : (~0ull >> (64 - lane));
        const int rank = __popcll(m & lt);
        if (valid) {
            const int pos = s_off[e] + rank;
            perm[pos] = lane;
            inv[lane] = pos;
            if (rank < SLOT_TOKS) reinterpret_cast<int *>(slots + (size_t)s_slot[e] * SLOT_INT4)[4 + rank] = lane / k;
        }
    }
    if (S > 0) write_shared(tid, 1024, S, E, T, k, P, s_nact, 0, 0, slots, perm, nullptr);
}

hipError_t launch_select_permute(const double *logits, const int32_t *idx_in, int T, int k, int E,
                                 int32_t *topk_idx, float *topk_w, const PermuteOut &po, int BM, int S,
                                 hipStream_t s)
{
    ProfScope ps(K_PERMUTE, s);
    const int P = T * k;
    if (logits && BM == 0 && T <= 8 && P <= 64 && E <= 128 && po.slots) {
        hipLaunchKernelGGL(select_small_kernel, dim3(1), dim3(512), 0, s, logits, T, k, E, topk_idx, topk_w,
                           po.counts, po.offsets, po.perm, po.inv, po.slots, po.n_active, S);
        return hipGetLastError();
    }
    if (logits && BM == 0 && E > 128 && E <= 512 && P <= 64 && T * topk_maxv(E) <= 16 && po.slots) {
#define SS(V) hipLaunchKernelGGL((select_small_sorted_kernel<V>), dim3(1), dim3(1024), 0, s, logits, T, k, E, topk_idx, \
                                 topk_w, po.counts, po.offsets, po.perm, po.inv, po.slots, po.n_active, S)
        if (topk_maxv(E) == 4) SS(4);
        else SS(8);
#undef SS
        return hipGetLastError();
    }
    if (logits && E > 128) {
        // More lists than one workgroup sorts in a pass: a workgroup per token selects (one pass
        // each), then the permute below reads the ids back.
        if (!topk_idx || !topk_w) return hipErrorInvalidValue;
        const hipError_t e = launch_topk_sorted(logits, T, E, k, topk_idx, topk_w, s);
        if (e != hipSuccess) return e;
        logits = nullptr;
        idx_in = topk_idx;
    }
    if (!logits && P > PERMUTE_ONE_BLOCK_MAX && po.scratch) {
        const int nb = (P + PB - 1) / PB;
        int32_t *hist = po.scratch;
        hipLaunchKernelGGL(pair_hist_kernel, dim3(nb), dim3(PB), 0, s, idx_in, P, E, hist);
        hipLaunchKernelGGL(pair_scan_scatter_kernel, dim3(nb), dim3(PB), 0, s, idx_in, P, k, E, nb, hist, BM,
                           po.counts, po.offsets, po.slots, po.n_active, po.tile_off, po.tiles, T, S, po.perm,
                           po.inv);
        return hipGetLastError();
    }
    const dim3 g(1), b(1024);
    if (logits) {
        if (T * k > SEL_P) return hipErrorInvalidValue;
#define SP(V) hipLaunchKernelGGL((select_permute_kernel<true, V>), g, b, 0, s, logits, nullptr, T, k, E, \
                                 topk_idx, topk_w, po.counts, po.offsets, po.perm, po.inv, po.slots,    \
                                 po.n_active, po.tile_off, po.tiles, BM, S)
        if (topk_maxv(E) == 1) SP(1);        // (E <= 128 here)
        else SP(2);
#undef SP
    } else {
        hipLaunchKernelGGL((select_permute_kernel<false, 1>), g, b, 0, s, nullptr, idx_in, T, k, E,
                           nullptr, nullptr, po.counts, po.offsets, po.perm, po.inv, po.slots,
                           po.n_active, po.tile_off, po.tiles, BM, S);
    }
    return hipGetLastError();
}

}  // namespace moe
