// Q8_0 and per-row-int8 expert FFN on the gfx950 bf16 matrix cores.
//
// Gate/up (the mul_mat_id over the stacked [n_embd, 2*n_ff, n_experts] tensor followed by
// fused_mul_unary(gate, up, SILU) of "Running Gemma 4 26B at 5 tokens/s on a 13-year-old Xeon",
// "Three-part fix"; or the ungated ReLU^2 up of the Nemotron page, "bytes per token") and down +
// weighted combine (the fixed-order per-(token, expert) sum of the Nemotron page, "How
// correctness is checked").
//
// Decode batches are small (a handful of tokens per expert) and the layer is a weight stream, so
// each workgroup streams a 16-row tile of one expert's matrix exactly once and multiplies it by
// every token routed to that expert with v_mfma_f32_16x16x32_bf16: A = 16 tokens x 32 K
// activations, B = 32 K x 16 weight rows.  One MFMA spans exactly one Q8_0 block, so its result
// is scaled by that block's fp16 scale before accumulation.  int8 weights and bf16 activations
// are exact in bf16; fp32 inputs (fp32 x, the fp32 h of the down projection) are split into two
// or three bf16 terms, so all products are exact and accumulate in fp32.
#include "moe_common.hpp"
#include "moe_launch.hpp"

namespace moe {

// Loads the A operand (8 consecutive activations of one token) as NT bf16x8 terms.
template <int XT, int NT>
__device__ __forceinline__ void load_x8(const void *__restrict__ x, size_t off, bool valid,
                                        bf16x8 *a)
{
    if (XT == X_BF16) {
        U4 t;
        t.u = valid ? *reinterpret_cast<const uint4 *>(reinterpret_cast<const uint16_t *>(x) + off)
                    : make_uint4(0, 0, 0, 0);
        a[0] = t.v;
    } else {
        float v[8];
        if (valid) {
            const float4 p = *reinterpret_cast<const float4 *>(reinterpret_cast<const float *>(x) + off);
            const float4 q = *reinterpret_cast<const float4 *>(reinterpret_cast<const float *>(x) + off + 4);
            v[0] = p.x; v[1] = p.y; v[2] = p.z; v[3] = p.w;
            v[4] = q.x; v[5] = q.y; v[6] = q.z; v[7] = q.w;
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) v[i] = 0.f;
        }
        split_f32x8<NT>(v, a);
    }
}

// grid.x = max_slots * (d_ff / 16); workgroup = NW waves splitting the K dimension.
template <int FMT, int ACT, int XT, int NW, int U>
__global__ __launch_bounds__(64 * NW) void gateup_int8_kernel(
    const void *__restrict__ x, int d, int k, const int8_t *__restrict__ wgu,
    const void *__restrict__ wgu_scales, int d_ff, const int32_t *__restrict__ offsets,
    const int32_t *__restrict__ perm, const int32_t *__restrict__ active,
    const int32_t *__restrict__ n_active, float *__restrict__ h)
{
    constexpr bool GATED = ACT == ACT_SWIGLU;
    constexpr int NT = XT == X_F32 ? 3 : 1;
    __shared__ f32x4 red[NW][2][WAVE];

    const int nft = d_ff >> 4;
    const int slot = blockIdx.x / nft;
    const int ft = blockIdx.x - slot * nft;
    if (slot >= *n_active) return;
    const int e = active[slot];
    const int row0 = offsets[e];
    const int n_e = offsets[e + 1] - row0;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int li = lane & 15, lg = lane >> 4;
    const int f = ft * 16 + li;
    const int rows = GATED ? 2 * d_ff : d_ff;
    const int nb = d >> 5;
    const int kb0 = wave * nb / NW, kb1 = (wave + 1) * nb / NW;
    const size_t r0 = (size_t)e * rows + f;       // gate row, or the up row when ungated
    const size_t r1 = r0 + (GATED ? d_ff : 0);    // up row (gated)
    const int8_t *w0 = wgu + r0 * d + lg * 8;
    const int8_t *w1 = wgu + r1 * d + lg * 8;
    const uint16_t *q0 = reinterpret_cast<const uint16_t *>(wgu_scales) + r0 * nb;
    const uint16_t *q1 = reinterpret_cast<const uint16_t *>(wgu_scales) + r1 * nb;

    for (int m0 = 0; m0 < n_e; m0 += 16) {
        const int mi = m0 + li;
        const bool mvalid = mi < n_e;
        const int tok = mvalid ? perm[row0 + mi] / k : 0;
        const size_t xoff = (size_t)tok * d + lg * 8;
        f32x4 acc0 = zero4(), acc1 = zero4();
        for (int kb = kb0; kb < kb1; kb += U) {
            uint2 wa[U], wb[U];
            float s0[U], s1[U];
            bf16x8 a[U][NT];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int kc = min(kb + u, kb1 - 1);   // the tail re-reads the last block
                load_x8<XT, NT>(x, xoff + (size_t)kc * 32, mvalid, a[u]);
                wa[u] = *reinterpret_cast<const uint2 *>(w0 + kc * 32);
                if (GATED) wb[u] = *reinterpret_cast<const uint2 *>(w1 + kc * 32);
                if (FMT == W_Q8_0) {
                    s0[u] = half_bits_to_float(q0[kc]);
                    if (GATED) s1[u] = half_bits_to_float(q1[kc]);
                }
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                if (kb + u < kb1) {
                    const bf16x8 b0 = i8x8_to_bf16x8(wa[u].x, wa[u].y);
                    if (FMT == W_Q8_0) {
                        f32x4 c = zero4();
#pragma unroll
                        for (int t = 0; t < NT; ++t) c = mfma16x16x32_bf16(a[u][t], b0, c);
                        acc0 += c * s0[u];
                    } else {
#pragma unroll
                        for (int t = 0; t < NT; ++t) acc0 = mfma16x16x32_bf16(a[u][t], b0, acc0);
                    }
                    if (GATED) {
                        const bf16x8 b1 = i8x8_to_bf16x8(wb[u].x, wb[u].y);
                        if (FMT == W_Q8_0) {
                            f32x4 c = zero4();
#pragma unroll
                            for (int t = 0; t < NT; ++t) c = mfma16x16x32_bf16(a[u][t], b1, c);
                            acc1 += c * s1[u];
                        } else {
#pragma unroll
                            for (int t = 0; t < NT; ++t) acc1 = mfma16x16x32_bf16(a[u][t], b1, acc1);
                        }
                    }
                }
            }
        }
        red[wave][0][lane] = acc0;
        red[wave][1][lane] = acc1;
        __syncthreads();
        if (wave == 0) {
            f32x4 g = red[0][0][lane], u = red[0][1][lane];
#pragma unroll
            for (int w = 1; w < NW; ++w) {
                g += red[w][0][lane];
                u += red[w][1][lane];
            }
            if (FMT == W_I8_ROW) {
                const float *rs = reinterpret_cast<const float *>(wgu_scales);
                g *= rs[r0];
                if (GATED) u *= rs[r1];
            }
            // lane holds C[token m0 + 4*lg + i][row f]
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int m = m0 + 4 * lg + i;
                if (m < n_e) {
                    float hv;
                    if (GATED) {
                        hv = silu_f32(g[i]) * u[i];
                    } else {
                        hv = g[i] > 0.f ? g[i] * g[i] : 0.f;
                    }
                    h[(size_t)(row0 + m) * d_ff + f] = hv;
                }
            }
        }
        __syncthreads();
    }
}

// grid.x = d_model / 16 output rows; NW waves take the active experts round robin.  FUSED: the
// y of every pair for these 16 outputs stays in LDS and the block combines them in slot order.
template <int FMT, int NW, int U, bool FUSED>
__global__ __launch_bounds__(64 * NW) void down_int8_kernel(
    const float *__restrict__ h, int d_ff, const int8_t *__restrict__ wd,
    const void *__restrict__ wd_scales, int d, const int32_t *__restrict__ offsets,
    const int32_t *__restrict__ active, const int32_t *__restrict__ n_active,
    const int32_t *__restrict__ inv, const float *__restrict__ topk_w, int T, int k,
    float *__restrict__ out, float *__restrict__ ybuf)
{
    extern __shared__ float y_lds[];
    const int o0 = blockIdx.x * 16;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int li = lane & 15, lg = lane >> 4;
    const int na = *n_active;
    const int nb = d_ff >> 5;
    for (int s = wave; s < na; s += NW) {
        const int e = active[s];
        const int row0 = offsets[e], n_e = offsets[e + 1] - row0;
        const size_t wr = (size_t)e * d + o0 + li;
        const int8_t *wrow = wd + wr * d_ff + lg * 8;
        const uint16_t *qs = reinterpret_cast<const uint16_t *>(wd_scales) + wr * nb;
        for (int m0 = 0; m0 < n_e; m0 += 16) {
            const int mi = m0 + li;
            const bool mvalid = mi < n_e;
            const float *hrow = h + (size_t)(row0 + (mvalid ? mi : 0)) * d_ff + lg * 8;
            f32x4 acc = zero4();
            for (int kb = 0; kb < nb; kb += U) {
                float hv[U][8];
                uint2 wv[U];
                float sc[U];
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const int kc = min(kb + u, nb - 1);
                    if (mvalid) {
                        const float4 p = *reinterpret_cast<const float4 *>(hrow + kc * 32);
                        const float4 q = *reinterpret_cast<const float4 *>(hrow + kc * 32 + 4);
                        hv[u][0] = p.x; hv[u][1] = p.y; hv[u][2] = p.z; hv[u][3] = p.w;
                        hv[u][4] = q.x; hv[u][5] = q.y; hv[u][6] = q.z; hv[u][7] = q.w;
                    } else {
#pragma unroll
                        for (int i = 0; i < 8; ++i) hv[u][i] = 0.f;
                    }
                    wv[u] = *reinterpret_cast<const uint2 *>(wrow + kc * 32);
                    if (FMT == W_Q8_0) sc[u] = half_bits_to_float(qs[kc]);
                }
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    if (kb + u < nb) {
                        bf16x8 a[2];
                        split_f32x8<2>(hv[u], a);
                        const bf16x8 b = i8x8_to_bf16x8(wv[u].x, wv[u].y);
                        if (FMT == W_Q8_0) {
                            f32x4 c = mfma16x16x32_bf16(a[0], b, zero4());
                            c = mfma16x16x32_bf16(a[1], b, c);
                            acc += c * sc[u];
                        } else {
                            acc = mfma16x16x32_bf16(a[0], b, acc);
                            acc = mfma16x16x32_bf16(a[1], b, acc);
                        }
                    }
                }
            }
            if (FMT == W_I8_ROW) acc *= reinterpret_cast<const float *>(wd_scales)[wr];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int m = m0 + 4 * lg + i;
                if (m < n_e) {
                    if (FUSED)
                        y_lds[(row0 + m) * 16 + li] = acc[i];
                    else
                        ybuf[(size_t)(row0 + m) * d + o0 + li] = acc[i];
                }
            }
        }
    }
    if (FUSED) {
        __syncthreads();
        for (int i = threadIdx.x; i < T * 16; i += 64 * NW) {
            const int t = i >> 4, n = i & 15;
            float a = 0.f;
            for (int j = 0; j < k; ++j) {
                const int p = t * k + j;
                a += topk_w[p] * y_lds[inv[p] * 16 + n];
            }
            out[(size_t)t * d + o0 + n] = a;
        }
    }
}

// out[t][o] = sum_j w[t][j] * sum_c ybuf[(inv[t*k+j] * nchunk + c) * d + o], in that order.
__global__ __launch_bounds__(256) void combine_rows_kernel(const float *__restrict__ ybuf,
                                                           const int32_t *__restrict__ inv,
                                                           const float *__restrict__ topk_w, int k,
                                                           int d, int nchunk,
                                                           float *__restrict__ out)
{
    const int t = blockIdx.y;
    const int o = blockIdx.x * 256 + threadIdx.x;
    if (o >= d) return;
    float a = 0.f;
    for (int j = 0; j < k; ++j) {
        const int p = t * k + j;
        const float *yr = ybuf + (size_t)inv[p] * nchunk * d + o;
        float y = 0.f;
        for (int c = 0; c < nchunk; ++c) y += yr[(size_t)c * d];
        a += topk_w[p] * y;
    }
    out[(size_t)t * d + o] = a;
}

// ------------------------------------------------------------------------------------------

template <int FMT, int ACT, int XT>
static void launch_gateup_t(dim3 g, hipStream_t s, const void *x, int d, int k, const ExpertsDev &ex,
                            const PermuteOut &po, float *h)
{
    hipLaunchKernelGGL((gateup_int8_kernel<FMT, ACT, XT, 4, 4>), g, dim3(256), 0, s, x, d, k,
                       reinterpret_cast<const int8_t *>(ex.gate_up), ex.gate_up_scales, ex.d_ff,
                       po.offsets, po.perm, po.active, po.n_active, h);
}

hipError_t launch_gateup_int8(const void *x, int xtype, int T, int k, const ExpertsDev &ex, int act,
                              const PermuteOut &po, float *h, hipStream_t s)
{
    const int max_slots = min(ex.E, T * k);
    const dim3 g(max_slots * (ex.d_ff / 16));
    const int d = ex.d_model;
    ProfScope ps(K_GATEUP_I8, s);
#define GU(F, A, X) launch_gateup_t<F, A, X>(g, s, x, d, k, ex, po, h)
    if (ex.fmt == W_Q8_0) {
        if (act == ACT_SWIGLU) { if (xtype == X_BF16) GU(W_Q8_0, ACT_SWIGLU, X_BF16); else GU(W_Q8_0, ACT_SWIGLU, X_F32); }
        else { if (xtype == X_BF16) GU(W_Q8_0, ACT_RELU2, X_BF16); else GU(W_Q8_0, ACT_RELU2, X_F32); }
    } else {
        if (act == ACT_SWIGLU) { if (xtype == X_BF16) GU(W_I8_ROW, ACT_SWIGLU, X_BF16); else GU(W_I8_ROW, ACT_SWIGLU, X_F32); }
        else { if (xtype == X_BF16) GU(W_I8_ROW, ACT_RELU2, X_BF16); else GU(W_I8_ROW, ACT_RELU2, X_F32); }
    }
#undef GU
    return hipGetLastError();
}

template <int FMT, int NW>
static void launch_down_t(hipStream_t s, const float *h, const ExpertsDev &ex, int T, int k,
                          const PermuteOut &po, const float *topk_w, float *out, float *ybuf)
{
    const dim3 g(ex.d_model / 16);
    const int P = T * k;
    const int8_t *wd = reinterpret_cast<const int8_t *>(ex.down);
    if (P <= FUSED_COMBINE_MAX_P)
        hipLaunchKernelGGL((down_int8_kernel<FMT, NW, 4, true>), g, dim3(64 * NW),
                           (size_t)P * 16 * sizeof(float), s, h, ex.d_ff, wd, ex.down_scales,
                           ex.d_model, po.offsets, po.active, po.n_active, po.inv, topk_w, T, k,
                           out, nullptr);
    else
        hipLaunchKernelGGL((down_int8_kernel<FMT, NW, 4, false>), g, dim3(64 * NW), 0, s, h,
                           ex.d_ff, wd, ex.down_scales, ex.d_model, po.offsets, po.active,
                           po.n_active, po.inv, topk_w, T, k, out, ybuf);
}

hipError_t launch_down_int8(const float *h, const ExpertsDev &ex, int T, int k,
                            const PermuteOut &po, const float *topk_w, float *out, float *ybuf,
                            hipStream_t s)
{
    const int max_slots = min(ex.E, T * k);
    const int nw = max_slots <= 4 ? 4 : (max_slots <= 8 ? 8 : 16);
    {
    ProfScope ps(K_DOWN_I8, s);
    if (ex.fmt == W_Q8_0) {
        if (nw == 4) launch_down_t<W_Q8_0, 4>(s, h, ex, T, k, po, topk_w, out, ybuf);
        else if (nw == 8) launch_down_t<W_Q8_0, 8>(s, h, ex, T, k, po, topk_w, out, ybuf);
        else launch_down_t<W_Q8_0, 16>(s, h, ex, T, k, po, topk_w, out, ybuf);
    } else {
        if (nw == 4) launch_down_t<W_I8_ROW, 4>(s, h, ex, T, k, po, topk_w, out, ybuf);
        else if (nw == 8) launch_down_t<W_I8_ROW, 8>(s, h, ex, T, k, po, topk_w, out, ybuf);
        else launch_down_t<W_I8_ROW, 16>(s, h, ex, T, k, po, topk_w, out, ybuf);
    }
    }
    hipError_t err = hipGetLastError();
    if (err != hipSuccess || T * k <= FUSED_COMBINE_MAX_P) return err;
    return launch_combine_rows(ybuf, po.inv, topk_w, T, k, ex.d_model, 1, out, s);
}

hipError_t launch_combine_rows(const float *ybuf, const int32_t *inv, const float *topk_w, int T,
                               int k, int d, int nchunk, float *out, hipStream_t s)
{
    ProfScope ps(K_COMBINE, s);
    hipLaunchKernelGGL(combine_rows_kernel, dim3((d + 255) / 256, T), dim3(256), 0, s, ybuf, inv,
                       topk_w, k, d, nchunk, out);
    return hipGetLastError();
}

}  // namespace moe
