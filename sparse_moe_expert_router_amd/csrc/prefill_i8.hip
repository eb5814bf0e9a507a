// Batched-prefill path with int8 activations on the gfx950 int8 matrix cores (the batched-prefill
// layer definition: x quantised per token, h per (token, slot) pair, int32 accumulation, fp32
// rescale).  Grouped GEMMs over the permuted pairs, one expert group at a time: the gate/up GEMM
// (the mul_mat_id of the Gemma-on-a-Xeon page's "Three-part fix" with its fused silu(gate) * up
// epilogue) and the down GEMM, both on v_mfma_i32_16x16x64_i8.
//
// Activation quantiser (rule Q): per row, a = max|v|; a = 0 gives q = 0 and scale 0; otherwise
// q = clamp(round_half_even(fp32(v * fp32(127 / a))), -127, 127), scale = fp32(a / 127).  Every
// step is one IEEE fp32 operation (correctly rounded division, v_rndne_f32), so the codes are the
// ones any IEEE fp32 implementation of the rule gets.
#include "moe_common.hpp"
#include "moe_launch.hpp"

namespace moe {

template <int XT>
__device__ __forceinline__ void load4(const void *v, size_t i, float *o)
{
    if (XT == X_BF16) {
        const uint2 b = *reinterpret_cast<const uint2 *>(reinterpret_cast<const uint16_t *>(v) + i);
        o[0] = __uint_as_float(b.x << 16);
        o[1] = __uint_as_float(b.x & 0xFFFF0000u);
        o[2] = __uint_as_float(b.y << 16);
        o[3] = __uint_as_float(b.y & 0xFFFF0000u);
    } else {
        const float4 f = *reinterpret_cast<const float4 *>(reinterpret_cast<const float *>(v) + i);
        o[0] = f.x; o[1] = f.y; o[2] = f.z; o[3] = f.w;
    }
}

// One workgroup (256 threads) per row.
template <int XT>
__global__ __launch_bounds__(256) void quantize_rows_kernel(const void *__restrict__ v, int cols,
                                                            int8_t *__restrict__ q,
                                                            float *__restrict__ scale)
{
    __shared__ float s_max[4];
    const size_t base = (size_t)blockIdx.x * cols;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    float a = 0.f;
    for (int i = tid * 4; i < cols; i += 1024) {
        float f[4];
        load4<XT>(v, base + i, f);
        a = fmaxf(a, fmaxf(fmaxf(fabsf(f[0]), fabsf(f[1])), fmaxf(fabsf(f[2]), fabsf(f[3]))));
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) a = fmaxf(a, __shfl_xor(a, off, WAVE));
    if (lane == 0) s_max[wave] = a;
    __syncthreads();
    a = fmaxf(fmaxf(s_max[0], s_max[1]), fmaxf(s_max[2], s_max[3]));
    const float inv = a > 0.f ? 127.0f / a : 0.f;
    for (int i = tid * 4; i < cols; i += 1024) {
        float f[4];
        load4<XT>(v, base + i, f);
        uint32_t packed = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            float r = __builtin_rintf(f[j] * inv);
            r = fminf(fmaxf(r, -127.f), 127.f);
            packed |= ((uint32_t)(int32_t)r & 0xFFu) << (8 * j);
        }
        *reinterpret_cast<uint32_t *>(q + base + i) = packed;
    }
    if (tid == 0) scale[blockIdx.x] = a / 127.0f;
}

// ------------------------------------------------------------------------------------------
// Grouped int8 GEMMs
// ------------------------------------------------------------------------------------------

typedef __attribute__((__vector_size__(4 * sizeof(int)))) int i32x4v;

// Expert of global M-tile mt: the largest e with tile_off[e] <= mt.
__device__ __forceinline__ int expert_of_tile(const int32_t *tile_off, int E, int mt)
{
    int lo = 0, hi = E - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (tile_off[mid] <= mt) lo = mid;
        else hi = mid - 1;
    }
    return lo;
}

// Logical block id: consecutive logical ids run on the same XCD (blocks are dealt to the 8 XCDs
// round robin), so the M-tiles of one (expert, N-tile) share that XCD's L2.
__device__ __forceinline__ int xcd_logical_block()
{
    const int b = blockIdx.x, G = gridDim.x;
    if (G & 7) return b;
    return (b & 7) * (G >> 3) + (b >> 3);
}

constexpr int GG_BM = 128;

// Grouped int8 GEMM over the permuted pairs of one expert group per block.
//  MODE_GU (gate/up): block = (N-tile nt: gate columns 64nt..64nt+63 and the same up columns,
//           global M-tile); A = quantised x rows gathered through perm, K = d_model; epilogue
//           g = sx * s_gate * acc, u likewise, h = silu(g) * u (fp32, permuted row order).
//  MODE_DN (down): block = (N-tile of 128 outputs, global M-tile); A = quantised h rows (already
//           in permuted order), K = d_ff; epilogue y = sh * s_down * acc (fp32 per pair row).
// Block tile 128 x 128, K step 64, 4 waves as 2 x 2 tiles of 64 x 64 (16 MFMAs per step each).
// Each K step's A (128 x 64 B) and B (8 tiles of 16 x 64 B) go through LDS, double buffered;
// LDS holds them in the lane order the MFMA consumes (lane (n, g) of a 16-row tile owns K offsets
// 8g..8g+7 and 32+8g..32+8g+7 of row n, 16 bytes), so every fragment is one ds_read_b128 and the
// tiled weight layout is copied as is.
enum { MODE_GU = 0, MODE_DN = 1 };

template <int MODE, int LAYOUT>
__global__ __launch_bounds__(256) void ggemm_i8_kernel(
    const int8_t *__restrict__ A, const float *__restrict__ a_scale, int K, int k,
    const int8_t *__restrict__ W, const float *__restrict__ w_scale, int NR,
    const int32_t *__restrict__ offsets, const int32_t *__restrict__ perm,
    const int32_t *__restrict__ tile_off, int E, int mt_bound, float *__restrict__ out)
{
    __shared__ __attribute__((aligned(16))) int8_t lds[2][16384];
    const int logical = xcd_logical_block();
    const int nt = logical / mt_bound, mt = logical - nt * mt_bound;
    if (mt >= tile_off[E]) return;                   // uniform across the block
    const int e = expert_of_tile(tile_off, E, mt);
    const int r_begin = offsets[e] + (mt - tile_off[e]) * GG_BM;
    const int rows = min(GG_BM, offsets[e + 1] - r_begin);
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int wm = wave >> 1, wn = wave & 1;
    const int li = lane & 15, lg = lane >> 4;
    const int S = K >> 6;
    // NR = d_ff (gate/up) or d_model (down)
    const int OT = NR >> 4;                          // 16-row weight tiles per half / per matrix

    // ---- this thread's two A chunks and two B chunks per K step --------------------------------
    const int8_t *a_src[2];
    int a_lds[2][2];                                 // LDS byte offsets of the two 8-byte halves
    bool a_ok[2];
    const int8_t *b_src[2];
    int b_lds[2][2];
    bool b_ok[2];
#pragma unroll
    for (int c2 = 0; c2 < 2; ++c2) {
        const int c = tid + 256 * c2;
        // A chunk: row r, 16-byte part p of the 64-byte K step
        const int r = c >> 2, p = c & 3;
        a_ok[c2] = r < rows;
        const int rr = a_ok[c2] ? r : 0;
        if (MODE == MODE_GU)
            a_src[c2] = A + (size_t)(perm[r_begin + rr] / k) * K + 16 * p;
        else
            a_src[c2] = A + (size_t)(r_begin + rr) * K + 16 * p;
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
            const int g = 2 * (p & 1) + hh, which = p >> 1;
            a_lds[c2][hh] = (((r >> 4) * 4 + g) * 16 + (r & 15)) * 16 + 8 * which;
        }
        // B chunk: tile j of the block's 8, slice q of 64
        const int j = c >> 6, q = c & 63;
        int wrow_tile;                               // global 16-row weight tile index
        int half_off = 0;                            // gate/up half
        if (MODE == MODE_GU) {
            wrow_tile = 4 * nt + (j & 3);
            half_off = j >> 2;
            b_ok[c2] = true;
        } else {
            wrow_tile = 8 * nt + j;
            b_ok[c2] = wrow_tile < OT;
            if (!b_ok[c2]) wrow_tile = 0;
        }
        if (LAYOUT == L_TILED) {
            const int M = MODE == MODE_GU ? 2 : 1;
            b_src[c2] = W + ((((size_t)e * OT + wrow_tile) * S) * M + half_off) * 1024 + q * 16;
            b_lds[c2][0] = j * 1024 + q * 16;
            b_lds[c2][1] = b_lds[c2][0] + 8;
        } else {
            const int n = q >> 2, pp = q & 3;
            const size_t row = (size_t)e * (MODE == MODE_GU ? 2 * NR : NR) + (size_t)half_off * NR + 16 * wrow_tile + n;
            b_src[c2] = W + row * K + 16 * pp;
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                const int g = 2 * (pp & 1) + hh, which = pp >> 1;
                b_lds[c2][hh] = j * 1024 + (g * 16 + n) * 16 + 8 * which;
            }
        }
    }
    const size_t b_step = LAYOUT == L_TILED ? (MODE == MODE_GU ? 2048 : 1024) : 64;

    uint4 ra[2], rb[2];
    auto gload = [&](int s) {
#pragma unroll
        for (int c2 = 0; c2 < 2; ++c2) {
            ra[c2] = a_ok[c2] ? *reinterpret_cast<const uint4 *>(a_src[c2] + (size_t)s * 64) : make_uint4(0, 0, 0, 0);
            rb[c2] = b_ok[c2] ? *reinterpret_cast<const uint4 *>(b_src[c2] + (size_t)s * b_step) : make_uint4(0, 0, 0, 0);
        }
    };
    auto lstore = [&](int buf) {
        int8_t *L = lds[buf];
#pragma unroll
        for (int c2 = 0; c2 < 2; ++c2) {
            *reinterpret_cast<uint2 *>(L + a_lds[c2][0]) = make_uint2(ra[c2].x, ra[c2].y);
            *reinterpret_cast<uint2 *>(L + a_lds[c2][1]) = make_uint2(ra[c2].z, ra[c2].w);
            if (LAYOUT == L_TILED) {
                *reinterpret_cast<uint4 *>(L + 8192 + b_lds[c2][0]) = rb[c2];
            } else {
                *reinterpret_cast<uint2 *>(L + 8192 + b_lds[c2][0]) = make_uint2(rb[c2].x, rb[c2].y);
                *reinterpret_cast<uint2 *>(L + 8192 + b_lds[c2][1]) = make_uint2(rb[c2].z, rb[c2].w);
            }
        }
    };
    // B tiles this wave multiplies: gate/up: gate tiles 2wn, 2wn+1 and up tiles 4+2wn, 5+2wn;
    // down: tiles 4wn .. 4wn+3.
    int btile[4];
#pragma unroll
    for (int ct = 0; ct < 4; ++ct)
        btile[ct] = MODE == MODE_GU ? ((ct >> 1) * 4 + 2 * wn + (ct & 1)) : (4 * wn + ct);

    i32x4v acc[4][4];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) acc[rt][ct] = i32x4v{0, 0, 0, 0};

    gload(0);
    lstore(0);
    __syncthreads();
    for (int s = 0; s < S; ++s) {
        if (s + 1 < S) gload(s + 1);
        const int8_t *L = lds[s & 1];
        i32x4v a[4], b[4];
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
            const uint4 v = *reinterpret_cast<const uint4 *>(L + (((4 * wm + rt) * 4 + lg) * 16 + li) * 16);
            a[rt] = i32x4v{(int)v.x, (int)v.y, (int)v.z, (int)v.w};
        }
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) {
            const uint4 v = *reinterpret_cast<const uint4 *>(L + 8192 + btile[ct] * 1024 + lane * 16);
            b[ct] = i32x4v{(int)v.x, (int)v.y, (int)v.z, (int)v.w};
        }
#pragma unroll
        for (int rt = 0; rt < 4; ++rt)
#pragma unroll
            for (int ct = 0; ct < 4; ++ct)
                acc[rt][ct] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[rt], b[ct], acc[rt][ct], 0, 0, 0);
        if (s + 1 < S) lstore((s + 1) & 1);
        __syncthreads();
    }

    // ---- epilogue: lane holds C[row 4*lg + i][col li] of each 16 x 16 tile --------------------
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = 64 * wm + 16 * rt + 4 * lg + i;
            if (r >= rows) continue;
            const int row = r_begin + r;
            if (MODE == MODE_GU) {
                const float s_x = a_scale[perm[row] / k];
#pragma unroll
                for (int ct = 0; ct < 2; ++ct) {
                    const int f = 64 * nt + 32 * wn + 16 * ct + li;
                    const float g = (float)acc[rt][ct][i] * s_x * w_scale[(size_t)e * 2 * NR + f];
                    const float u = (float)acc[rt][2 + ct][i] * s_x * w_scale[(size_t)e * 2 * NR + NR + f];
                    out[(size_t)row * NR + f] = silu_f32(g) * u;
                }
            } else {
                const float s_h = a_scale[row];
#pragma unroll
                for (int ct = 0; ct < 4; ++ct) {
                    const int ot = 8 * nt + 4 * wn + ct;
                    if (ot < OT) {
                        const int o = 16 * ot + li;
                        out[(size_t)row * NR + o] = (float)acc[rt][ct][i] * s_h * w_scale[(size_t)e * NR + o];
                    }
                }
            }
        }
}

int prefill_tile_rows() { return GG_BM; }

static int mt_bound_of(int P, int E)
{
    const int b = P / GG_BM + min(E, P);
    return (b + 7) & ~7;
}

hipError_t launch_ggemm_gateup_i8(const int8_t *xq, const float *sx, int T, int k, const ExpertsDev &ex,
                                  const PermuteOut &po, float *h, hipStream_t s)
{
    const int mtb = mt_bound_of(T * k, ex.E);
    const dim3 g(mtb * (ex.d_ff / 64));
    ProfScope ps(K_GG_GATEUP, s);
    const int8_t *w = reinterpret_cast<const int8_t *>(ex.gate_up);
    const float *sc = reinterpret_cast<const float *>(ex.gate_up_scales);
    if (ex.fmt == W_I8_ROW_TILED)
        hipLaunchKernelGGL((ggemm_i8_kernel<MODE_GU, L_TILED>), g, dim3(256), 0, s, xq, sx, ex.d_model, k, w,
                           sc, ex.d_ff, po.offsets, po.perm, po.tile_off, ex.E, mtb, h);
    else
        hipLaunchKernelGGL((ggemm_i8_kernel<MODE_GU, L_PLAIN>), g, dim3(256), 0, s, xq, sx, ex.d_model, k, w,
                           sc, ex.d_ff, po.offsets, po.perm, po.tile_off, ex.E, mtb, h);
    return hipGetLastError();
}

hipError_t launch_ggemm_down_i8(const int8_t *hq, const float *sh, int T, int k, const ExpertsDev &ex,
                                const PermuteOut &po, float *ybuf, hipStream_t s)
{
    const int mtb = mt_bound_of(T * k, ex.E);
    const dim3 g(mtb * ((ex.d_model + 127) / 128));
    ProfScope ps(K_GG_DOWN, s);
    const int8_t *w = reinterpret_cast<const int8_t *>(ex.down);
    const float *sc = reinterpret_cast<const float *>(ex.down_scales);
    if (ex.fmt == W_I8_ROW_TILED)
        hipLaunchKernelGGL((ggemm_i8_kernel<MODE_DN, L_TILED>), g, dim3(256), 0, s, hq, sh, ex.d_ff, k, w, sc,
                           ex.d_model, po.offsets, po.perm, po.tile_off, ex.E, mtb, ybuf);
    else
        hipLaunchKernelGGL((ggemm_i8_kernel<MODE_DN, L_PLAIN>), g, dim3(256), 0, s, hq, sh, ex.d_ff, k, w, sc,
                           ex.d_model, po.offsets, po.perm, po.tile_off, ex.E, mtb, ybuf);
    return hipGetLastError();
}

hipError_t launch_quantize_rows(const void *v, int xtype, int rows, int cols, int8_t *q,
                                float *scale, hipStream_t s)
{
    ProfScope ps(K_QUANT, s);
    if (xtype == X_BF16)
        hipLaunchKernelGGL(quantize_rows_kernel<X_BF16>, dim3(rows), dim3(256), 0, s, v, cols, q, scale);
    else
        hipLaunchKernelGGL(quantize_rows_kernel<X_F32>, dim3(rows), dim3(256), 0, s, v, cols, q, scale);
    return hipGetLastError();
}

}  // namespace moe
