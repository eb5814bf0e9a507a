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

// K -> lane mapping shared by A and B: in each 64-wide super-block s, lane (n, g) owns K offsets
// 8g..8g+7 and 32+8g..32+8g+7 of its row (the tiled weight layout's slice), as one int8x16.
__device__ __forceinline__ i32x4v load_row16(const int8_t *row, int s, int g)
{
    const uint2 a = *reinterpret_cast<const uint2 *>(row + 64 * s + 8 * g);
    const uint2 b = *reinterpret_cast<const uint2 *>(row + 64 * s + 32 + 8 * g);
    i32x4v v = {(int)a.x, (int)a.y, (int)b.x, (int)b.y};
    return v;
}

__device__ __forceinline__ i32x4v load_tile16(const int8_t *tile_lane)
{
    const uint4 a = *reinterpret_cast<const uint4 *>(tile_lane);
    i32x4v v = {(int)a.x, (int)a.y, (int)a.z, (int)a.w};
    return v;
}

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

// Gate/up: block = (N-tile nt of 64 gate + the same 64 up columns, global M-tile); 4 waves, wave
// (wm, wn) owns rows 64wm..64wm+63 and gate/up columns f0 + 32wn .. +31.  Epilogue:
// g = sx[tok] * s_gate[f] * acc, u likewise, h = silu(g) * u in fp32, written in permuted order.
template <int LAYOUT>
__global__ __launch_bounds__(256) void ggemm_gateup_i8_kernel(
    const int8_t *__restrict__ xq, const float *__restrict__ sx, int d, int k,
    const int8_t *__restrict__ wgu, const float *__restrict__ wscale, int d_ff,
    const int32_t *__restrict__ offsets, const int32_t *__restrict__ perm,
    const int32_t *__restrict__ tile_off, int E, int mt_bound, float *__restrict__ h)
{
    const int logical = xcd_logical_block();
    const int nt = logical / mt_bound, mt = logical - nt * mt_bound;
    if (mt >= tile_off[E]) return;
    const int e = expert_of_tile(tile_off, E, mt);
    const int r_begin = offsets[e] + (mt - tile_off[e]) * GG_BM;
    const int rows = min(GG_BM, offsets[e + 1] - r_begin);
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int wm = wave >> 1, wn = wave & 1;
    const int li = lane & 15, lg = lane >> 4;
    const int S = d >> 6;
    const int NTt = d_ff >> 4;
    const int fbase = nt * 64 + 32 * wn;             // first gate column of this wave

    const int8_t *arow[4];
    bool aval[4];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
        const int r = 64 * wm + 16 * rt + li;
        aval[rt] = r < rows;
        const int tok = aval[rt] ? perm[r_begin + r] / k : 0;
        arow[rt] = xq + (size_t)tok * d;
    }
    // B: 2 column tiles x {gate, up}
    const int8_t *bptr[2][2];
#pragma unroll
    for (int ct = 0; ct < 2; ++ct)
#pragma unroll
        for (int m = 0; m < 2; ++m) {
            const int t = (fbase >> 4) + ct;
            if (LAYOUT == L_TILED)
                bptr[ct][m] = wgu + ((((size_t)e * NTt + t) * S) * 2 + m) * 1024 + lane * 16;
            else
                bptr[ct][m] = wgu + ((size_t)e * 2 * d_ff + m * d_ff + 16 * t + li) * d;
        }
    i32x4v acc[4][2][2];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
        for (int ct = 0; ct < 2; ++ct)
#pragma unroll
            for (int m = 0; m < 2; ++m) acc[rt][ct][m] = i32x4v{0, 0, 0, 0};

    for (int s = 0; s < S; ++s) {
        i32x4v a[4], b[2][2];
#pragma unroll
        for (int rt = 0; rt < 4; ++rt)
            a[rt] = aval[rt] ? load_row16(arow[rt], s, lg) : i32x4v{0, 0, 0, 0};
#pragma unroll
        for (int ct = 0; ct < 2; ++ct)
#pragma unroll
            for (int m = 0; m < 2; ++m)
                b[ct][m] = LAYOUT == L_TILED ? load_tile16(bptr[ct][m] + (size_t)s * 2048)
                                             : load_row16(bptr[ct][m], s, lg);
#pragma unroll
        for (int rt = 0; rt < 4; ++rt)
#pragma unroll
            for (int ct = 0; ct < 2; ++ct)
#pragma unroll
                for (int m = 0; m < 2; ++m)
                    acc[rt][ct][m] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[rt], b[ct][m], acc[rt][ct][m], 0, 0, 0);
    }
    // epilogue: lane holds C[row 4*lg + i][col li] of each 16x16 tile
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = 64 * wm + 16 * rt + 4 * lg + i;
            if (r < rows) {
                const int row = r_begin + r;
                const float s_x = sx[perm[row] / k];
#pragma unroll
                for (int ct = 0; ct < 2; ++ct) {
                    const int f = fbase + 16 * ct + li;
                    const float g = (float)acc[rt][ct][0][i] * s_x * wscale[(size_t)e * 2 * d_ff + f];
                    const float u = (float)acc[rt][ct][1][i] * s_x * wscale[(size_t)e * 2 * d_ff + d_ff + f];
                    h[(size_t)row * d_ff + f] = silu_f32(g) * u;
                }
            }
        }
}

// Down: block = (N-tile of 128 outputs, global M-tile); wave (wm, wn) owns rows 64wm.. and
// outputs n0 + 64wn .. +63.  y = s_h[row] * s_down[o] * acc, fp32, per pair row.
template <int LAYOUT>
__global__ __launch_bounds__(256) void ggemm_down_i8_kernel(
    const int8_t *__restrict__ hq, const float *__restrict__ sh, int d_ff,
    const int8_t *__restrict__ wd, const float *__restrict__ wscale, int d,
    const int32_t *__restrict__ offsets, const int32_t *__restrict__ tile_off, int E, int mt_bound,
    float *__restrict__ ybuf)
{
    const int logical = xcd_logical_block();
    const int nt = logical / mt_bound, mt = logical - nt * mt_bound;
    if (mt >= tile_off[E]) return;
    const int e = expert_of_tile(tile_off, E, mt);
    const int r_begin = offsets[e] + (mt - tile_off[e]) * GG_BM;
    const int rows = min(GG_BM, offsets[e + 1] - r_begin);
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int wm = wave >> 1, wn = wave & 1;
    const int li = lane & 15, lg = lane >> 4;
    const int n0 = nt * 128 + 64 * wn;
    if (n0 >= d) return;                             // waves are independent: no block barrier
    const int S = d_ff >> 6;
    const int OT = d >> 4;

    const int8_t *arow[4];
    bool aval[4];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
        const int r = 64 * wm + 16 * rt + li;
        aval[rt] = r < rows;
        arow[rt] = hq + (size_t)(r_begin + (aval[rt] ? r : 0)) * d_ff;
    }
    const int8_t *bptr[4];
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
        const int ot = (n0 >> 4) + ct;
        if (LAYOUT == L_TILED)
            bptr[ct] = wd + (((size_t)e * OT + ot) * S) * 1024 + lane * 16;
        else
            bptr[ct] = wd + ((size_t)e * d + 16 * ot + li) * d_ff;
    }
    i32x4v acc[4][4];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) acc[rt][ct] = i32x4v{0, 0, 0, 0};
    for (int s = 0; s < S; ++s) {
        i32x4v a[4], b[4];
#pragma unroll
        for (int rt = 0; rt < 4; ++rt)
            a[rt] = aval[rt] ? load_row16(arow[rt], s, lg) : i32x4v{0, 0, 0, 0};
#pragma unroll
        for (int ct = 0; ct < 4; ++ct)
            b[ct] = LAYOUT == L_TILED ? load_tile16(bptr[ct] + (size_t)s * 1024) : load_row16(bptr[ct], s, lg);
#pragma unroll
        for (int rt = 0; rt < 4; ++rt)
#pragma unroll
            for (int ct = 0; ct < 4; ++ct)
                acc[rt][ct] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[rt], b[ct], acc[rt][ct], 0, 0, 0);
    }
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = 64 * wm + 16 * rt + 4 * lg + i;
            if (r < rows) {
                const int row = r_begin + r;
                const float s_h = sh[row];
#pragma unroll
                for (int ct = 0; ct < 4; ++ct) {
                    const int o = n0 + 16 * ct + li;
                    ybuf[(size_t)row * d + o] = (float)acc[rt][ct][i] * s_h * wscale[(size_t)e * d + o];
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
        hipLaunchKernelGGL(ggemm_gateup_i8_kernel<L_TILED>, g, dim3(256), 0, s, xq, sx, ex.d_model, k, w,
                           sc, ex.d_ff, po.offsets, po.perm, po.tile_off, ex.E, mtb, h);
    else
        hipLaunchKernelGGL(ggemm_gateup_i8_kernel<L_PLAIN>, g, dim3(256), 0, s, xq, sx, ex.d_model, k, w,
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
        hipLaunchKernelGGL(ggemm_down_i8_kernel<L_TILED>, g, dim3(256), 0, s, hq, sh, ex.d_ff, w, sc,
                           ex.d_model, po.offsets, po.tile_off, ex.E, mtb, ybuf);
    else
        hipLaunchKernelGGL(ggemm_down_i8_kernel<L_PLAIN>, g, dim3(256), 0, s, hq, sh, ex.d_ff, w, sc,
                           ex.d_model, po.offsets, po.tile_off, ex.E, mtb, ybuf);
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
