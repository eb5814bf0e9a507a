// Diagnostics: the intermediate activations a layer call leaves in its workspace, copied out in
// pair order (row t k + j for slot j of token t, then row P + s T + t for shared expert s).
// Not on the layer's path; used to count the realized zero-skip groups and to compare h and its
// prefill codes with a reference element by element.
#include "moe_common.hpp"
#include "moe_launch.hpp"

namespace moe {

// Destination row of permuted row r: the pair it holds (routed rows), or r itself (shared rows).
__device__ __forceinline__ int pair_row(const int32_t *__restrict__ perm, int r, int P)
{
    return r < P ? min(max(perm[r], 0), P - 1) : r;
}

// One block per permuted row.  h32 != nullptr: fp32 h; otherwise the two bf16 planes, summed.
__global__ __launch_bounds__(256) void unpermute_h_kernel(const float *__restrict__ h32,
                                                          const uint16_t *__restrict__ h_hi,
                                                          const uint16_t *__restrict__ h_lo,
                                                          const int32_t *__restrict__ perm, int P, int d_ff,
                                                          float *__restrict__ out)
{
    const int r = blockIdx.x;
    const size_t src = (size_t)r * d_ff, dst = (size_t)pair_row(perm, r, P) * d_ff;
    for (int c = threadIdx.x; c < d_ff; c += blockDim.x)
        out[dst + c] = h32 ? h32[src + c] : bf16_bits_to_f32(h_hi[src + c]) + bf16_bits_to_f32(h_lo[src + c]);
}

// One block per 128-row tile of the down GEMM's A operand (see quantize_h_tiles_kernel for the
// layout): each 16-byte slot goes back to its row's columns 8g .. 8g+7 and 32+8g .. 32+8g+7 of
// its 64-column block; the row scales follow their rows.
__global__ __launch_bounds__(256) void untile_hq_kernel(const int8_t *__restrict__ q, const float *__restrict__ sh,
                                                        const int4 *__restrict__ tiles,
                                                        const int32_t *__restrict__ tile_off, int E,
                                                        const int32_t *__restrict__ perm, int P, int d_ff,
                                                        int8_t *__restrict__ out_q, float *__restrict__ out_s)
{
    const int mt = blockIdx.x;
    if (mt >= tile_off[E]) return;
    const int4 rec = tiles[mt];
    const int S = d_ff >> 6;
    const int n = rec.z * S * 4;                     // 16-byte slots of this tile's rows
    for (int i = threadIdx.x; i < n; i += blockDim.x) {
        const int ti = i / (S * 4), rem = i - ti * (S * 4), sb = rem >> 2, g = rem & 3;
        const int row = rec.y + ti;
        const uint4 v = *reinterpret_cast<const uint4 *>(
            q + ((size_t)mt * S + sb) * 8192 + (size_t)(64 * (ti >> 4) + 16 * g + (ti & 15)) * 16);
        int8_t *d = out_q + (size_t)pair_row(perm, row, P) * d_ff + sb * 64 + 8 * g;
        *reinterpret_cast<uint2 *>(d) = make_uint2(v.x, v.y);
        *reinterpret_cast<uint2 *>(d + 32) = make_uint2(v.z, v.w);
    }
    for (int ti = threadIdx.x; ti < rec.z; ti += blockDim.x) {
        const int row = rec.y + ti;
        out_s[pair_row(perm, row, P)] = sh[row];
    }
}

hipError_t launch_unpermute_h(const float *h32, const uint16_t *h_hi, const uint16_t *h_lo, const int32_t *perm,
                              int P, int rows, int d_ff, float *out, hipStream_t s)
{
    hipLaunchKernelGGL(unpermute_h_kernel, dim3(rows), dim3(256), 0, s, h32, h_hi, h_lo, perm, P, d_ff, out);
    return hipGetLastError();
}

hipError_t launch_untile_hq(const int8_t *q, const float *sh, const PermuteOut &po, int E, int tile_bound, int P,
                            int d_ff, int8_t *out_q, float *out_s, hipStream_t s)
{
    hipLaunchKernelGGL(untile_hq_kernel, dim3(tile_bound), dim3(256), 0, s, q, sh, po.tiles, po.tile_off, E,
                       po.perm, P, d_ff, out_q, out_s);
    return hipGetLastError();
}

}  // namespace moe
