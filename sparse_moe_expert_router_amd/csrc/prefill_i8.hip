// Batched-prefill path with int8 activations on the gfx950 int8 matrix cores.
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
