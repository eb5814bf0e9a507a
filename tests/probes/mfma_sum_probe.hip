// Test-only numerics probe of two gfx950 matrix-core instructions (not part of the library): each
// runs one wave of one MFMA whose every output is the sum 256 + a over one row of A against
// B = 1, so the exact result is known.  v_mfma_scale_f32_32x32x64_f8f6f4 takes E4M3 codes (scale
// exponents 127, i.e. 1.0) and v_mfma_f32_32x32x16_f16 takes f16 values; A's row i (lanes 0..31)
// holds 256 and a in its first two K slots, zeros elsewhere; lanes 32..63 hold zeros.
#include <hip/hip_runtime.h>

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));

__global__ __launch_bounds__(64) void f8f6f4_kernel(float *out, int addend_code)
{
    const int lane = threadIdx.x;
    v8i a = {0, 0, 0, 0, 0, 0, 0, 0}, b;
#pragma unroll
    for (int i = 0; i < 8; ++i) b[i] = 0x38383838;          // E4M3 1.0 in every code
    if (lane < 32) a[0] = 0x78 | ((addend_code & 0xFF) << 8);  // codes 0, 1: 256 and the addend
    v16f c = {};
    c = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
#pragma unroll
    for (int i = 0; i < 16; ++i) out[lane * 16 + i] = c[i];
}

__global__ __launch_bounds__(64) void f16_kernel(float *out, float addend)
{
    const int lane = threadIdx.x;
    h8 a = {}, b;
#pragma unroll
    for (int i = 0; i < 8; ++i) b[i] = (_Float16)1.0f;
    if (lane < 32) {
        a[0] = (_Float16)256.0f;
        a[1] = (_Float16)addend;
    }
    v16f c = {};
    c = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
#pragma unroll
    for (int i = 0; i < 16; ++i) out[lane * 16 + i] = c[i];
}

}  // namespace

// kind 0: the E4M3 instruction with addend code `addend_code`; kind 1: the f16 instruction with
// `addend`.  Writes the 64 x 16 results to host_out (1024 floats).  Returns 0, or the HIP error.
extern "C" int mfma_sum_probe(int kind, int addend_code, float addend, float *host_out)
{
    float *d = nullptr;
    hipError_t e = hipMalloc(&d, 1024 * sizeof(float));
    if (e != hipSuccess) return (int)e;
    if (kind == 0) hipLaunchKernelGGL(f8f6f4_kernel, dim3(1), dim3(64), 0, 0, d, addend_code);
    else hipLaunchKernelGGL(f16_kernel, dim3(1), dim3(64), 0, 0, d, addend);
    e = hipGetLastError();
    if (e == hipSuccess) e = hipMemcpy(host_out, d, 1024 * sizeof(float), hipMemcpyDeviceToHost);
    hipFree(d);
    return (int)e;
}
