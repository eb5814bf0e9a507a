// Device helpers shared by the gfx950 kernels of the MoE layer library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// Matrix-core operand and accumulator types (gfx950 builtins).
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(2 * sizeof(float)))) float f32x2;
typedef __attribute__((__vector_size__(4 * sizeof(int)))) int i32x4;

enum { X_F32 = 0, X_BF16 = 1 };
enum { W_Q8_0 = 0, W_I8_ROW = 1, W_E2M1 = 2, W_Q8_0_TILED = 3, W_I8_ROW_TILED = 4 };
enum { L_PLAIN = 0, L_TILED = 1 };
enum { ACT_SWIGLU = 0, ACT_RELU2 = 1 };

constexpr int WAVE = 64;

union U4 {
    uint4 u;
    uint32_t w[4];
    bf16x8 v;
};

__device__ __forceinline__ float half_bits_to_float(uint16_t h)
{
    return (float)__builtin_bit_cast(_Float16, h);
}

// int8 byte `b` of `w` as an exact float.
__device__ __forceinline__ float i8_to_f32(uint32_t w, int b)
{
    return (float)((int32_t)(w << (24 - 8 * b)) >> 24);
}

// Two floats that are exactly representable in bf16 (|int8| values, E2M1 values, ...) packed as
// bf16x2: the upper halves of their fp32 encodings, `lo` in bits 0..15.
__device__ __forceinline__ uint32_t pack_bf16_exact(float lo, float hi)
{
    return __builtin_amdgcn_perm(__float_as_uint(hi), __float_as_uint(lo), 0x07060302u);
}

// Eight int8 (two little-endian words, element 0 in the low byte of w0) as an exact bf16x8.
__device__ __forceinline__ bf16x8 i8x8_to_bf16x8(uint32_t w0, uint32_t w1)
{
    U4 r;
    r.w[0] = pack_bf16_exact(i8_to_f32(w0, 0), i8_to_f32(w0, 1));
    r.w[1] = pack_bf16_exact(i8_to_f32(w0, 2), i8_to_f32(w0, 3));
    r.w[2] = pack_bf16_exact(i8_to_f32(w1, 0), i8_to_f32(w1, 1));
    r.w[3] = pack_bf16_exact(i8_to_f32(w1, 2), i8_to_f32(w1, 3));
    return r.v;
}

// fp32 -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f)
{
    uint32_t u = __float_as_uint(f);
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b)
{
    return __uint_as_float(b << 16);
}

// Split eight fp32 values into NT bf16x8 terms whose sum approximates them: with NT = 3 the sum
// is exact for every normal fp32 (8 + 8 + 8 significant bits), with NT = 2 the residual is below
// 2^-17 relative.  Products of the terms with exact bf16 weights are exact in fp32.
template <int NT>
__device__ __forceinline__ void split_f32x8(const float *v, bf16x8 *terms)
{
    float r[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) r[i] = v[i];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        U4 o;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            uint32_t b0 = f32_to_bf16_rne(r[2 * i]), b1 = f32_to_bf16_rne(r[2 * i + 1]);
            o.w[i] = b0 | (b1 << 16);
            r[2 * i] -= bf16_bits_to_f32(b0);
            r[2 * i + 1] -= bf16_bits_to_f32(b1);
        }
        terms[t] = o.v;
    }
}

__device__ __forceinline__ f32x4 mfma16x16x32_bf16(bf16x8 a, bf16x8 b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 zero4()
{
    f32x4 z = {0.f, 0.f, 0.f, 0.f};
    return z;
}

__device__ __forceinline__ float silu_f32(float g)
{
    return g / (1.0f + expf(-g));
}

template <typename Tv>
__device__ __forceinline__ Tv wave_sum(Tv v)
{
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, WAVE);
    return v;
}

__device__ __forceinline__ int clamp_id(int e, int E)
{
    return e < 0 ? 0 : (e >= E ? E - 1 : e);
}

}  // namespace moe
