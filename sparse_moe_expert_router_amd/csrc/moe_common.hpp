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
enum { W_Q8_0 = 0, W_I8_ROW = 1, W_E2M1 = 2, W_Q8_0_TILED = 3, W_I8_ROW_TILED = 4, W_FP8_ROW = 5, W_FP8_ROW_TILED = 6 };
enum { L_PLAIN = 0, L_TILED = 1 };
enum { ACT_SWIGLU = 0, ACT_RELU2 = 1 };

constexpr int WAVE = 64;

union U4 {
    uint4 u;
    uint32_t w[4];
    bf16x8 v;
};

// Loads of expert weights and their scales in the decode kernels: each byte is read once per
// layer call, so where a wave's load covers whole 128-byte lines the loads carry the non-temporal
// hint (the caches stream them instead of keeping them, leaving room for the activations, h and
// routing records that are read again).  Measured against plain loads, 30 distinct Gemma-shaped
// Q8_0 layers at T = 8: 108.5k -> 115.1k tokens/s; MiniMax-M3-shaped T = 32: gate/up 476 -> 429 us
// (6.7 TB/s).  A plain streaming read reaches 6.0 TB/s with plain and 6.6 TB/s with these loads.
typedef unsigned int u32x4e __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2e __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint4 ld_stream16(const void *p)
{
    const u32x4e v = __builtin_nontemporal_load(reinterpret_cast<const u32x4e *>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint2 ld_stream8(const void *p)
{
    const u32x2e v = __builtin_nontemporal_load(reinterpret_cast<const u32x2e *>(p));
    return make_uint2(v.x, v.y);
}
__device__ __forceinline__ uint32_t ld_stream4(const void *p)
{
    return __builtin_nontemporal_load(reinterpret_cast<const uint32_t *>(p));
}

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

// ---- exchanges inside one wavefront without LDS (DPP row patterns and the gfx950 permlane swaps)

// the value of lane l's partner under a DPP row pattern: 0xB1 = l ^ 1, 0x4E = l ^ 2 (quad_perm),
// 0x141 = 7 - l within 8 (row_half_mirror), 0x140 = 15 - l within 16 (row_mirror)
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v)
{
    return __builtin_amdgcn_update_dpp(0u, v, CTRL, 0xF, 0xF, false);
}

template <int CTRL>
__device__ __forceinline__ uint64_t dpp_u64(uint64_t v)
{
    return (uint64_t)dpp_u32<CTRL>((uint32_t)v) | ((uint64_t)dpp_u32<CTRL>((uint32_t)(v >> 32)) << 32);
}

// Value of lane (lane ^ stride), stride a power of two <= 32 known at compile time after
// unrolling: DPP for strides up to 8 (4 = half-row mirror then quad reverse, 8 = row mirror then
// half-row mirror), the permlane swaps for 16 and 32.  Every lane active.
__device__ __forceinline__ uint32_t xor_lane_u32(uint32_t v, int stride, int lane)
{
    switch (stride) {
    case 1: return dpp_u32<0xB1>(v);
    case 2: return dpp_u32<0x4E>(v);
    case 4: return dpp_u32<0x1B>(dpp_u32<0x141>(v));
    case 8: return dpp_u32<0x141>(dpp_u32<0x140>(v));
    case 16: {
        const auto p = __builtin_amdgcn_permlane16_swap(v, v, false, false);
        return (lane & 16) ? p[0] : p[1];
    }
    default: {
        const auto p = __builtin_amdgcn_permlane32_swap(v, v, false, false);
        return (lane & 32) ? p[0] : p[1];
    }
    }
}

// v_permlane16_swap / v_permlane32_swap with both operands v: element 0 is the value of the lower
// row (half) of the pair {l, l ^ 16} ({l, l ^ 32}), element 1 that of the upper one, on both lanes.
struct Pair64 {
    uint64_t lo, hi;
};

template <int W>
__device__ __forceinline__ Pair64 permlane_pair(uint64_t v)
{
    const uint32_t a = (uint32_t)v, b = (uint32_t)(v >> 32);
    if (W == 16) {
        const auto ra = __builtin_amdgcn_permlane16_swap(a, a, false, false);
        const auto rb = __builtin_amdgcn_permlane16_swap(b, b, false, false);
        return {(uint64_t)ra[0] | ((uint64_t)rb[0] << 32), (uint64_t)ra[1] | ((uint64_t)rb[1] << 32)};
    } else {
        const auto ra = __builtin_amdgcn_permlane32_swap(a, a, false, false);
        const auto rb = __builtin_amdgcn_permlane32_swap(b, b, false, false);
        return {(uint64_t)ra[0] | ((uint64_t)rb[0] << 32), (uint64_t)ra[1] | ((uint64_t)rb[1] << 32)};
    }
}

// Wave-wide maximum of a 32-bit unsigned value; every lane receives it.  Call with every lane active.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v)
{
    uint32_t o;
    o = dpp_u32<0xB1>(v); v = o > v ? o : v;
    o = dpp_u32<0x4E>(v); v = o > v ? o : v;
    o = dpp_u32<0x141>(v); v = o > v ? o : v;
    o = dpp_u32<0x140>(v); v = o > v ? o : v;
    auto p = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    v = p[0] > p[1] ? p[0] : p[1];
    p = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    v = p[0] > p[1] ? p[0] : p[1];
    return v;
}

// Wave-wide maximum of a 64-bit unsigned key; every lane receives it.  Call with every lane active.
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v)
{
    uint64_t o;
    o = dpp_u64<0xB1>(v); v = o > v ? o : v;
    o = dpp_u64<0x4E>(v); v = o > v ? o : v;
    o = dpp_u64<0x141>(v); v = o > v ? o : v;
    o = dpp_u64<0x140>(v); v = o > v ? o : v;
    Pair64 p = permlane_pair<16>(v); v = p.lo > p.hi ? p.lo : p.hi;
    p = permlane_pair<32>(v); v = p.lo > p.hi ? p.lo : p.hi;
    return v;
}

// Wave-wide sum of a double in one fixed order (a butterfly; both lanes of each exchange add the
// same two operands, so every lane ends with the same bits).  Call with every lane active.
__device__ __forceinline__ double wave_sum_f64(double v)
{
    auto f = [](uint64_t u) { return __builtin_bit_cast(double, u); };
    auto u = [](double d) { return __builtin_bit_cast(uint64_t, d); };
    v += f(dpp_u64<0xB1>(u(v)));
    v += f(dpp_u64<0x4E>(u(v)));
    v += f(dpp_u64<0x141>(u(v)));
    v += f(dpp_u64<0x140>(u(v)));
    Pair64 p = permlane_pair<16>(u(v)); v = f(p.lo) + f(p.hi);
    p = permlane_pair<32>(u(v)); v = f(p.lo) + f(p.hi);
    // (the builtin returns a signed int: widen through uint32_t, not by sign extension)
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)u(v));
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(u(v) >> 32));
    return __builtin_bit_cast(double, (uint64_t)lo | ((uint64_t)hi << 32));
}

__device__ __forceinline__ int clamp_id(int e, int E)
{
    return e < 0 ? 0 : (e >= E ? E - 1 : e);
}

}  // namespace moe
