// E2M1 (4-bit, one fp16 scale per 16 values) expert FFN for the Nemotron-style latent MoE
// ("Running NVIDIA's new 120B Nemotron-3.5-Super on an 8 GB GPU", sections "bytes per token" and
// "How the engine works" step 4).
//
// Up: a GEMV per (expert, token) on the vector ALUs.  Each lane takes 16 contiguous bytes (32
// codes = two scale groups) of a row, converts code pairs with v_cvt_scalef32_pk_bf16_fp4 (exact:
// every E2M1 value is a bf16) and multiplies them with the bf16 activations by v_dot2_f32_bf16.
// The per-group fp16 scale is applied once per 16 values.  Rows of a tile are contiguous in
// memory, so a wave's loads cover one contiguous span.
//
// Down: the matrix is neuron-major (neuron f's d_model codes contiguous, scales S[g][o] per group
// of 16 neurons).  With zero-skip a wave reads a 16-neuron group (8 KB of codes + 2 KB of scales
// at d_model = 1024) only when one of its 16 activations is nonzero; skipped groups contribute
// exact zeros, so the result is the dense one bit for bit.  Partial sums over fixed group chunks
// are combined in a fixed order afterwards.
#include "moe_common.hpp"
#include "moe_launch.hpp"

namespace moe {

__device__ __forceinline__ bf16x2 as_bf16x2(uint32_t u)
{
    return __builtin_bit_cast(bf16x2, u);
}

// dot of 8 E2M1 codes (one little-endian word, code 2b in the low nibble of byte b) with 8 bf16
// activations (a uint4, element 2i in the low half of word i).
__device__ __forceinline__ float dot8_e2m1_bf16(uint32_t codes, uint4 xv, float acc)
{
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, 1.0f, 0),
                                          as_bf16x2(xv.x), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, 1.0f, 1),
                                          as_bf16x2(xv.y), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, 1.0f, 2),
                                          as_bf16x2(xv.z), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, 1.0f, 3),
                                          as_bf16x2(xv.w), acc, false);
    return acc;
}

__device__ __forceinline__ float dot8_e2m1_f32(uint32_t codes, const float *xv, float acc)
{
    f32x2 v;
    v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, 0);
    acc = fmaf(v[0], xv[0], acc); acc = fmaf(v[1], xv[1], acc);
    v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, 1);
    acc = fmaf(v[0], xv[2], acc); acc = fmaf(v[1], xv[3], acc);
    v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, 2);
    acc = fmaf(v[0], xv[4], acc); acc = fmaf(v[1], xv[5], acc);
    v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, 3);
    acc = fmaf(v[0], xv[6], acc); acc = fmaf(v[1], xv[7], acc);
    return acc;
}

// grid.x = max_slots * ceil(d_ff / (16 * NW)); each wave owns 16 neurons.
template <int ACT, int XT, int NW>
__global__ __launch_bounds__(64 * NW) void up_e2m1_kernel(
    const void *__restrict__ x, int d, int k, const uint8_t *__restrict__ wgu,
    const uint16_t *__restrict__ wgu_scales, int d_ff, const int32_t *__restrict__ perm,
    const int4 *__restrict__ slots, const int32_t *__restrict__ n_active, float *__restrict__ h)
{
    constexpr int RT = 16;
    constexpr bool GATED = ACT == ACT_SWIGLU;
    constexpr int LMAX = 64;                         // 16-byte chunks per row (d_model <= 2048)
    __shared__ float part[NW][RT * (LMAX + 1)];
    const int ntile = (d_ff + RT * NW - 1) / (RT * NW);
    const int slot = blockIdx.x / ntile, tile = blockIdx.x - slot * ntile;
    const int nact = *n_active;
    const int4 si = slots[(size_t)slot * SLOT_INT4];
    if ((slot >= nact) | (si.z < 1)) return;       // count and record in one round trip
    const int e = si.x, row0 = si.y, n_e = si.z;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int fw0 = (tile * NW + wave) * RT;
    if (fw0 >= d_ff) return;                         // waves are independent: no block barrier
    const int L = d >> 5;
    const int nrows = min(RT, d_ff - fw0);
    const int nchunks = nrows * L;
    const int rows = GATED ? 2 * d_ff : d_ff;
    float *pw = part[wave];

    for (int m = 0; m < n_e; ++m) {
        const int tok = perm[row0 + m] / k;
        float res[2] = {0.f, 0.f};
#pragma unroll
        for (int mat = 0; mat < (GATED ? 2 : 1); ++mat) {
            const size_t rbase = (size_t)e * rows + (mat ? d_ff : 0) + fw0;
            const uint8_t *wt = wgu + rbase * (size_t)(d / 2);
            const uint16_t *st = wgu_scales + rbase * (size_t)(d / 16);
            for (int c = lane; c < nchunks; c += WAVE) {
                const int r = c / L, cc = c - r * L;
                const uint4 q = *reinterpret_cast<const uint4 *>(wt + (size_t)c * 16);
                const uint32_t s2 = *reinterpret_cast<const uint32_t *>(st + (size_t)r * (d / 16) + cc * 2);
                float d0 = 0.f, d1 = 0.f;
                if (XT == X_BF16) {
                    const uint4 *xp = reinterpret_cast<const uint4 *>(
                        reinterpret_cast<const uint16_t *>(x) + (size_t)tok * d + cc * 32);
                    d0 = dot8_e2m1_bf16(q.x, xp[0], d0);
                    d0 = dot8_e2m1_bf16(q.y, xp[1], d0);
                    d1 = dot8_e2m1_bf16(q.z, xp[2], d1);
                    d1 = dot8_e2m1_bf16(q.w, xp[3], d1);
                } else {
                    const float *xp = reinterpret_cast<const float *>(x) + (size_t)tok * d + cc * 32;
                    float xv[32];
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        const float4 t = reinterpret_cast<const float4 *>(xp)[i];
                        xv[4 * i] = t.x; xv[4 * i + 1] = t.y; xv[4 * i + 2] = t.z; xv[4 * i + 3] = t.w;
                    }
                    d0 = dot8_e2m1_f32(q.x, xv, d0);
                    d0 = dot8_e2m1_f32(q.y, xv + 8, d0);
                    d1 = dot8_e2m1_f32(q.z, xv + 16, d1);
                    d1 = dot8_e2m1_f32(q.w, xv + 24, d1);
                }
                pw[r * (LMAX + 1) + cc] = d0 * half_bits_to_float(s2 & 0xFFFFu) +
                                          d1 * half_bits_to_float(s2 >> 16);
            }
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            if (lane < nrows) {
                float s = 0.f;
                for (int i = 0; i < L; ++i) s += pw[lane * (LMAX + 1) + i];
                res[mat] = s;
            }
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        }
        if (lane < nrows) {
            const float hv = GATED ? silu_f32(res[0]) * res[1] : (res[0] > 0.f ? res[0] * res[0] : 0.f);
            h[(size_t)(row0 + m) * d_ff + fw0 + lane] = hv;
        }
    }
}

// grid.x = max_slots * nchunk; block (slot, chunk c) covers groups [c*gpc, (c+1)*gpc).
// CPL = 8-byte code chunks per lane per neuron row = ceil(d_model / 1024).
template <bool ZS, int NW, int CPL>
__global__ __launch_bounds__(64 * NW) void down_e2m1_kernel(
    const float *__restrict__ h, int d_ff, const uint8_t *__restrict__ wd,
    const uint16_t *__restrict__ wd_scales, int d, const int4 *__restrict__ slots,
    const int32_t *__restrict__ n_active, float *__restrict__ partial, int nchunk, int gpc)
{
    constexpr int NO = 16 * CPL;                    // outputs per lane
    __shared__ float red[NW][NO][WAVE];
    const int slot = blockIdx.x / nchunk, c = blockIdx.x - slot * nchunk;
    const int nact = *n_active;
    const int4 si = slots[(size_t)slot * SLOT_INT4];
    if ((slot >= nact) | (si.z < 1)) return;        // uniform; count and record in one round trip
    const int e = si.x, row0 = si.y, n_e = si.z;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int G = d_ff >> 4;
    const int g_begin = c * gpc, g_end = min(G, g_begin + gpc);
    const int nb8 = d >> 4;                         // 8-byte chunks per neuron row

    for (int m = 0; m < n_e; ++m) {
        const float *hr = h + (size_t)(row0 + m) * d_ff;
        float acc[NO];
#pragma unroll
        for (int i = 0; i < NO; ++i) acc[i] = 0.f;
        for (int g = g_begin + wave; g < g_end; g += NW) {
            const float hl = lane < 16 ? hr[16 * g + lane] : 0.f;
            if (ZS && __ballot(hl != 0.f) == 0ull) continue;
            float ag[NO];
#pragma unroll
            for (int i = 0; i < NO; ++i) ag[i] = 0.f;
            uint2 q[16][CPL];
#pragma unroll
            for (int fi = 0; fi < 16; ++fi) {
                const uint8_t *vrow = wd + ((size_t)e * d_ff + 16 * g + fi) * (size_t)(d / 2);
#pragma unroll
                for (int cc = 0; cc < CPL; ++cc) {
                    const int ch = lane + WAVE * cc;
                    q[fi][cc] = ch < nb8 ? *reinterpret_cast<const uint2 *>(vrow + (size_t)ch * 8)
                                         : make_uint2(0, 0);
                }
            }
#pragma unroll
            for (int fi = 0; fi < 16; ++fi) {
                const float hf = __shfl(hl, fi, WAVE);
#pragma unroll
                for (int cc = 0; cc < CPL; ++cc) {
                    f32x2 v;
#define DE(W, B, I)                                                    \
    v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(W, 1.0f, B);          \
    ag[cc * 16 + (I)] = fmaf(hf, v[0], ag[cc * 16 + (I)]);             \
    ag[cc * 16 + (I) + 1] = fmaf(hf, v[1], ag[cc * 16 + (I) + 1]);
                    DE(q[fi][cc].x, 0, 0) DE(q[fi][cc].x, 1, 2) DE(q[fi][cc].x, 2, 4) DE(q[fi][cc].x, 3, 6)
                    DE(q[fi][cc].y, 0, 8) DE(q[fi][cc].y, 1, 10) DE(q[fi][cc].y, 2, 12) DE(q[fi][cc].y, 3, 14)
#undef DE
                }
            }
            const uint16_t *srow = wd_scales + ((size_t)e * G + g) * (size_t)d;
#pragma unroll
            for (int cc = 0; cc < CPL; ++cc) {
                const int ch = lane + WAVE * cc;
                if (ch < nb8) {
                    const uint4 s0 = *reinterpret_cast<const uint4 *>(srow + (size_t)ch * 16);
                    const uint4 s1 = *reinterpret_cast<const uint4 *>(srow + (size_t)ch * 16 + 8);
                    const uint32_t sw[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        acc[cc * 16 + 2 * i] = fmaf(half_bits_to_float(sw[i] & 0xFFFFu), ag[cc * 16 + 2 * i], acc[cc * 16 + 2 * i]);
                        acc[cc * 16 + 2 * i + 1] = fmaf(half_bits_to_float(sw[i] >> 16), ag[cc * 16 + 2 * i + 1], acc[cc * 16 + 2 * i + 1]);
                    }
                }
            }
        }
#pragma unroll
        for (int i = 0; i < NO; ++i) red[wave][i][lane] = acc[i];
        __syncthreads();
        if (wave == 0) {
            float *pr = partial + ((size_t)(row0 + m) * nchunk + c) * d;
#pragma unroll
            for (int cc = 0; cc < CPL; ++cc) {
                const int ch = lane + WAVE * cc;
                if (ch < nb8) {
#pragma unroll
                    for (int ii = 0; ii < 16; ++ii) {
                        float s = red[0][cc * 16 + ii][lane];
#pragma unroll
                        for (int w = 1; w < NW; ++w) s += red[w][cc * 16 + ii][lane];
                        pr[ch * 16 + ii] = s;
                    }
                }
            }
        }
        __syncthreads();
    }
}

// ------------------------------------------------------------------------------------------

hipError_t launch_up_e2m1(const void *x, int xtype, int T, int k, const ExpertsDev &ex, int act,
                          const PermuteOut &po, float *h, hipStream_t s)
{
    constexpr int NW = 4;
    const int max_slots = min(ex.E, T * k);
    const int ntile = (ex.d_ff + 16 * NW - 1) / (16 * NW);
    const dim3 g(max_slots * ntile), b(64 * NW);
    const uint8_t *w = reinterpret_cast<const uint8_t *>(ex.gate_up);
    const uint16_t *sc = reinterpret_cast<const uint16_t *>(ex.gate_up_scales);
    ProfScope ps(K_UP_E2M1, s);
#define UP(A, X) hipLaunchKernelGGL((up_e2m1_kernel<A, X, NW>), g, b, 0, s, x, ex.d_model, k, w, sc, \
                                    ex.d_ff, po.perm, po.slots, po.n_active, h)
    if (act == ACT_RELU2) { if (xtype == X_BF16) UP(ACT_RELU2, X_BF16); else UP(ACT_RELU2, X_F32); }
    else { if (xtype == X_BF16) UP(ACT_SWIGLU, X_BF16); else UP(ACT_SWIGLU, X_F32); }
#undef UP
    return hipGetLastError();
}

static constexpr int E2M1_GPC = 16;   // groups of 16 neurons per down block

int e2m1_down_chunks(int d_ff)
{
    return ((d_ff / 16) + E2M1_GPC - 1) / E2M1_GPC;
}

hipError_t launch_down_e2m1(const float *h, const ExpertsDev &ex, int T, int k, bool zero_skip,
                            const PermuteOut &po, float *partial, int nchunk, hipStream_t s)
{
    constexpr int NW = 4;
    const int max_slots = min(ex.E, T * k);
    const dim3 g(max_slots * nchunk), b(64 * NW);
    const uint8_t *w = reinterpret_cast<const uint8_t *>(ex.down);
    const uint16_t *sc = reinterpret_cast<const uint16_t *>(ex.down_scales);
    const bool two = ex.d_model > 1024;
    ProfScope ps(K_DOWN_E2M1, s);
#define DN(Z, C) hipLaunchKernelGGL((down_e2m1_kernel<Z, NW, C>), g, b, 0, s, h, ex.d_ff, w, sc, \
                                    ex.d_model, po.slots, po.n_active, partial, nchunk, E2M1_GPC)
    if (zero_skip) { if (two) DN(true, 2); else DN(true, 1); }
    else { if (two) DN(false, 2); else DN(false, 1); }
#undef DN
    return hipGetLastError();
}

}  // namespace moe
