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
#include "route_dev.hpp"

namespace moe {

// 1.0f produced by an instruction the optimiser does not fold (see dot8_e2m1_bf16)
__device__ __forceinline__ float opaque_one()
{
    float one;
    asm volatile("v_mov_b32 %0, 1.0" : "=v"(one));
    return one;
}

__device__ __forceinline__ bf16x2 as_bf16x2(uint32_t u)
{
    return __builtin_bit_cast(bf16x2, u);
}

// dot of 8 E2M1 codes (one little-endian word, code 2b in the low nibble of byte b) with 8 bf16
// activations (a uint4, element 2i in the low half of word i).
// `one` is 1.0 (the conversion scale); passing a value the compiler cannot see through keeps it from
// hoisting the conversions of loop-invariant codes out of a per-token loop, which costs a
// register per converted pair.
__device__ __forceinline__ float dot8_e2m1_bf16(uint32_t codes, uint4 xv, float acc, float one = 1.0f)
{
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, one, 0),
                                          as_bf16x2(xv.x), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, one, 1),
                                          as_bf16x2(xv.y), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, one, 2),
                                          as_bf16x2(xv.z), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, one, 3),
                                          as_bf16x2(xv.w), acc, false);
    return acc;
}

__device__ __forceinline__ float dot8_e2m1_f32(uint32_t codes, const float *xv, float acc, float one = 1.0f)
{
    f32x2 v;
    v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, one, 0);
    acc = fmaf(v[0], xv[0], acc); acc = fmaf(v[1], xv[1], acc);
    v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, one, 1);
    acc = fmaf(v[0], xv[2], acc); acc = fmaf(v[1], xv[3], acc);
    v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, one, 2);
    acc = fmaf(v[0], xv[4], acc); acc = fmaf(v[1], xv[5], acc);
    v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, one, 3);
    acc = fmaf(v[0], xv[6], acc); acc = fmaf(v[1], xv[7], acc);
    return acc;
}

// Pairs per slot (the first ones) whose zero-skip group masks the lane-group up kernel writes for
// the down projection: [slot][pair][group] bytes, so that a down block can read its groups' masks
// together with its slot record (the address needs neither) and issue its weight loads at once.
constexpr int E2M1_MASK_PAIRS = 2;

// Up: grid.x = max_slots * ceil(d_ff / (16 * NW)); wave w of a block owns 16 neurons (rows) of
// one active expert.  The wave's codes and scales (16 rows x d_model / 2 bytes per matrix) are
// loaded once, all at the start, and reused for every token routed to the expert; each token's
// row of x is staged in LDS.  Chunk c = lane + 64 i of the wave's 16 x L chunks (32 codes, 16
// bytes each, L = d_model / 32 per row) is row c / L, column chunk c % L; per-chunk dot products
// meet in LDS and are summed per row in column order.
template <int ACT, int XT, int NW, int NI>
__global__ __launch_bounds__(64 * NW) void up_e2m1_kernel(
    const void *__restrict__ x, int T, int d, int k, const uint8_t *__restrict__ wgu,
    const uint16_t *__restrict__ wgu_scales, int d_ff, const int32_t *__restrict__ perm,
    const int4 *__restrict__ slots, const int32_t *__restrict__ n_active, float *__restrict__ h)
{
    constexpr int RT = 16;
    constexpr bool GATED = ACT == ACT_SWIGLU;
    constexpr int M = GATED ? 2 : 1;
    constexpr int LMAX = 64;                         // 16-byte chunks per row (d_model <= 2048)
    constexpr int XB = XT == X_BF16 ? 2 : 4;         // bytes per activation
    __shared__ float part[NW][RT * (LMAX + 1)];
    __shared__ uint4 xs4[2048 * XB / 16];            // one token's x row
    const int ntile = (d_ff + RT * NW - 1) / (RT * NW);
    const int slot = blockIdx.x / ntile, tile = blockIdx.x - slot * ntile;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int nact = *n_active;
    const int4 si = slots[(size_t)slot * SLOT_INT4];
    const int tok16 = slot_token(slots, slot, lane & 15);
    if ((slot >= nact) | (si.z < 1) | (__builtin_amdgcn_readfirstlane(tok16) < 0)) return;
    const int e = si.x, row0 = si.y, n_e = si.z;
    const int fw0 = (tile * NW + wave) * RT;
    const bool live = fw0 < d_ff;                    // dead waves still join the barriers
    const int fwc = live ? fw0 : 0;
    const int nrows = live ? min(RT, d_ff - fw0) : 1;
    const int L = d >> 5;
    const int nchunks = nrows * L;
    const int rows = GATED ? 2 * d_ff : d_ff;
    float *pw = part[wave];

    uint4 q[M][NI];
    uint32_t s2[M][NI];
#pragma unroll
    for (int mat = 0; mat < M; ++mat)
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const int c = min(lane + WAVE * i, nchunks - 1);   // past the tile: re-read, unused
            const int r = c / L, cc = c - r * L;
            const size_t row = (size_t)e * rows + (mat ? d_ff : 0) + fwc + r;
            q[mat][i] = ld_stream16(wgu + row * (size_t)(d / 2) + cc * 16);
            s2[mat][i] = ld_stream4(wgu_scales + row * (size_t)(d / 16) + cc * 2);
        }

    for (int m = 0; m < n_e; ++m) {
        int tok = m < SLOT_TOKS ? __builtin_amdgcn_readlane(tok16, m) : perm[row0 + m] / k;
        tok = min(max(tok, 0), T - 1);
        __syncthreads();                             // the previous token's x is no longer read
        const uint4 *xg = reinterpret_cast<const uint4 *>(static_cast<const uint8_t *>(x) + (size_t)tok * d * XB);
        for (int i = tid; i < d * XB / 16; i += 64 * NW) xs4[i] = xg[i];
        __syncthreads();
        float res[M];
        const float one = opaque_one();
#pragma unroll
        for (int mat = 0; mat < M; ++mat) {
#pragma unroll
            for (int i = 0; i < NI; ++i) {
                const int c = lane + WAVE * i;
                if (c < nchunks) {
                    const int r = c / L, cc = c - r * L;
                    float d0 = 0.f, d1 = 0.f;
                    if (XT == X_BF16) {
                        const uint4 *xp = xs4 + cc * 4;
                        d0 = dot8_e2m1_bf16(q[mat][i].x, xp[0], d0, one);
                        d0 = dot8_e2m1_bf16(q[mat][i].y, xp[1], d0, one);
                        d1 = dot8_e2m1_bf16(q[mat][i].z, xp[2], d1, one);
                        d1 = dot8_e2m1_bf16(q[mat][i].w, xp[3], d1, one);
                    } else {
                        const float *xp = reinterpret_cast<const float *>(xs4) + cc * 32;
                        d0 = dot8_e2m1_f32(q[mat][i].x, xp, d0, one);
                        d0 = dot8_e2m1_f32(q[mat][i].y, xp + 8, d0, one);
                        d1 = dot8_e2m1_f32(q[mat][i].z, xp + 16, d1, one);
                        d1 = dot8_e2m1_f32(q[mat][i].w, xp + 24, d1, one);
                    }
                    pw[r * (LMAX + 1) + cc] = d0 * half_bits_to_float(s2[mat][i] & 0xFFFFu) +
                                              d1 * half_bits_to_float(s2[mat][i] >> 16);
                }
            }
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            float sacc = 0.f;
            if (lane < nrows)
                for (int i = 0; i < L; ++i) sacc += pw[lane * (LMAX + 1) + i];
            res[mat] = sacc;
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        }
        if (live && lane < nrows) {
            const float hv = GATED ? silu_f32(res[0]) * res[M - 1] : (res[0] > 0.f ? res[0] * res[0] : 0.f);
            h[(size_t)(row0 + m) * d_ff + fw0 + lane] = hv;
        }
    }
}

// Sum of v over each aligned group of L lanes (L = 2 .. 64, a power of two), as a fixed butterfly
// (DPP quad / row patterns, then the permlane swaps); every lane of a group gets the same bits.
template <int L>
__device__ __forceinline__ float lane_group_sum(float v)
{
    auto f = [](uint32_t u) { return __builtin_bit_cast(float, u); };
    auto u = [](float x) { return __builtin_bit_cast(uint32_t, x); };
    if (L >= 2) v += f(dpp_u32<0xB1>(u(v)));
    if (L >= 4) v += f(dpp_u32<0x4E>(u(v)));
    if (L >= 8) v += f(dpp_u32<0x141>(u(v)));
    if (L >= 16) v += f(dpp_u32<0x140>(u(v)));
    if (L >= 32) {
        const auto p = __builtin_amdgcn_permlane16_swap(u(v), u(v), false, false);
        v = f(p[0]) + f(p[1]);
    }
    if (L >= 64) {
        const auto p = __builtin_amdgcn_permlane32_swap(u(v), u(v), false, false);
        v = f(p[0]) + f(p[1]);
    }
    return v;
}

// Up for rows of L = d_model / 32 chunks with L in {16, 32, 64}: lane l always takes column chunk
// l % L of rows l / L + (64 / L) i, so it reads its 32 activations straight from global memory
// (L2) once per token, right behind its weight loads, and the row sums are lane-group
// butterflies: no LDS and no barrier.  Otherwise as up_e2m1_kernel.  ROUTE: the block selects the
// experts itself (route_slot_any; small batches), instead of reading the permute step's records.
template <int ACT, int XT, int NW, int L, int RT, bool ROUTE>
__global__ __launch_bounds__(64 * NW) void up_e2m1_rows_kernel(
    const void *__restrict__ x, int T, int d, int k, const uint8_t *__restrict__ wgu,
    const uint16_t *__restrict__ wgu_scales, int d_ff, const int32_t *__restrict__ perm,
    const int4 *__restrict__ slots, const int32_t *__restrict__ n_active, float *__restrict__ h, RouteIn ri,
    uint8_t *__restrict__ gmask)
{
    constexpr bool GATED = ACT == ACT_SWIGLU;
    constexpr int M = GATED ? 2 : 1;
    static_assert(RT == 16, "one wave = one 16-neuron group (the zero-skip masks)");
    constexpr int RPL = WAVE / L;                    // rows per load instruction
    constexpr int NI = RT / RPL;                     // loads per lane per matrix
    constexpr int XB = XT == X_BF16 ? 2 : 4;
    constexpr int DD = L * 32;                       // d_model
    const int ntile = (d_ff + RT * NW - 1) / (RT * NW);
    const int slot = blockIdx.x / ntile, tile = blockIdx.x - slot * ntile;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    int e, row0, n_e, tok16;
    if constexpr (ROUTE) {
        const RouteSlot rs = route_slot_any<NW>(ri, T, k, slot, tile == 0, lane & 15);
        if (rs.e < 0) return;                        // uniform across the block
        e = rs.e;
        row0 = rs.row0;
        n_e = rs.n_e;
        tok16 = rs.tok;
    } else {
        const int nact = *n_active;
        const int4 si = slots[(size_t)slot * SLOT_INT4];
        tok16 = slot_token(slots, slot, lane & 15);
        if ((slot >= nact) | (si.z < 1) | (__builtin_amdgcn_readfirstlane(tok16) < 0)) return;
        e = si.x;
        row0 = si.y;
        n_e = si.z;
    }
    const int fw0 = (tile * NW + wave) * RT;
    const bool live = fw0 < d_ff;                    // dead waves still join the barriers
    const int fwc = live ? fw0 : 0;
    const int nrows = live ? min(RT, d_ff - fw0) : 1;
    const int cc = lane % L, rs = lane / L;
    const int rows = GATED ? 2 * d_ff : d_ff;

    uint4 q[M][NI];
    uint32_t s2[M][NI];
#pragma unroll
    for (int mat = 0; mat < M; ++mat)
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const int r = min(rs + RPL * i, nrows - 1);      // past the tile: re-read, unused
            const size_t row = (size_t)e * rows + (mat ? d_ff : 0) + fwc + r;
            q[mat][i] = ld_stream16(wgu + row * (size_t)(DD / 2) + cc * 16);
            s2[mat][i] = ld_stream4(wgu_scales + row * (size_t)(DD / 16) + cc * 2);
        }

    for (int m = 0; m < n_e; ++m) {
        int tok = m < SLOT_TOKS ? __builtin_amdgcn_readlane(tok16, m) : perm[row0 + m] / k;
        tok = min(max(tok, 0), T - 1);
        const uint4 *xg = reinterpret_cast<const uint4 *>(static_cast<const uint8_t *>(x) + (size_t)tok * DD * XB);
        const float one = opaque_one();
        uint4 xb[4];
        float xf[32];
        if (XT == X_BF16) {
#pragma unroll
            for (int j = 0; j < 4; ++j) xb[j] = xg[cc * 4 + j];
        } else {
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const uint4 t = xg[cc * 8 + j];
                xf[4 * j] = __uint_as_float(t.x); xf[4 * j + 1] = __uint_as_float(t.y);
                xf[4 * j + 2] = __uint_as_float(t.z); xf[4 * j + 3] = __uint_as_float(t.w);
            }
        }
        bool nz = false;                             // a nonzero h among this lane's rows
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            float res[M];
#pragma unroll
            for (int mat = 0; mat < M; ++mat) {
                float d0 = 0.f, d1 = 0.f;
                if (XT == X_BF16) {
                    d0 = dot8_e2m1_bf16(q[mat][i].x, xb[0], d0, one);
                    d0 = dot8_e2m1_bf16(q[mat][i].y, xb[1], d0, one);
                    d1 = dot8_e2m1_bf16(q[mat][i].z, xb[2], d1, one);
                    d1 = dot8_e2m1_bf16(q[mat][i].w, xb[3], d1, one);
                } else {
                    d0 = dot8_e2m1_f32(q[mat][i].x, xf, d0, one);
                    d0 = dot8_e2m1_f32(q[mat][i].y, xf + 8, d0, one);
                    d1 = dot8_e2m1_f32(q[mat][i].z, xf + 16, d1, one);
                    d1 = dot8_e2m1_f32(q[mat][i].w, xf + 24, d1, one);
                }
                res[mat] = lane_group_sum<L>(d0 * half_bits_to_float(s2[mat][i] & 0xFFFFu) +
                                             d1 * half_bits_to_float(s2[mat][i] >> 16));
            }
            const int r = rs + RPL * i;
            if (live && cc == 0 && r < nrows) {
                const float hv = GATED ? silu_f32(res[0]) * res[M - 1] : (res[0] > 0.f ? res[0] * res[0] : 0.f);
                h[(size_t)(row0 + m) * d_ff + fw0 + r] = hv;
                nz |= hv != 0.f;
            }
        }
        // the zero-skip mask of this wave's group for the slot's first two pairs: 1 if any of the
        // group's 16 h values is nonzero (the down projection's own criterion)
        if (gmask && m < E2M1_MASK_PAIRS) {
            const bool any = __ballot(nz) != 0ull;
            if (live && lane == 0)
                gmask[((size_t)slot * E2M1_MASK_PAIRS + m) * (d_ff >> 4) + (fw0 >> 4)] = any ? 1 : 0;
        }
    }
}

// Up for d_model > 2048 (L = d_model / 32 > 64 chunks per row): a row is LG lanes wide (64, or 32
// with two rows side by side in a wave), lane l of a row takes column chunks l + LG u (u < CPR,
// chunks past L contribute nothing) of each of its RT / (64 / LG) rows, reads their activations
// from global memory once per token, and a row's sum is the lane's chunks in order, then a
// butterfly over the row's LG lanes.  Otherwise as up_e2m1_rows_kernel.  (LG and CPR are chosen
// so that LG CPR covers L with little to spare: d_model 2816 is 88 chunks, 32 x 3 instead of
// 64 x 2; 6144 is 192, 64 x 3 instead of 64 x 4.)
template <int ACT, int XT, int NW, int CPR, int RT, int LG>
__global__ __launch_bounds__(64 * NW) void up_e2m1_wide_kernel(
    const void *__restrict__ x, int T, int d, int k, const uint8_t *__restrict__ wgu,
    const uint16_t *__restrict__ wgu_scales, int d_ff, const int32_t *__restrict__ perm,
    const int4 *__restrict__ slots, const int32_t *__restrict__ n_active, float *__restrict__ h)
{
    constexpr bool GATED = ACT == ACT_SWIGLU;
    constexpr int M = GATED ? 2 : 1;
    constexpr int XB = XT == X_BF16 ? 2 : 4;
    constexpr int RG = WAVE / LG;                    // rows side by side in a wave
    constexpr int RI = RT / RG;                      // row steps per wave
    static_assert(RI * RG == RT, "RT rows in steps of RG");
    const int ntile = (d_ff + RT * NW - 1) / (RT * NW);
    const int slot = blockIdx.x / ntile, tile = blockIdx.x - slot * ntile;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int rg = lane / LG, cl = lane % LG;
    const int nact = *n_active;
    const int4 si = slots[(size_t)slot * SLOT_INT4];
    const int tok16 = slot_token(slots, slot, lane & 15);
    if ((slot >= nact) | (si.z < 1) | (__builtin_amdgcn_readfirstlane(tok16) < 0)) return;
    const int e = si.x, row0 = si.y, n_e = si.z;
    const int fw0 = (tile * NW + wave) * RT;
    if (fw0 >= d_ff) return;                         // uniform across the wave (no block barrier)
    const int nrows = min(RT, d_ff - fw0);
    const int L = d >> 5;
    const int rows = GATED ? 2 * d_ff : d_ff;

    uint4 q[M][RI][CPR];
    uint32_t s2[M][RI][CPR];
#pragma unroll
    for (int mat = 0; mat < M; ++mat)
#pragma unroll
        for (int i = 0; i < RI; ++i)
#pragma unroll
            for (int u = 0; u < CPR; ++u) {
                const int cc = min(cl + LG * u, L - 1);              // past the row: re-read, unused
                const int r = min(i * RG + rg, nrows - 1);          // past the tile: re-read, unused
                const size_t row = (size_t)e * rows + (mat ? d_ff : 0) + fw0 + r;
                q[mat][i][u] = ld_stream16(wgu + row * (size_t)(d / 2) + cc * 16);
                s2[mat][i][u] = ld_stream4(wgu_scales + row * (size_t)(d / 16) + cc * 2);
            }

    for (int m = 0; m < n_e; ++m) {
        int tok = m < SLOT_TOKS ? __builtin_amdgcn_readlane(tok16, m) : perm[row0 + m] / k;
        tok = min(max(tok, 0), T - 1);
        const uint4 *xg = reinterpret_cast<const uint4 *>(static_cast<const uint8_t *>(x) + (size_t)tok * d * XB);
        const float one = opaque_one();
        uint4 xb[CPR][XT == X_BF16 ? 4 : 8];
#pragma unroll
        for (int u = 0; u < CPR; ++u) {
            const int cc = min(cl + LG * u, L - 1);
#pragma unroll
            for (int j = 0; j < (XT == X_BF16 ? 4 : 8); ++j) xb[u][j] = xg[cc * (XT == X_BF16 ? 4 : 8) + j];
        }
#pragma unroll
        for (int i = 0; i < RI; ++i) {
            float res[M];
#pragma unroll
            for (int mat = 0; mat < M; ++mat) {
                float part = 0.f;
#pragma unroll
                for (int u = 0; u < CPR; ++u) {
                    float d0 = 0.f, d1 = 0.f;
                    if (XT == X_BF16) {
                        d0 = dot8_e2m1_bf16(q[mat][i][u].x, xb[u][0], d0, one);
                        d0 = dot8_e2m1_bf16(q[mat][i][u].y, xb[u][1], d0, one);
                        d1 = dot8_e2m1_bf16(q[mat][i][u].z, xb[u][2], d1, one);
                        d1 = dot8_e2m1_bf16(q[mat][i][u].w, xb[u][3], d1, one);
                    } else {
                        const float *xf = reinterpret_cast<const float *>(&xb[u][0]);
                        d0 = dot8_e2m1_f32(q[mat][i][u].x, xf, d0, one);
                        d0 = dot8_e2m1_f32(q[mat][i][u].y, xf + 8, d0, one);
                        d1 = dot8_e2m1_f32(q[mat][i][u].z, xf + 16, d1, one);
                        d1 = dot8_e2m1_f32(q[mat][i][u].w, xf + 24, d1, one);
                    }
                    const float cv = d0 * half_bits_to_float(s2[mat][i][u] & 0xFFFFu) +
                                     d1 * half_bits_to_float(s2[mat][i][u] >> 16);
                    part += cl + LG * u < L ? cv : 0.f;
                }
                res[mat] = lane_group_sum<LG>(part);
            }
            const int r = i * RG + rg;
            if (cl == 0 && r < nrows) {
                const float hv = GATED ? silu_f32(res[0]) * res[M - 1] : (res[0] > 0.f ? res[0] * res[0] : 0.f);
                h[(size_t)(row0 + m) * d_ff + fw0 + r] = hv;
            }
        }
    }
}

// Down: grid.x = max_slots * nchunk; block (slot, c) covers the GPC 16-neuron groups starting at
// c * GPC for every pair of the slot.  Wave w owns the groups w and w + NW of
// the chunk (fixed by group index, so the dense and the zero-skip reads sum the same terms in the
// same order); a group is 16 neuron rows of d_model codes (lane l holds output chunks l + 64 cc,
// 16 outputs of 8 bytes each) plus its d_model scales.  Both groups' loads go out before either is
// used.  With ZS a group whose 16 h values are all zero is not read: it would add exact zeros,
// so the result equals the dense one bit for bit.  The NW per-wave sums meet in LDS in wave order.
// Groups per block and waves per block: 16 groups / 8 waves for batches of at most 2 tokens, 8
// groups / 4 waves above (twice the blocks and partial sums).  Nemotron-shaped zero-skip, us per
// layer: T = 1, 34.9 (16 / 8) vs 35.5 (8 / 4), 36.8 (8 / 8), 44.2 (32 / 8); T = 8, 161.3 (16 / 8)
// vs 146.2 (8 / 4).
constexpr int E2M1_GPC_SMALL_T = 16, E2M1_NW_SMALL_T = 8;
constexpr int E2M1_GPC = 8, E2M1_DOWN_NW = 4;

template <bool ZS, int NW, int CPL, int GPC>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(4, 8))) void down_e2m1_kernel(
    const float *__restrict__ h, int d_ff, const uint8_t *__restrict__ wd,
    const uint16_t *__restrict__ wd_scales, int d, const int4 *__restrict__ slots,
    const int32_t *__restrict__ n_active, float *__restrict__ partial, int nchunk,
    const uint8_t *__restrict__ gmask)
{
    constexpr int NO = 16 * CPL;                     // outputs per lane
    constexpr int NT = 64 * NW;
    constexpr int GPW = GPC / NW;
    __shared__ float red[NW][NO][WAVE];
    // block (slot, c, op): output part op covers the 16-output chunks 64 CPL op .. 64 CPL op + 64 CPL - 1
    const int nb8 = d >> 4;                          // 8-byte code chunks per neuron row
    const int nop = (nb8 + WAVE * CPL - 1) / (WAVE * CPL);
    const int op = blockIdx.x % nop, sc_ = blockIdx.x / nop;
    const int slot = sc_ / nchunk, c = sc_ - slot * nchunk;
    const int ch0 = op * WAVE * CPL;
    // the wave index and the masks are wave-uniform: read as such, the group addresses stay
    // scalar (one 64-bit VGPR address per loaded row otherwise)
    const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int G = d_ff >> 4;
    // the zero-skip masks of this wave's groups for the slot's first pairs, read in the same round
    // trip as the active count and the record (slot < max_slots keeps them in bounds)
    uint32_t mk[E2M1_MASK_PAIRS][GPW];
    if (ZS && gmask) {
#pragma unroll
        for (int m = 0; m < E2M1_MASK_PAIRS; ++m)
#pragma unroll
            for (int q = 0; q < GPW; ++q)
                mk[m][q] = __builtin_amdgcn_readfirstlane(
                    gmask[((size_t)slot * E2M1_MASK_PAIRS + m) * G + min(c * GPC + wave + NW * q, G - 1)]);
    }
    const int nact = *n_active;
    const int4 si = slots[(size_t)slot * SLOT_INT4];
    if ((slot >= nact) | (si.z < 1)) return;         // uniform; count and record in one trip
    const int e = si.x, row0 = si.y, n_e = si.z;

    // This wave's groups and their liveness over all of the slot's pairs: a group is read when
    // one of its 16 h values is nonzero for some pair (the up kernel's masks for the first pairs,
    // which need no wait for h; the h values of the pairs after those).  The weights are loaded
    // once and serve every pair; for a pair whose 16 h values of a live group are all zero the
    // products are exact zeros, so the sums equal the dense ones bit for bit.
    int gg[GPW];
    bool live[GPW];
    {
        bool any[GPW];
#pragma unroll
        for (int q = 0; q < GPW; ++q) {
            gg[q] = min(c * GPC + wave + NW * q, G - 1);
            any[q] = false;
        }
        const int m0 = ZS && gmask ? min(n_e, E2M1_MASK_PAIRS) : 0;
        if (ZS)
            for (int m = m0; m < n_e; ++m) {             // independent loads: all in flight
                const float *hr = h + (size_t)(row0 + m) * d_ff;
#pragma unroll
                for (int q = 0; q < GPW; ++q) any[q] |= hr[16 * gg[q] + (lane & 15)] != 0.f;
            }
#pragma unroll
        for (int q = 0; q < GPW; ++q) {
            const int g = c * GPC + wave + NW * q;
            bool lv = true;
            if (ZS) {
                uint32_t mm = 0u;
                if (gmask) {
                    mm = mk[0][q];
#pragma unroll
                    for (int m = 1; m < E2M1_MASK_PAIRS; ++m) mm |= m < n_e ? mk[m][q] : 0u;
                }
                lv = mm != 0u || __ballot(any[q]) != 0ull;
            }
            live[q] = g < G && lv;
        }
    }

    // QB groups' loads at a time: all of the wave's at d_model <= 1024, loaded once for every
    // pair; one at a time above, where a group needs twice the registers, re-read per pair.
    // Loads are unconditional: a group that is not read loads the first rows of expert 0
    // instead, which stay in cache (no HBM bytes), and takes zero codes, scales and h, so its
    // products add exact zeros.  (With the loads and products of each group under a branch, the
    // compiler issued the second group's loads only after the first group's products.)  The dense
    // projection streams its weights with the non-temporal hint; zero-skip keeps plain loads, so
    // that those stand-in rows stay cached (with the hint: Nemotron-shaped T = 1 down 12.2 ->
    // 13.5 us, T = 8 47.7 -> 48.8; dense Gemma-shaped E2M1 T = 8 down 22.6 -> 21.9 with it).
    constexpr int QB = CPL == 1 ? GPW : 1;
    uint2 qv[GPW][16][CPL];
    uint4 sv[GPW][CPL][2];
    auto load_group = [&](int q) {
        const size_t rows0 = live[q] ? (size_t)e * d_ff + 16 * gg[q] : 0;
        const size_t srow0 = live[q] ? ((size_t)e * G + gg[q]) * (size_t)d : 0;
        // wave-uniform row bases plus one unsigned 32-bit lane offset
        const uint8_t *wq = wd + rows0 * (size_t)(d / 2);
        const uint8_t *ws = reinterpret_cast<const uint8_t *>(wd_scales + srow0);
#pragma unroll
        for (int cc = 0; cc < CPL; ++cc) {
            const uint32_t ch = (uint32_t)min(ch0 + lane + WAVE * cc, nb8 - 1);   // past the row: re-read, unused
#pragma unroll
            for (int fi = 0; fi < 16; ++fi)
                qv[q][fi][cc] = ZS ? *reinterpret_cast<const uint2 *>(wq + (size_t)fi * (size_t)(d / 2) + ch * 8u)
                                   : ld_stream8(wq + (size_t)fi * (size_t)(d / 2) + ch * 8u);
            sv[q][cc][0] = ZS ? *reinterpret_cast<const uint4 *>(ws + ch * 32u) : ld_stream16(ws + ch * 32u);
            sv[q][cc][1] = ZS ? *reinterpret_cast<const uint4 *>(ws + ch * 32u + 16u) : ld_stream16(ws + ch * 32u + 16u);
        }
    };
    auto zero_dead = [&](int q) {
        if (!live[q]) {
#pragma unroll
            for (int cc = 0; cc < CPL; ++cc) {
#pragma unroll
                for (int fi = 0; fi < 16; ++fi) qv[q][fi][cc] = make_uint2(0u, 0u);
                sv[q][cc][0] = make_uint4(0u, 0u, 0u, 0u);
                sv[q][cc][1] = sv[q][cc][0];
            }
        }
    };
    float hl0[GPW];                                  // pair 0's h, loaded with the weights
#pragma unroll
    for (int q = 0; q < GPW; ++q) hl0[q] = h[(size_t)row0 * d_ff + 16 * gg[q] + (lane & 15)];
    if constexpr (QB == GPW) {
#pragma unroll
        for (int q = 0; q < GPW; ++q) load_group(q);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int q = 0; q < GPW; ++q) zero_dead(q);
    }
    for (int m = 0; m < n_e; ++m) {
        const float *hr = h + (size_t)(row0 + m) * d_ff;
        float acc[NO];
#pragma unroll
        for (int i = 0; i < NO; ++i) acc[i] = 0.f;
#pragma unroll
        for (int q0 = 0; q0 < GPW; q0 += QB) {
            float hl[GPW];
#pragma unroll
            for (int q = q0; q < q0 + QB; ++q) hl[q] = m == 0 ? hl0[q] : hr[16 * gg[q] + (lane & 15)];
            if constexpr (QB < GPW) {
#pragma unroll
                for (int q = q0; q < q0 + QB; ++q) load_group(q);
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int q = q0; q < q0 + QB; ++q) zero_dead(q);
            }
#pragma unroll
            for (int q = q0; q < q0 + QB; ++q) {
                if (!live[q]) hl[q] = 0.f;
                float ag[NO];
#pragma unroll
                for (int i = 0; i < NO; ++i) ag[i] = 0.f;
#pragma unroll
                for (int fi = 0; fi < 16; ++fi) {
                    // neuron fi's h value sits in lane fi: a scalar read, no LDS permute
                    const float hf = __builtin_bit_cast(
                        float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, hl[q]), fi));
#pragma unroll
                    for (int cc = 0; cc < CPL; ++cc) {
                        f32x2 v;
#define DE(W, B, I)                                                    \
    v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(W, 1.0f, B);          \
    ag[cc * 16 + (I)] = fmaf(hf, v[0], ag[cc * 16 + (I)]);             \
    ag[cc * 16 + (I) + 1] = fmaf(hf, v[1], ag[cc * 16 + (I) + 1]);
                        DE(qv[q][fi][cc].x, 0, 0) DE(qv[q][fi][cc].x, 1, 2) DE(qv[q][fi][cc].x, 2, 4) DE(qv[q][fi][cc].x, 3, 6)
                        DE(qv[q][fi][cc].y, 0, 8) DE(qv[q][fi][cc].y, 1, 10) DE(qv[q][fi][cc].y, 2, 12) DE(qv[q][fi][cc].y, 3, 14)
#undef DE
                    }
                }
#pragma unroll
                for (int cc = 0; cc < CPL; ++cc) {
                    const uint32_t sw[8] = {sv[q][cc][0].x, sv[q][cc][0].y, sv[q][cc][0].z, sv[q][cc][0].w,
                                            sv[q][cc][1].x, sv[q][cc][1].y, sv[q][cc][1].z, sv[q][cc][1].w};
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        acc[cc * 16 + 2 * i] = fmaf(half_bits_to_float(sw[i] & 0xFFFFu), ag[cc * 16 + 2 * i], acc[cc * 16 + 2 * i]);
                        acc[cc * 16 + 2 * i + 1] = fmaf(half_bits_to_float(sw[i] >> 16), ag[cc * 16 + 2 * i + 1], acc[cc * 16 + 2 * i + 1]);
                    }
                }
            }
            // the codes and scales are the same for every pair: hide that from the compiler, which
            // would otherwise convert all of them once, outside the pair loop, into far more
            // registers than the codes take (an empty asm that claims to change them; placed
            // after the products, so the first pair's products still start as loads arrive)
#pragma unroll
            for (int q = q0; q < q0 + QB; ++q)
#pragma unroll
                for (int cc = 0; cc < CPL; ++cc) {
#pragma unroll
                    for (int fi = 0; fi < 16; ++fi) {
                        uint32_t a0 = qv[q][fi][cc].x, a1 = qv[q][fi][cc].y;
                        asm volatile("" : "+v"(a0), "+v"(a1));
                        qv[q][fi][cc] = make_uint2(a0, a1);
                    }
#pragma unroll
                    for (int j = 0; j < 2; ++j) {
                        uint32_t b0 = sv[q][cc][j].x, b1 = sv[q][cc][j].y, b2 = sv[q][cc][j].z, b3 = sv[q][cc][j].w;
                        asm volatile("" : "+v"(b0), "+v"(b1), "+v"(b2), "+v"(b3));
                        sv[q][cc][j] = make_uint4(b0, b1, b2, b3);
                    }
                }
        }
        __syncthreads();                             // the previous pair's sums have been read
#pragma unroll
        for (int i = 0; i < NO; ++i) red[wave][i][lane] = acc[i];
        __syncthreads();
        float *pr = partial + ((size_t)(row0 + m) * nchunk + c) * d;
        const int o_end = min(16 * (ch0 + WAVE * CPL), d);
        for (int o = 16 * ch0 + tid; o < o_end; o += NT) {
            const int ch = (o >> 4) - ch0, j = o & 15;
            const int ln = ch & (WAVE - 1), i = (ch >> 6) * 16 + j;
            float sacc = red[0][i][ln];
#pragma unroll
            for (int w = 1; w < NW; ++w) sacc += red[w][i][ln];
            pr[o] = sacc;
        }
    }
}

// ------------------------------------------------------------------------------------------

// Rows per wave and waves per block of the lane-group up kernel.  Measured on the Nemotron-shaped
// T = 1 up (22 experts x 2688 rows of 1024 codes): 8 x 4 -> 10.2 us, 16 x 4 -> 10.4, 16 x 8 ->
// 10.5, 32 x 4 -> 11.7 (the kernel is latency-bound at this size: one round trip for the slot
// record, one for the weights).  16 rows keeps every activation / format variant in registers.
constexpr int UPR_RT = 16, UPR_NW = 4;

// Waves per block of the lane-group up kernel when it routes the batch itself (the sorted
// selection over up to 512 experts takes eight waves).
constexpr int UPR_ROUTE_NW = 8;

template <int ACT, int XT>
static void launch_up_t(dim3 g, dim3 b, hipStream_t s, int ni, const void *x, int T, int k,
                        const ExpertsDev &ex, const uint8_t *w, const uint16_t *sc, const PermuteOut &po,
                        float *h, const RouteIn &ri, uint8_t *gmask)
{
    constexpr int NW = 4;
    static_assert(UPR_RT == 16 && UPR_NW == NW, "the launch grid assumes the up kernels' tiling");
#define UPR(L) hipLaunchKernelGGL((up_e2m1_rows_kernel<ACT, XT, UPR_NW, L, UPR_RT, false>), g, b, 0, s, x, T, \
                                  ex.d_model, k, w, sc, ex.d_ff, po.perm, po.slots, po.n_active, h, ri, gmask)
#define UPRR(L) hipLaunchKernelGGL((up_e2m1_rows_kernel<ACT, XT, UPR_ROUTE_NW, L, UPR_RT, true>), \
                                   dim3((min(ex.E, T * k) + ex.S) * ((ex.d_ff + UPR_RT * UPR_ROUTE_NW - 1) / \
                                                                     (UPR_RT * UPR_ROUTE_NW))), \
                                   dim3(64 * UPR_ROUTE_NW), 0, s, x, T, ex.d_model, k, w, sc, ex.d_ff, po.perm, \
                                   po.slots, po.n_active, h, ri, gmask)
#define UP(N) hipLaunchKernelGGL((up_e2m1_kernel<ACT, XT, NW, N>), g, b, 0, s, x, T, ex.d_model, k, w, sc, \
                                 ex.d_ff, po.perm, po.slots, po.n_active, h)
    // the lane-group kernel for rows of 512, 1024 or 2048 codes, routing itself when asked to
    if (ri.logits) {
        if (ex.d_model == 512) UPRR(16);
        else if (ex.d_model == 1024) UPRR(32);
        else UPRR(64);
        return;
    }
    if (ex.d_model == 512) { UPR(16); return; }
    if (ex.d_model == 1024) { UPR(32); return; }
    if (ex.d_model == 2048) { UPR(64); return; }
    if (ni <= 4) UP(4);
    else if (ni <= 8) UP(8);
    else UP(16);
#undef UP
#undef UPRR
#undef UPR
}

// Rows per wave of the wide-row up kernel at 2 chunks per lane (d_model > 2048; RT x CPR x matrices
// code pieces per lane, so RT halves as CPR doubles)
constexpr int UPW_RT = 4, UPW_NW = 4;

template <int ACT, int XT>
static void launch_up_wide_t(hipStream_t s, const void *x, int T, int k, const ExpertsDev &ex, const uint8_t *w,
                             const uint16_t *sc, const PermuteOut &po, float *h)
{
    const int max_slots = min(ex.E, T * k) + ex.S;   // routed slots, then the shared ones
    const dim3 b(64 * UPW_NW);
    const int L = ex.d_model / 32;
#define UPW(C, R, G) hipLaunchKernelGGL((up_e2m1_wide_kernel<ACT, XT, UPW_NW, C, R, G>), \
                                        dim3(max_slots * ((ex.d_ff + R * UPW_NW - 1) / (R * UPW_NW))), b, 0, s, x, T, \
                                        ex.d_model, k, w, sc, ex.d_ff, po.perm, po.slots, po.n_active, h)
    if (L <= 3 * 32) UPW(3, UPW_RT, 32);
    else if (L <= 2 * WAVE) UPW(2, UPW_RT, WAVE);
    else if (L <= 3 * WAVE) UPW(3, UPW_RT / 2, WAVE);
    else if (L <= 4 * WAVE) UPW(4, UPW_RT / 2, WAVE);
    else UPW(8, UPW_RT / 4, WAVE);
#undef UPW
}

// The widths the lane-group up kernel takes (it routes small batches itself and writes the
// zero-skip masks).
static bool up_e2m1_rows_width(int d_model) { return d_model == 512 || d_model == 1024 || d_model == 2048; }

// In-block routing for one token, or two over at most 256 experts: above that the blocks'
// selection takes one pass per token (8 waves sort one token's 512 keys), and a separate
// selection launch is cheaper (Nemotron-shaped T = 2: 34.2k -> 38.8k tokens/s).
bool up_e2m1_can_route(int T, int k, int E, int d_model)
{
    return (T == 1 || (T == 2 && E <= 256)) && T * k <= 64 && E <= MAX_E && up_e2m1_rows_width(d_model);
}

size_t e2m1_mask_bytes(int E, int S, int d_ff) { return (size_t)(E + S) * E2M1_MASK_PAIRS * (d_ff / 16); }

hipError_t launch_up_e2m1(const void *x, int xtype, int T, int k, const ExpertsDev &ex, int act,
                          const PermuteOut &po, float *h, const RouteIn &ri, uint8_t *gmask, hipStream_t s)
{
    if (ri.logits && !up_e2m1_can_route(T, k, ex.E, ex.d_model)) return hipErrorInvalidValue;
    constexpr int NW = 4;
    const int max_slots = min(ex.E, T * k) + ex.S;   // routed slots, then the shared ones
    const int ntile = (ex.d_ff + 16 * NW - 1) / (16 * NW);
    const int ni = (16 * (ex.d_model / 32) + WAVE - 1) / WAVE;     // chunks per lane per matrix
    const dim3 g(max_slots * ntile), b(64 * NW);
    const uint8_t *w = reinterpret_cast<const uint8_t *>(ex.gate_up);
    const uint16_t *sc = reinterpret_cast<const uint16_t *>(ex.gate_up_scales);
    ProfScope ps(K_UP_E2M1, s);
    if (ex.d_model > 2048) {
        if (act == ACT_RELU2) {
            if (xtype == X_BF16) launch_up_wide_t<ACT_RELU2, X_BF16>(s, x, T, k, ex, w, sc, po, h);
            else launch_up_wide_t<ACT_RELU2, X_F32>(s, x, T, k, ex, w, sc, po, h);
        } else {
            if (xtype == X_BF16) launch_up_wide_t<ACT_SWIGLU, X_BF16>(s, x, T, k, ex, w, sc, po, h);
            else launch_up_wide_t<ACT_SWIGLU, X_F32>(s, x, T, k, ex, w, sc, po, h);
        }
        return hipGetLastError();
    }
    if (act == ACT_RELU2) {
        if (xtype == X_BF16) launch_up_t<ACT_RELU2, X_BF16>(g, b, s, ni, x, T, k, ex, w, sc, po, h, ri, gmask);
        else launch_up_t<ACT_RELU2, X_F32>(g, b, s, ni, x, T, k, ex, w, sc, po, h, ri, gmask);
    } else {
        if (xtype == X_BF16) launch_up_t<ACT_SWIGLU, X_BF16>(g, b, s, ni, x, T, k, ex, w, sc, po, h, ri, gmask);
        else launch_up_t<ACT_SWIGLU, X_F32>(g, b, s, ni, x, T, k, ex, w, sc, po, h, ri, gmask);
    }
    return hipGetLastError();
}

static int e2m1_down_gpc(int T) { return T <= 2 ? E2M1_GPC_SMALL_T : E2M1_GPC; }

int e2m1_down_chunks(int d_ff, int T)
{
    const int gpc = e2m1_down_gpc(T);
    return ((d_ff / 16) + gpc - 1) / gpc;
}

hipError_t launch_down_e2m1(const float *h, const ExpertsDev &ex, int T, int k, bool zero_skip,
                            const PermuteOut &po, float *partial, int nchunk, const uint8_t *gmask, hipStream_t s)
{
    // the masks exist where the lane-group up kernel ran
    if (!zero_skip || !up_e2m1_rows_width(ex.d_model)) gmask = nullptr;
    if (nchunk != e2m1_down_chunks(ex.d_ff, T)) return hipErrorInvalidValue;
    const int max_slots = min(ex.E, T * k) + ex.S;   // routed slots, then the shared ones
    // one 1024-output part per block (two parts per lane hold twice the code registers and spill)
    const int nop = ((ex.d_model >> 4) + WAVE - 1) / WAVE;
    const dim3 g(max_slots * nchunk * nop);
    const uint8_t *w = reinterpret_cast<const uint8_t *>(ex.down);
    const uint16_t *sc = reinterpret_cast<const uint16_t *>(ex.down_scales);
    ProfScope ps(K_DOWN_E2M1, s);
#define DN(Z, NW, GPC) hipLaunchKernelGGL((down_e2m1_kernel<Z, NW, 1, GPC>), g, dim3(64 * NW), 0, s, h, ex.d_ff, w, \
                                          sc, ex.d_model, po.slots, po.n_active, partial, nchunk, gmask)
    if (T <= 2) {
        if (zero_skip) DN(true, E2M1_NW_SMALL_T, E2M1_GPC_SMALL_T);
        else DN(false, E2M1_NW_SMALL_T, E2M1_GPC_SMALL_T);
    } else {
        if (zero_skip) DN(true, E2M1_DOWN_NW, E2M1_GPC);
        else DN(false, E2M1_DOWN_NW, E2M1_GPC);
    }
#undef DN
    return hipGetLastError();
}

}  // namespace moe
