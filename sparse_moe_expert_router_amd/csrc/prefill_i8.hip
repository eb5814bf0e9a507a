// Batched-prefill path with int8 activations on the gfx950 int8 matrix cores (the batched-prefill
// layer definition: x quantised per token, h per (token, slot) pair, int32 accumulation, fp32
// rescale).  Grouped GEMMs over the permuted pairs, one expert group at a time: the gate/up GEMM
// (the mul_mat_id of the Gemma-on-a-Xeon page's "Three-part fix" with its fused silu(gate) * up
// epilogue) and the down GEMM, both on v_mfma_i32_32x32x32_i8.
//
// Activation quantiser (rule Q): per row, a = max|v|; a = 0 gives q = 0 and scale 0; otherwise
// q = clamp(round_half_even(fp32(v * fp32(127 / a))), -127, 127), scale = fp32(a / 127).  Every
// step is one IEEE fp32 operation (correctly rounded division, v_rndne_f32), so the codes are the
// ones any IEEE fp32 implementation of the rule gets.
//
// The fp8 variant of the path (rule Q8; OCP 8-bit floating point E4M3 codes, largest finite
// magnitude 448) takes the same steps with 448 in place of 127: q = E4M3(fp32(v * fp32(448 / a)))
// rounded to nearest, ties to even (v_cvt_pk_fp8_f32), scale = fp32(a / 448); a = 0 gives codes 0.
// Its GEMMs keep the codes at one byte in HBM and LDS and widen them to f16 in registers (see the
// F8 kind of the grouped GEMM).
#include <type_traits>

#include "moe_common.hpp"
#include "moe_launch.hpp"

namespace moe {

enum { R_I8 = 0, R_F8 = 1 };     // rule Q (int8) or rule Q8 (E4M3)

template <int RULE>
__device__ __forceinline__ float rule_inv(float a)
{
    return a > 0.f ? (RULE == R_F8 ? 448.0f : 127.0f) / a : 0.f;
}

template <int RULE>
__device__ __forceinline__ float rule_scale(float a)
{
    return a / (RULE == R_F8 ? 448.0f : 127.0f);
}

// The codes of the 4 values f[0..3] (times inv), value i in byte i.  a_pos: the row's max|v| > 0
// (otherwise every code is 0; for E4M3 the sign of a zero product would give code 0x80).
template <int RULE>
__device__ __forceinline__ uint32_t rule_pack4(const float *f, float inv, bool a_pos)
{
    if (RULE == R_F8) {
        int w = __builtin_amdgcn_cvt_pk_fp8_f32(f[0] * inv, f[1] * inv, 0, false);
        w = __builtin_amdgcn_cvt_pk_fp8_f32(f[2] * inv, f[3] * inv, w, true);
        return a_pos ? (uint32_t)w : 0u;
    }
    uint32_t packed = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        float r = __builtin_rintf(f[j] * inv);
        r = fminf(fmaxf(r, -127.f), 127.f);
        packed |= ((uint32_t)(int32_t)r & 0xFFu) << (8 * j);
    }
    return packed;
}

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

// One workgroup (256 threads) per row; thread tid owns the 4-column groups 4 tid + 1024 c,
// c < CH (CH * 1024 >= cols), all loaded at once (clamped, zeroed past the row) and kept in
// registers for the second pass.  Code layouts:
//  Q_COLS  row-major, column order.
//  Q_SLOTS row-major; within each 64-column block, column 32 j + 8 g + i is stored at byte
//          16 g + 8 j + i, so the two 8-byte K pieces one MFMA lane takes (offsets 8g.. and
//          32+8g..) are one contiguous 16-byte load (the gate/up GEMM's gathered x rows).
enum { Q_COLS = 0, Q_SLOTS = 1 };

template <int RULE, int XT, int LAY, int CH>
__global__ __launch_bounds__(256) void quantize_rows_kernel(const void *__restrict__ v, int cols,
                                                            int8_t *__restrict__ q,
                                                            float *__restrict__ scale)
{
    __shared__ uint32_t s_max[4];
    const int row = blockIdx.x;
    const size_t base = (size_t)row * cols;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    float f[CH][4];
#pragma unroll
    for (int c = 0; c < CH; ++c) {
        const int i = tid * 4 + 1024 * c;
        load4<XT>(v, base + min(i, cols - 4), f[c]);
#pragma unroll
        for (int j = 0; j < 4; ++j) f[c][j] = i < cols ? f[c][j] : 0.f;
    }
    float a = 0.f;
#pragma unroll
    for (int c = 0; c < CH; ++c)
        a = fmaxf(a, fmaxf(fmaxf(fabsf(f[c][0]), fabsf(f[c][1])), fmaxf(fabsf(f[c][2]), fabsf(f[c][3]))));
    // |v| >= 0, so the float order is the order of the bit patterns
    const uint32_t wm = wave_max_u32(__float_as_uint(a));
    if (lane == 0) s_max[wave] = wm;
    __syncthreads();
    a = __uint_as_float(max(max(s_max[0], s_max[1]), max(s_max[2], s_max[3])));
    const float inv = rule_inv<RULE>(a);
#pragma unroll
    for (int c = 0; c < CH; ++c) {
        const int i = tid * 4 + 1024 * c;
        const uint32_t packed = rule_pack4<RULE>(f[c], inv, a > 0.f);
        const int cc = i & 63;                       // 4 columns at cc .. cc + 3, cc % 4 == 0
        size_t dst = base + i;
        if (LAY == Q_SLOTS) dst = base + (i - cc) + 16 * ((cc & 31) >> 3) + 8 * (cc >> 5) + (cc & 7);
        if (i < cols) *reinterpret_cast<uint32_t *>(q + dst) = packed;
    }
    if (tid == 0) scale[row] = rule_scale<RULE>(a);
}

// Rule Q for the fp32 h rows of the permuted pairs, codes in the down GEMM's A tiles: one wave
// per row, 4 rows per workgroup; the codes of 64-column block sb of row i of 128-row tile mt go to
// the 8 KB block (mt, sb), 16-byte slot 64 (i / 16) + 16 g + i % 16 holding columns 8g .. 8g+7
// and 32+8g .. 32+8g+7 (the slot order above), so the GEMM thread of slot c reads 16 bytes at
// 16 c, contiguous across a wave.  Lane l owns the 16-column units l + 64 u (u < UPL) of its row.
template <int RULE, int UPL>
__global__ __launch_bounds__(256) void quantize_h_tiles_kernel(const float *__restrict__ h, int cols,
                                                               int8_t *__restrict__ q,
                                                               float *__restrict__ scale,
                                                               const int4 *__restrict__ tiles,
                                                               const int32_t *__restrict__ tile_off, int E)
{
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int mt = blockIdx.x >> 5, ti = (blockIdx.x & 31) * 4 + wave;
    // the tile count and the tile record in one round trip (mt is below the grid's tile bound,
    // so the record read is in bounds; it is used only for a valid tile)
    const int MT = tile_off[E];
    const int4 rec = tiles[mt];
    if ((mt >= MT) | (ti >= rec.z)) return;          // uniform across the wave (no block barrier)
    const int row = rec.y + ti, S = cols >> 6, units = S * 4;
    const float *src = h + (size_t)row * cols;
    float f[UPL][16];
#pragma unroll
    for (int u = 0; u < UPL; ++u) {                  // all loads at once, clamped and zeroed past the row
        const int un = lane + 64 * u, uc = min(un, units - 1);
        const float *p = src + (uc >> 2) * 64 + 8 * (uc & 3);
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const float4 a = *reinterpret_cast<const float4 *>(p + 32 * j);
            const float4 b = *reinterpret_cast<const float4 *>(p + 32 * j + 4);
            const float vv[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
            for (int i = 0; i < 8; ++i) f[u][8 * j + i] = un < units ? vv[i] : 0.f;
        }
    }
    float a = 0.f;
#pragma unroll
    for (int u = 0; u < UPL; ++u)
#pragma unroll
        for (int i = 0; i < 16; ++i) a = fmaxf(a, fabsf(f[u][i]));
    // |v| >= 0, so the float order is the order of the bit patterns
    a = __uint_as_float(wave_max_u32(__float_as_uint(a)));
    const float inv = rule_inv<RULE>(a);
#pragma unroll
    for (int u = 0; u < UPL; ++u) {
        const int un = lane + 64 * u;
        uint32_t w[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) w[i] = rule_pack4<RULE>(&f[u][4 * i], inv, a > 0.f);
        if (un < units)
            *reinterpret_cast<uint4 *>(q + ((size_t)mt * S + (un >> 2)) * 8192 +
                                       (size_t)(64 * (ti >> 4) + 16 * (un & 3) + (ti & 15)) * 16) =
                make_uint4(w[0], w[1], w[2], w[3]);
    }
    if (lane == 0) scale[row] = rule_scale<RULE>(a);
}

// ------------------------------------------------------------------------------------------
// Grouped int8 GEMMs
// ------------------------------------------------------------------------------------------

typedef __attribute__((__vector_size__(4 * sizeof(int)))) int i32x4v;
typedef __attribute__((__vector_size__(16 * sizeof(int)))) int i32x16v;
typedef _Float16 f16x8v __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2v __attribute__((ext_vector_type(2)));


constexpr int GG_BM = 128;

// Grouped int8 GEMM over the permuted pairs of one expert group per block.
//  MODE_GU (gate/up): block = (N-tile nt: gate columns 64nt..64nt+63 and the same up columns,
//           global M-tile); A = quantised x rows gathered through perm, K = d_model; epilogue
//           g = sx * s_gate * acc, u likewise, h = silu(g) * u (fp32, permuted row order).
//  MODE_DN (down): block = (N-tile of 128 outputs, global M-tile); A = quantised h in M-tile
//           order (Q_TILES: one contiguous 8 KB block per 64-wide K super-block), K = d_ff;
//           epilogue y = sh * s_down * acc (fp32 per pair row).
// Block tile 128 x 128, K step 64, 4 waves as 2 x 2 tiles of 64 x 64, each 2 x 2 sub-tiles of
// v_mfma_i32_32x32x32_i8 (8 MFMAs per step; this shape runs the int8 matrix cores well above the
// 16x16x64 one).  The down GEMM on per-row int8 tiled weights (BD) splits the block's N among the
// waves instead (4 x 1 sub-tiles of all 128 rows by 32 columns each): B then has one reader, so
// its fragments go from global memory straight into registers and LDS holds only A (down 112.1 ->
// 106.7 us on the Gemma-shaped prefill, 168 VGPRs and three blocks per CU instead of 182 and two;
// the same for gate/up measured 158 -> 172 us and is not used there).  LDS holds a K step of A (8 tiles of 16 rows) and B (8 tiles of 16 weight rows)
// in the tiled weight order: lane (n, g) of a 16-row tile owns K offsets 8g..8g+7 and
// 32+8g..32+8g+7 of row n, 16 bytes.  An MFMA lane l (row l % 32, half l / 32) takes, in K
// half-step ks, the 16 bytes of slot (n = l % 16, g = l / 32 + 2 ks) of tile (l % 32) / 16: A and B
// use the same K order, so every fragment is one ds_read_b128.  Thread c (of 512 per step and operand)
// fills exactly the 16 bytes at LDS offset 16c, so the LDS writes are contiguous (conflict-free);
// A (in slot or tile order from the quantiser) and tiled B are read as one 16-byte piece, plain B
// as the two 8-byte pieces of that slot.  Global loads run two K steps ahead of the MFMAs (two
// register stages, LDS double buffered).  Rows past the tile's pair count and tiles past the
// weight matrix read valid addresses (the tile's last row or unwritten tile codes, the last
// weight tile); their results are never stored.
enum { MODE_GU = 0, MODE_DN = 1 };

// 64-byte super-blocks per K step and the occupancy target (two blocks per CU fit the LDS).
// Measured on the Gemma-shaped prefill (T = 2048, per-row int8 tiled), gate/up / down: one
// register stage 200 / 158 us, two 171 / 123, three 177 / 127; one super-block per step with
// three blocks per CU: 175 / 119.
constexpr int GG_KS = 2, GG_WPE = 2;

// DMA variant (tiled weights): operands go from global memory straight into LDS
// (global_load_lds_dwordx4: lane l's 16 bytes land at the wave's base + 16 l, which is the slot
// order above), through a ring of GD_NB stages of one super-block each; no register staging and no
// LDS store instructions.  Every stage issues the same loads (past the end of K the last
// super-block is re-read into a buffer nobody reads), so the wait for the oldest stage is one
// constant vmcnt.  Three stages (48 KB) let three blocks share a CU with ~115-225 VGPRs each.
// Measured on the Gemma-shaped prefill (T = 2048, tiled), gate/up / down us, register stages vs
// this ring of 3 / 4 stages: per-row int8 170 / 110 vs 181 / 122, 185 / 138; Q8_0 284 / 153 vs
// 252 / 133, 273 / 149; E4M3 220 / 132 vs 201 / 135, 217 / 156.  The kinds whose K steps carry
// VALU work (Q8_0 block scaling, E4M3 widening) take the ring; per-row int8 keeps register stages.
constexpr int GD_NB = 3;

// One direct-to-LDS load per lane: 16 (or 4) bytes from g to LDS byte address lds + 16 l (4 l) for
// lane l; lds must be the same in every lane.  Written as asm so that the compiler, which cannot
// tell the ring's stages apart, does not wait for every outstanding load before each LDS read;
// the K loop orders them itself (vmcnt and a barrier).  M0 -> LDS-DMA needs one wait state.
__device__ __forceinline__ void lds_dma16(const void *g, uint32_t lds)
{
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
                 :: "s"(__builtin_amdgcn_readfirstlane(lds)), "v"(g) : "memory", "m0");
}
__device__ __forceinline__ void lds_dma4(const void *g, uint32_t lds)
{
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, off"
                 :: "s"(__builtin_amdgcn_readfirstlane(lds)), "v"(g) : "memory", "m0");
}
template <typename T>
__device__ __forceinline__ uint32_t lds_addr(T *p)
{
    return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) T *)p;
}

// One K step of this thread's global loads: 16-byte slot q (A slot c = tid + 256 (q % 2) of
// super-block q / 2) in elements 4q .. 4q + 3.  Vector values, not arrays, so that the stages stay
// in registers when they alternate roles.
typedef uint32_t u32x16v __attribute__((ext_vector_type(4 * 2 * GG_KS)));
typedef float f32x16v __attribute__((ext_vector_type(16)));
struct GStage {
    u32x16v a, b;
    uint32_t sc;          // Q8_0: the two fp16 block scales of one (weight tile, super-block, row)
};
__device__ __forceinline__ void put16(u32x16v &v, int q, uint4 x)
{
    v[4 * q] = x.x; v[4 * q + 1] = x.y; v[4 * q + 2] = x.z; v[4 * q + 3] = x.w;
}
__device__ __forceinline__ uint4 get16(const u32x16v &v, int q)
{
    return make_uint4(v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]);
}

// Q8 (Q8_0 weights): every MFMA covers exactly one 32-wide Q8_0 block (K offsets 32 blk + 16 h ..
// +15 for lane half h, gathered from the low or high 8 bytes of slots 2h and 2h + 1), starts from
// zero, and its int32 result is scaled by the block's fp16 weight scale into fp32 accumulators;
// the epilogue then applies the activation scale only.  The block scales of a step (8 weight tiles
// x 2 super-blocks x 16 rows, one 32-bit pair each) are loaded with the step, one per thread,
// and staged in LDS with it.
// F8 (E4M3 per-row weights and E4M3 activations): a lane's two 16-byte slots of a super-block (the
// int8 path's K half-steps ks 0 and 1) are widened to f16 by v_cvt_scalef32_pk_f16_fp8 with scale
// 1 (exact: every E4M3 value is an f16 normal) and fed, 8 codes at a time, to four
// v_mfma_f32_32x32x16_f16 per sub-tile, A and B alike, so both see the same K order.  The f16
// matrix cores add the exact products in fp32; the epilogue applies both row scales.  (The gfx950
// E4M3 instruction v_mfma_f32_32x32x64_f8f6f4 was measured to drop, within each 8-code group of
// a lane, products more than 13 bits below the group's largest: ~1e-5..1e-4 relative error on
// these dot products, which re-quantising h turns into output errors of several 1e-3.)
enum { WK_I8ROW = 0, WK_Q8 = 1, WK_F8ROW = 2 };

template <int MODE, int LAYOUT, int WK, bool DMA>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(GG_WPE))) void ggemm_i8_kernel(
    const int8_t *__restrict__ A, const float *__restrict__ a_scale, int K, int k,
    const int8_t *__restrict__ W, const void *__restrict__ w_scale, int NR,
    const int4 *__restrict__ tiles, const int32_t *__restrict__ perm,
    const int32_t *__restrict__ tile_off, int E, int mt_bound, float *__restrict__ out)
{
    constexpr bool Q8 = WK == WK_Q8, F8 = WK == WK_F8ROW;
    static_assert(!DMA || LAYOUT == L_TILED, "direct LDS loads need 16-byte weight slots");
    constexpr int SBB = 8192;                        // bytes of one operand's super-block
    constexpr int KS = DMA ? 1 : GG_KS;              // super-blocks per K step
    constexpr int NBUF = DMA ? GD_NB : 2;            // LDS stages
    // BD (down, per-row int8, tiled, through registers): the 4 waves split N instead of M and B
    // skips LDS (see the BD notes below); LDS then holds A only
    constexpr bool BD = MODE == MODE_DN && LAYOUT == L_TILED && !DMA && WK == WK_I8ROW;
    __shared__ __attribute__((aligned(16))) int8_t lds[NBUF][(BD ? 1 : 2) * KS * SBB];
    __shared__ float s_rowscale[GG_BM];
    __shared__ uint32_t s_wsc[Q8 ? NBUF * 256 : 1];  // per stage: (weight tile, super-block, row)
    // Block order: XCD x (blocks are dealt to the 8 XCDs round robin) takes the x-th eighth of the
    // valid M-tiles with all of their N-tiles, N fastest, so an M-tile's activation rows are
    // fetched into one L2 and reused by its N-tiles, and an expert's M-tiles share that L2 too.
    const int MT = tile_off[E];                      // valid M-tiles
    const int NNT = gridDim.x / mt_bound;            // N-tiles
    int mt, nt;
    {
        const int G = gridDim.x;
        if ((G & 7) == 0) {
            const int x = blockIdx.x & 7, local = blockIdx.x >> 3;
            const int mt0 = (x * MT) >> 3, mt1 = ((x + 1) * MT) >> 3;
            mt = mt0 + local / NNT;
            nt = local - (local / NNT) * NNT;
            if (mt >= mt1) return;                   // uniform across the block
        } else {
            nt = blockIdx.x / mt_bound;
            mt = blockIdx.x - nt * mt_bound;
            if (mt >= MT) return;
        }
    }
    const int4 ti = tiles[mt];                       // {expert, first permuted row, rows, 0}
    const int e = ti.x, r_begin = ti.y, rows = ti.z;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int wm = BD ? 0 : wave >> 1, wn = wave & 1;
    const int S = K >> 6;                            // super-blocks
    const int NS = (S + KS - 1) / KS;                // K steps
    // NR = d_ff (gate/up) or d_model (down)
    const int OT = NR >> 4;                          // 16-row weight tiles per half / per matrix

    // ---- this thread's slots: c = tid + 256 c2 -> tile c / 64, lane (n, g) = (c % 16, c / 16 % 4)
    // The epilogue's scales are loaded now, behind the main loop: the activation scale of row
    // tid < 128 (kept in a register until the loop is done) and this lane's weight-row scales.
    const int col = lane & 31;
    float rscale = 0.f, cscale[2];
    if (tid < GG_BM) {
        const int r = min(tid, rows - 1);
        rscale = MODE == MODE_GU ? a_scale[perm[r_begin + r] / k] : a_scale[r_begin + r];
    }
    const float *wsf = reinterpret_cast<const float *>(w_scale);
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) {
        if (BD)                       // this lane's column: gate / up feature, or output
            cscale[ct] = MODE == MODE_GU
                             ? wsf[(size_t)e * 2 * NR + ((lane >> 4) & 1) * NR + 64 * nt + 16 * wave + (lane & 15)]
                             : wsf[(size_t)e * NR + min(128 * nt + 32 * wave + col, NR - 1)];
        else if (Q8)                  // (per-block scales, applied in the K loop)
            cscale[ct] = 1.f;
        else if (MODE == MODE_GU)     // gate (ct 0) and up (ct 1) scales of weight row f
            cscale[ct] = wsf[(size_t)e * 2 * NR + ct * NR + 64 * nt + 32 * wn + col];
        else
            cscale[ct] = wsf[(size_t)e * NR + min(128 * nt + 64 * wn + 32 * ct + col, NR - 1)];
    }
    // Q8: this thread's scale word: weight tile ts, super-block js of the step, row ns = tid % 16
    // of the tile, at word tid of the stage (one super-block per step: threads 128.. repeat 0..)
    const uint32_t *sc_src = nullptr;
    size_t sc_step = 0;
    const int ts = (tid >> (KS == 2 ? 5 : 4)) & 7, js = KS == 2 ? (tid >> 4) & 1 : 0, ns = tid & 15;
    if (Q8) {
        const uint32_t *s32 = reinterpret_cast<const uint32_t *>(w_scale);
        const int wrt = MODE == MODE_GU ? 4 * nt + (ts & 3) : min(8 * nt + ts, OT - 1);
        const int hf = MODE == MODE_GU ? ts >> 2 : 0;
        const int M = MODE == MODE_GU ? 2 : 1;
        if (LAYOUT == L_TILED) {      // 32 fp16 per (tile, super-block), row n's two at 2n
            sc_src = s32 + (((size_t)e * OT + wrt) * S * M + hf) * 16 + ns;
            sc_step = (size_t)M * 16;
        } else {                      // [rows][K / 32] fp16: blocks 2 sb, 2 sb + 1 of the row
            const size_t row = (size_t)e * (M * NR) + (size_t)hf * NR + 16 * wrt + ns;
            sc_src = s32 + row * (K >> 6);
            sc_step = 1;
        }
    }

    // Gate/up activations through registers (KS = 2): a step's two super-blocks of a row are one
    // 128-byte line, so load i of a thread takes row 8 (wave + 4 i) + lane % 8 and its 16-byte piece
    // lane / 8 of the line (super-block lane / 32, group lane / 8 % 4): every load instruction
    // covers eight whole lines, and the eight lanes of a piece write eight consecutive LDS slots.
    constexpr bool LINES = MODE == MODE_GU && !DMA && KS == 2;
    const int8_t *a_row[LINES ? 4 : 1];
    int a_lds[LINES ? 4 : 1];                        // the LDS byte offset of load i's slot
    if (LINES) {
        const int pj = lane >> 5, pg = (lane >> 3) & 3;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = 8 * (wave + 4 * i) + (lane & 7);
            a_row[i] = A + (size_t)(perm[r_begin + min(row, rows - 1)] / k) * K + 16 * pg;
            a_lds[i] = pj * SBB + (64 * (row >> 4) + 16 * pg + (row & 15)) * 16;
        }
    }
    const int8_t *a_src[2];
    const int8_t *b_src[2];
#pragma unroll
    for (int c2 = 0; c2 < 2; ++c2) {
        const int c = tid + 256 * c2;
        const int t = c >> 6, n = c & 15, g = (c >> 4) & 3;
        const int r = min(16 * t + n, rows - 1);
        // gate/up: x rows in slot order (quantize_rows_kernel, Q_SLOTS), the lane's 16 bytes of a
        // 64-column block at 16 g
        if (LINES)
            a_src[c2] = nullptr;
        else if (MODE == MODE_GU)
            a_src[c2] = A + (size_t)(perm[r_begin + r] / k) * K + 16 * g;
        else                                         // the tile's codes (quantize_rows_kernel, Q_TILES)
            a_src[c2] = A + (size_t)mt * S * 8192 + (size_t)c * 16;
        int wrow_tile;                               // global 16-row weight tile index
        int half_off = 0;                            // gate/up half
        if (MODE == MODE_GU) {
            wrow_tile = 4 * nt + (t & 3);
            half_off = t >> 2;
        } else {
            wrow_tile = min(8 * nt + t, OT - 1);
        }
        if (LAYOUT == L_TILED) {
            const int M = MODE == MODE_GU ? 2 : 1;
            b_src[c2] = W + ((((size_t)e * OT + wrow_tile) * S) * M + half_off) * 1024 + (c & 63) * 16;
        } else {
            const size_t row = (size_t)e * (MODE == MODE_GU ? 2 * NR : NR) + (size_t)half_off * NR + 16 * wrow_tile + n;
            b_src[c2] = W + row * K + 8 * g;
        }
    }
    const size_t b_step = LAYOUT == L_TILED ? (MODE == MODE_GU ? 2048 : 1024) : 64;
    // BD: wave w multiplies all 128 rows by one 32-column tile pair, gate / up: the gate (lanes
    // with l % 32 < 16) and up rows of features 64 nt + 16 w .. + 15; down: output tiles 8 nt + 2 w
    // and + 1.  Its lanes load, per super-block and K half-step ks, the 16 bytes of slot
    // (l / 32 + 2 ks) * 16 + l % 16 of their tile (what they read from LDS otherwise) straight
    // into their MFMA operand: B is used by one wave only, so it needs no LDS.
    const int8_t *bd_src = nullptr;
    if (BD) {
        const int tb = (lane >> 4) & 1, M = MODE == MODE_GU ? 2 : 1;
        const int wrt = MODE == MODE_GU ? 4 * nt + wave : min(8 * nt + 2 * wave + tb, OT - 1);
        const int hof = MODE == MODE_GU ? tb : 0;
        bd_src = W + ((((size_t)e * OT + wrt) * S) * M + hof) * 1024 + ((lane >> 5) * 16 + (lane & 15)) * 16;
    }

    // step st covers super-blocks st * KS + j; past the end of K the last one is re-read (unused)
    auto gload = [&](GStage &R, int st) {
        if (Q8) R.sc = sc_src[(size_t)min(st * KS + js, S - 1) * sc_step];
        if (LINES) {
            // this lane's super-block of the step (the last one re-read past the end of K)
            const size_t off = (size_t)64 * min(st * KS + (lane >> 5), S - 1);
#pragma unroll
            for (int i = 0; i < 4; ++i) put16(R.a, i, *reinterpret_cast<const uint4 *>(a_row[i] + off));
        }
#pragma unroll
        for (int j = 0; j < KS; ++j) {
            const size_t sb = min(st * KS + j, S - 1);
#pragma unroll
            for (int c2 = 0; c2 < 2; ++c2) {
                if (!LINES)
                    put16(R.a, 2 * j + c2, *reinterpret_cast<const uint4 *>(a_src[c2] + sb * (MODE == MODE_GU ? 64 : 8192)));
                if (BD) {                     // (c2 is the K half-step here)
                    put16(R.b, 2 * j + c2, *reinterpret_cast<const uint4 *>(bd_src + sb * b_step + 512 * c2));
                } else if (LAYOUT == L_TILED) {
                    put16(R.b, 2 * j + c2, *reinterpret_cast<const uint4 *>(b_src[c2] + sb * b_step));
                } else {
                    const uint2 blo = *reinterpret_cast<const uint2 *>(b_src[c2] + sb * 64);
                    const uint2 bhi = *reinterpret_cast<const uint2 *>(b_src[c2] + sb * 64 + 32);
                    put16(R.b, 2 * j + c2, make_uint4(blo.x, blo.y, bhi.x, bhi.y));
                }
            }
        }
    };
    auto lstore = [&](const GStage &R, int buf) {
        int8_t *L = lds[buf];
        if (Q8) s_wsc[buf * 256 + tid] = R.sc;
#pragma unroll
        for (int j = 0; j < KS; ++j)
#pragma unroll
            for (int c2 = 0; c2 < 2; ++c2) {
                if (LINES)
                    *reinterpret_cast<uint4 *>(L + a_lds[2 * j + c2]) = get16(R.a, 2 * j + c2);
                else
                    *reinterpret_cast<uint4 *>(L + j * SBB + (tid + 256 * c2) * 16) = get16(R.a, 2 * j + c2);
                if (!BD)
                    *reinterpret_cast<uint4 *>(L + (KS + j) * SBB + (tid + 256 * c2) * 16) = get16(R.b, 2 * j + c2);
            }
    };
    // DMA: super-block st (clamped) into stage st % NBUF; each call is 4 loads (5 with Q8 scales)
    auto issue = [&](int st) {
        const size_t sb = min(st, S - 1);
        const uint32_t L = lds_addr(lds[st % NBUF]);
#pragma unroll
        for (int c2 = 0; c2 < 2; ++c2) {
            lds_dma16(a_src[c2] + sb * (MODE == MODE_GU ? 64 : 8192), L + (64 * wave + 256 * c2) * 16);
            lds_dma16(b_src[c2] + sb * b_step, L + SBB + (64 * wave + 256 * c2) * 16);
        }
        if (Q8) lds_dma4(sc_src + sb * sc_step, lds_addr(s_wsc + (st % NBUF) * 256 + 64 * wave));
    };
    // 32-row B sub-tiles this wave multiplies (pairs of 16-row tiles): gate/up: ct 0 = gate tiles
    // 2wn, 2wn+1, ct 1 = up tiles 4+2wn, 5+2wn; down: ct = tiles 4wn+2ct, 4wn+2ct+1.
    int btile[2];
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) btile[ct] = MODE == MODE_GU ? (4 * ct + 2 * wn) : (4 * wn + 2 * ct);

    i32x16v acc[2][2];
    f32x16v accf[2][2];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
        for (int ct = 0; ct < 2; ++ct)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                acc[rt][ct][r] = 0;
                accf[rt][ct][r] = 0.f;
            }

    const int half = lane >> 5, l16 = lane & 15, t16 = (lane >> 4) & 1;
    // TAIL: the last K step, which may hold fewer than GG_KS super-blocks.  Full steps have no
    // branch, so the next step's global loads stay ahead of the MFMAs in one basic block.
    auto compute = [&](int buf, int st, auto tail, const u32x16v &bcur) {
        const int8_t *L = lds[buf];
#pragma unroll
        for (int j = 0; j < KS; ++j) {
            if (decltype(tail)::value && st * KS + j >= S) break;
            if (BD) {
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) {
                    const int slot = (half + 2 * ks) * 16 + l16;
                    const uint4 bv = get16(bcur, 2 * j + ks);
                    const i32x4v b = i32x4v{(int)bv.x, (int)bv.y, (int)bv.z, (int)bv.w};
#pragma unroll
                    for (int rt = 0; rt < 4; ++rt) {
                        const uint4 v = *reinterpret_cast<const uint4 *>(L + j * SBB + ((2 * rt + t16) * 64 + slot) * 16);
                        const i32x4v a = i32x4v{(int)v.x, (int)v.y, (int)v.z, (int)v.w};
                        acc[rt >> 1][rt & 1] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, acc[rt >> 1][rt & 1], 0, 0, 0);
                    }
                }
                continue;
            }
            if (Q8) {
#pragma unroll
                for (int blk = 0; blk < 2; ++blk) {
                    i32x4v a[2], b[2];
                    auto frag = [&](int sbase, int tile) {
                        const uint2 lo = *reinterpret_cast<const uint2 *>(L + sbase + (tile * 64 + (2 * half) * 16 + l16) * 16 + 8 * blk);
                        const uint2 hi = *reinterpret_cast<const uint2 *>(L + sbase + (tile * 64 + (2 * half + 1) * 16 + l16) * 16 + 8 * blk);
                        return i32x4v{(int)lo.x, (int)lo.y, (int)hi.x, (int)hi.y};
                    };
#pragma unroll
                    for (int rt = 0; rt < 2; ++rt) a[rt] = frag(j * SBB, 4 * wm + 2 * rt + t16);
                    float sc[2];
#pragma unroll
                    for (int ct = 0; ct < 2; ++ct) {
                        b[ct] = frag((KS + j) * SBB, btile[ct] + t16);
                        const uint32_t w2 = s_wsc[buf * 256 + ((btile[ct] + t16) * KS + j) * 16 + l16];
                        sc[ct] = half_bits_to_float(blk ? (w2 >> 16) : (w2 & 0xFFFFu));
                    }
                    const i32x16v z = {};
#pragma unroll
                    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
                        for (int ct = 0; ct < 2; ++ct) {
                            const i32x16v p = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[rt], b[ct], z, 0, 0, 0);
                            accf[rt][ct] += __builtin_convertvector(p, f32x16v) * sc[ct];
                        }
                }
                continue;
            }
            if (F8) {
                const int s0 = half * 16 + l16, s1 = (half + 2) * 16 + l16;
                uint4 a[2][2], b[2][2];
#pragma unroll
                for (int rt = 0; rt < 2; ++rt) {
                    const int8_t *base = L + j * SBB + (4 * wm + 2 * rt + t16) * 64 * 16;
                    a[rt][0] = *reinterpret_cast<const uint4 *>(base + s0 * 16);
                    a[rt][1] = *reinterpret_cast<const uint4 *>(base + s1 * 16);
                }
#pragma unroll
                for (int ct = 0; ct < 2; ++ct) {
                    const int8_t *base = L + (KS + j) * SBB + (btile[ct] + t16) * 64 * 16;
                    b[ct][0] = *reinterpret_cast<const uint4 *>(base + s0 * 16);
                    b[ct][1] = *reinterpret_cast<const uint4 *>(base + s1 * 16);
                }
                // 8 codes (two dwords) -> 8 f16, code i in element i
                auto widen = [](uint32_t lo, uint32_t hi) {
                    const f16x2v p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(lo, 1.0f, false);
                    const f16x2v p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(lo, 1.0f, true);
                    const f16x2v p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(hi, 1.0f, false);
                    const f16x2v p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(hi, 1.0f, true);
                    return f16x8v{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
                };
                auto piece = [&](const uint4 (&f)[2], int i) {      // codes 8i .. 8i + 7 of the 32
                    const uint4 &v = f[i >> 1];
                    return (i & 1) ? widen(v.z, v.w) : widen(v.x, v.y);
                };
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    f16x8v ah[2], bh[2];
#pragma unroll
                    for (int rt = 0; rt < 2; ++rt) ah[rt] = piece(a[rt], i);
#pragma unroll
                    for (int ct = 0; ct < 2; ++ct) bh[ct] = piece(b[ct], i);
#pragma unroll
                    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
                        for (int ct = 0; ct < 2; ++ct)
                            accf[rt][ct] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ah[rt], bh[ct], accf[rt][ct], 0, 0, 0);
                }
                continue;
            }
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                const int slot = (half + 2 * ks) * 16 + l16;
                i32x4v a[2], b[2];
#pragma unroll
                for (int rt = 0; rt < 2; ++rt) {
                    const uint4 v = *reinterpret_cast<const uint4 *>(L + j * SBB + ((4 * wm + 2 * rt + t16) * 64 + slot) * 16);
                    a[rt] = i32x4v{(int)v.x, (int)v.y, (int)v.z, (int)v.w};
                }
#pragma unroll
                for (int ct = 0; ct < 2; ++ct) {
                    const uint4 v = *reinterpret_cast<const uint4 *>(L + (KS + j) * SBB + ((btile[ct] + t16) * 64 + slot) * 16);
                    b[ct] = i32x4v{(int)v.x, (int)v.y, (int)v.z, (int)v.w};
                }
#pragma unroll
                for (int rt = 0; rt < 2; ++rt)
#pragma unroll
                    for (int ct = 0; ct < 2; ++ct)
                        acc[rt][ct] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[rt], b[ct], acc[rt][ct], 0, 0, 0);
            }
        }
    };

    // The barrier between K steps only orders LDS (its own lgkmcnt wait): __syncthreads() would
    // also wait for every outstanding global load and so drain the prefetch.  The LDS stores wait
    // for just the loads they store (the compiler's vmcnt for those registers).  Loads are issued
    // unconditionally, so the wait counts do not depend on the path taken.
    auto lds_barrier = [] { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); };
    // Two register stages: during step st the loads of steps st + 1 (issued a step earlier) and
    // st + 2 are in flight.  Rf holds a step already in LDS (free), Rp the pending step st + 1.
    auto step = [&](GStage &Rf, GStage &Rp, int st) {
        const u32x16v bcur = Rf.b;                   // BD: step st's B, before Rf takes step st + 2
        gload(Rf, st + 2);
        compute(st & 1, st, std::false_type{}, bcur);
        lstore(Rp, (st + 1) & 1);
        // schedule: the global loads, then the MFMAs, then the LDS stores
        __builtin_amdgcn_sched_group_barrier(0x020, 4 * KS + (Q8 ? 1 : 0), 0);
        __builtin_amdgcn_sched_group_barrier(0x008, (F8 ? 16 : 8) * KS, 0);
        __builtin_amdgcn_sched_group_barrier(0x200, (BD ? 2 : 4) * KS + (Q8 ? 1 : 0), 0);
        lds_barrier();
    };
    if (DMA) {
        // stage st's loads are the oldest in flight; NBUF - 2 newer stages may stay outstanding
        constexpr int LPS = Q8 ? 5 : 4;
        static_assert(LPS * (NBUF - 2) < 64, "vmcnt field");
#pragma unroll
        for (int i = 0; i < NBUF - 1; ++i) issue(i);
        for (int st = 0; st < NS; ++st) {
            // this wave's loads of stage st have landed; after the barrier every wave's have, and
            // every wave is done reading stage st - 1, which the next issue overwrites
            asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(LPS * (NBUF - 2)) : "memory");
            issue(st + NBUF - 1);
            compute(st % NBUF, st, std::false_type{}, u32x16v{});
        }
        // no load may still be writing this block's LDS when it exits
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    } else {
        GStage R0, R1;
        gload(R0, 0);
        gload(R1, 1);
        lstore(R0, 0);
        lds_barrier();
        int st = 0;
        for (; st + 2 < NS; st += 2) {      // steps st and st + 1, both followed by another
            step(R0, R1, st);
            step(R1, R0, st + 1);
        }
        if (st + 1 < NS) step(R0, R1, st);
        // step NS - 1's operands are in R0 or R1 by its parity
        compute((NS - 1) & 1, NS - 1, std::true_type{}, ((NS - 1) & 1) ? R1.b : R0.b);
    }

    // ---- epilogue: lane l, register r of a 32 x 32 sub-tile holds
    //      C[8 (r / 4) + 4 (l / 32) + r % 4][l % 32]; only stores remain conditional
    if (tid < GG_BM) s_rowscale[tid] = rscale;
    __syncthreads();
    if (BD) {
        // sub-tile rt = 2 i + j of acc[i][j] holds rows 32 rt ..; lane column col: gate / up
        // halves of this wave's 16 features (up in the lane 16 above), or outputs
#pragma unroll
        for (int rt = 0; rt < 4; ++rt)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int rr = 32 * rt + 8 * (r >> 2) + 4 * half + (r & 3);
                const size_t row = (size_t)(r_begin + rr);
                const float v = (float)acc[rt >> 1][rt & 1][r] * s_rowscale[rr] * cscale[0];
                if (MODE == MODE_GU) {
                    const float u = __shfl_xor(v, 16, WAVE);
                    if (t16 == 0 && rr < rows) out[row * NR + 64 * nt + 16 * wave + l16] = silu_f32(v) * u;
                } else {
                    const int o = 128 * nt + 32 * wave + col;
                    if (rr < rows && o < NR) out[row * NR + o] = v;
                }
            }
        return;
    }
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int rr = 64 * wm + 32 * rt + 8 * (r >> 2) + 4 * half + (r & 3);
            const float rs = s_rowscale[rr];
            const size_t row = (size_t)(r_begin + rr);
            if (MODE == MODE_GU) {
                const int f = 64 * nt + 32 * wn + col;
                const float g = Q8 ? accf[rt][0][r] * rs
                                   : (F8 ? accf[rt][0][r] : (float)acc[rt][0][r]) * rs * cscale[0];
                const float u = Q8 ? accf[rt][1][r] * rs
                                   : (F8 ? accf[rt][1][r] : (float)acc[rt][1][r]) * rs * cscale[1];
                if (rr < rows) out[row * NR + f] = silu_f32(g) * u;
            } else {
#pragma unroll
                for (int ct = 0; ct < 2; ++ct) {
                    const int o = 128 * nt + 64 * wn + 32 * ct + col;
                    if (rr < rows && o < NR)
                        out[row * NR + o] = Q8 ? accf[rt][ct][r] * rs
                                               : (F8 ? accf[rt][ct][r] : (float)acc[rt][ct][r]) * rs * cscale[ct];
                }
            }
        }
}

int prefill_tile_rows() { return GG_BM; }

int prefill_tile_bound(int P, int E)
{
    const int b = P / GG_BM + min(E, P);
    return (b + 7) & ~7;
}

template <int MODE>
static void launch_ggemm(dim3 g, hipStream_t s, const int8_t *a, const float *sa, int K, int k, const ExpertsDev &ex,
                         const int8_t *w, const void *sc, int NR, const PermuteOut &po, int mtb, float *out)
{
#define GG(L, Q) hipLaunchKernelGGL((ggemm_i8_kernel<MODE, L, Q, L == L_TILED && Q != WK_I8ROW>), g, dim3(256), 0, s, \
                                    a, sa, K, k, w, sc, NR, \
                                    po.tiles, po.perm, po.tile_off, ex.E, mtb, out)
    switch (ex.fmt) {
    case W_I8_ROW_TILED: GG(L_TILED, WK_I8ROW); break;
    case W_Q8_0_TILED: GG(L_TILED, WK_Q8); break;
    case W_Q8_0: GG(L_PLAIN, WK_Q8); break;
    case W_FP8_ROW_TILED: GG(L_TILED, WK_F8ROW); break;
    case W_FP8_ROW: GG(L_PLAIN, WK_F8ROW); break;
    default: GG(L_PLAIN, WK_I8ROW); break;
    }
#undef GG
}

hipError_t launch_ggemm_gateup_i8(const int8_t *xq, const float *sx, int T, int k, const ExpertsDev &ex,
                                  const PermuteOut &po, float *h, hipStream_t s)
{
    const int mtb = prefill_tile_bound(T * k + ex.S * T, ex.E + ex.S);   // routed and shared tiles
    ProfScope ps(K_GG_GATEUP, s);
    launch_ggemm<MODE_GU>(dim3(mtb * (ex.d_ff / 64)), s, xq, sx, ex.d_model, k, ex,
                          reinterpret_cast<const int8_t *>(ex.gate_up), ex.gate_up_scales, ex.d_ff, po, mtb, h);
    return hipGetLastError();
}

hipError_t launch_ggemm_down_i8(const int8_t *hq, const float *sh, int T, int k, const ExpertsDev &ex,
                                const PermuteOut &po, float *ybuf, hipStream_t s)
{
    const int mtb = prefill_tile_bound(T * k + ex.S * T, ex.E + ex.S);   // routed and shared tiles
    ProfScope ps(K_GG_DOWN, s);
    launch_ggemm<MODE_DN>(dim3(mtb * ((ex.d_model + 127) / 128)), s, hq, sh, ex.d_ff, k, ex,
                          reinterpret_cast<const int8_t *>(ex.down), ex.down_scales, ex.d_model, po, mtb, ybuf);
    return hipGetLastError();
}

template <int RULE>
static void launch_qrows(const void *v, int xtype, int rows, int cols, int8_t *q, float *scale, bool slot_order,
                         hipStream_t s)
{
#define QR(X, L, CH) hipLaunchKernelGGL((quantize_rows_kernel<RULE, X, L, CH>), dim3(rows), dim3(256), 0, s, v, cols, \
                                        q, scale)
#define QR2(X, L) do { if (cols <= 4096) QR(X, L, 4); else QR(X, L, 16); } while (0)
    if (xtype == X_BF16) { if (slot_order) QR2(X_BF16, Q_SLOTS); else QR2(X_BF16, Q_COLS); }
    else { if (slot_order) QR2(X_F32, Q_SLOTS); else QR2(X_F32, Q_COLS); }
#undef QR2
#undef QR
}

hipError_t launch_quantize_rows(const void *v, int xtype, int rows, int cols, int8_t *q,
                                float *scale, bool slot_order, bool fp8, hipStream_t s)
{
    ProfScope ps(K_QUANT, s);
    if (fp8) launch_qrows<R_F8>(v, xtype, rows, cols, q, scale, slot_order, s);
    else launch_qrows<R_I8>(v, xtype, rows, cols, q, scale, slot_order, s);
    return hipGetLastError();
}

size_t prefill_h_tiles_bytes(int P, int E, int d_ff) { return (size_t)prefill_tile_bound(P, E) * GG_BM * d_ff; }

hipError_t launch_quantize_h_tiles(const float *h, int T, int k, int E, int S, int d_ff, const PermuteOut &po,
                                   int8_t *q, float *scale, bool fp8, hipStream_t s)
{
    ProfScope ps(K_QUANT, s);
    // the grid covers the tile bound of the routed and shared rows; the tile count is at tile_off[E]
    const dim3 g((unsigned)prefill_tile_bound(T * k + S * T, E + S) * (GG_BM / 4));
#define QH(R, U) hipLaunchKernelGGL((quantize_h_tiles_kernel<R, U>), g, dim3(256), 0, s, h, d_ff, q, scale, \
                                    po.tiles, po.tile_off, E)
#define QH2(R) do { if (d_ff <= 1024) QH(R, 1); else if (d_ff <= 4096) QH(R, 4); else QH(R, 16); } while (0)
    if (fp8) QH2(R_F8);
    else QH2(R_I8);
#undef QH2
#undef QH
    return hipGetLastError();
}

}  // namespace moe
