// Q8_0 and per-row-int8 expert FFN on the gfx950 bf16 matrix cores.
//
// Gate/up (the mul_mat_id over the stacked [n_embd, 2*n_ff, n_experts] tensor followed by
// fused_mul_unary(gate, up, SILU) of "Running Gemma 4 26B at 5 tokens/s on a 13-year-old Xeon",
// "Three-part fix"; or the ungated ReLU^2 up of the Nemotron page, "bytes per token") and down +
// weighted combine (the fixed-order per-(token, expert) sum of the Nemotron page, "How
// correctness is checked").
//
// Decode batches are small (a handful of tokens per expert) and the layer is a weight stream, so
// each workgroup streams a 16-row tile of one expert's matrix exactly once and multiplies it by
// every token routed to that expert with v_mfma_f32_16x16x32_bf16: A = 16 tokens x 32 K
// activations, B = 32 K x 16 weight rows.  One MFMA spans exactly one Q8_0 block, so its result
// is scaled by that block's fp16 scale before accumulation.  int8 weights and bf16 activations
// are exact in bf16; fp32 inputs (fp32 x, the fp32 h of the down projection) are split into two
// or three bf16 terms, so all products are exact and accumulate in fp32.
#include "moe_common.hpp"
#include "moe_launch.hpp"
#include "route_dev.hpp"

namespace moe {

// Loads the A operand (8 consecutive activations of one token) as NT bf16x8 terms.
// PX: only lanes of a valid row load (the others are masked off); otherwise the load is
// unconditional (off must address valid memory).  Either way an invalid row becomes zeros.
template <int XT, int NT, bool PX>
__device__ __forceinline__ void load_x8(const void *__restrict__ x, size_t off, bool valid,
                                        bf16x8 *a)
{
    if (XT == X_BF16) {
        U4 t;
        if (PX) {
            t.u = make_uint4(0, 0, 0, 0);
            if (valid) t.u = *reinterpret_cast<const uint4 *>(reinterpret_cast<const uint16_t *>(x) + off);
        } else {
            t.u = *reinterpret_cast<const uint4 *>(reinterpret_cast<const uint16_t *>(x) + off);
            if (!valid) t.u = make_uint4(0, 0, 0, 0);
        }
        a[0] = t.v;
    } else {
        float4 p = make_float4(0.f, 0.f, 0.f, 0.f), q = p;
        if (!PX || valid) {
            p = *reinterpret_cast<const float4 *>(reinterpret_cast<const float *>(x) + off);
            q = *reinterpret_cast<const float4 *>(reinterpret_cast<const float *>(x) + off + 4);
        }
        float v[8] = {p.x, p.y, p.z, p.w, q.x, q.y, q.z, q.w};
        if (!PX && !valid) {
#pragma unroll
            for (int i = 0; i < 8; ++i) v[i] = 0.f;
        }
        split_f32x8<NT>(v, a);
    }
}

// Weight addressing.  Both layouts are walked in 64-wide K super-blocks (two Q8_0 blocks); lane
// (n = lane & 15, g = lane >> 4) owns K offsets 8g..8g+7 of each of the two blocks of row n.
//  PLAIN: row-major [rows][K]; the lane's 16 bytes are two 8-byte pieces 32 bytes apart.
//  TILED: per (16-row tile, super-block) 1 KB contiguous, lane l's 16 bytes at 16 l (see the
//         repack kernel); Q8_0 scales per (tile, super-block) 32 fp16, row n's two at 2n.
template <int LAYOUT>
struct WAddr {
    const int8_t *w;     // PLAIN: row start + 8g;  TILED: tile start + 16 lane
    const uint16_t *s;   // Q8_0 scales: PLAIN: row's scale array; TILED: tile's first scale + 2n
    size_t wstride;      // bytes between super-blocks
    size_t sstride;      // fp16 between super-blocks (scales)

    __device__ __forceinline__ uint4 load(int sb) const
    {
        // tiled: a wave's load covers whole lines, streamed with the non-temporal hint; plain:
        // each 8-byte piece is half of a 16-byte run whose other half another load takes, so the
        // lines stay cacheable (with the hint the plain Q8_0 gate/up fetched 1.9x its bytes)
        if (LAYOUT == L_TILED) return ld_stream16(w + (size_t)sb * wstride);
        const uint2 a = *reinterpret_cast<const uint2 *>(w + (size_t)sb * 64);
        const uint2 b = *reinterpret_cast<const uint2 *>(w + (size_t)sb * 64 + 32);
        return make_uint4(a.x, a.y, b.x, b.y);
    }
    // the two Q8_0 scales of super-block sb (block 2sb in the low half)
    __device__ __forceinline__ uint32_t scales(int sb) const
    {
        if (LAYOUT == L_TILED) return ld_stream4(s + (size_t)sb * sstride);
        return *reinterpret_cast<const uint32_t *>(s + (size_t)sb * sstride);
    }
};

// grid.x = max_slots * (d_ff / 16); workgroup = NW waves splitting the K super-blocks.  h is
// written as two bf16 planes (hi, lo) in permuted row order.  ROUTE: the slot comes from the
// in-block routing above instead of the permute step's records.  PX: activation loads only in
// the lanes of valid rows (see load_x8).
template <int FMT, int LAYOUT, int ACT, int XT, int NW, int U, bool ROUTE, bool PX>
__global__ __launch_bounds__(64 * NW) void gateup_int8_kernel(
    const void *__restrict__ x, int T, int d, int k, const int8_t *__restrict__ wgu,
    const void *__restrict__ wgu_scales, int d_ff, const int32_t *__restrict__ perm,
    const int4 *__restrict__ slots, const int32_t *__restrict__ n_active,
    uint16_t *__restrict__ h_hi, uint16_t *__restrict__ h_lo, RouteIn ri)
{
    constexpr bool GATED = ACT == ACT_SWIGLU;
    constexpr int M = GATED ? 2 : 1;
    constexpr int NT = XT == X_F32 ? 3 : 1;
    __shared__ f32x4 red[NW][2][WAVE];

    const int nft = d_ff >> 4;
    const int slot = blockIdx.x / nft;
    const int ft = blockIdx.x - slot * nft;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int li = lane & 15, lg = lane >> 4;
    // the slot record (with the tokens of the first 16 pairs) is read together with the active
    // count: slot < max_slots <= E + S keeps the reads in bounds even for an unused slot, whose
    // record is then ignored, and token values are only used for rows below the pair count
    int e, row0, n_e, tok16;
    if constexpr (ROUTE) {
        const RouteSlot rs = route_slot_any<NW>(ri, T, k, slot, ft == 0, li);
        if (rs.e < 0) return;                        // uniform across the block
        e = rs.e;
        row0 = rs.row0;
        n_e = rs.n_e;
        tok16 = rs.tok;
    } else {
        const int nact = *n_active;
        const int4 si = slots[(size_t)slot * SLOT_INT4];
        tok16 = slot_token(slots, slot, li);
        // (the record and token enter the exit test so that all three loads are issued at once;
        // an active slot has a pair count >= 1 and token 0 >= 0)
        if ((slot >= nact) | (si.z < 1) | (__builtin_amdgcn_readfirstlane(tok16) < 0)) return;
        e = si.x;
        row0 = si.y;
        n_e = si.z;
    }
    const int f = ft * 16 + li;
    const int S = d >> 6;
    const int s0 = wave * S / NW, s1 = (wave + 1) * S / NW;
    const size_t r0 = (size_t)e * (M * d_ff) + f;      // gate row (or the up row when ungated)
    const size_t r1 = r0 + (GATED ? d_ff : 0);          // up row (gated)
    const uint16_t *sc = reinterpret_cast<const uint16_t *>(wgu_scales);
    WAddr<LAYOUT> a0, a1;
    if (LAYOUT == L_TILED) {
        const size_t tile = ((size_t)e * nft + ft) * S * M;     // (tile, super-block 0, m 0)
        a0.w = wgu + tile * 1024 + lane * 16;
        a1.w = a0.w + 1024;
        a0.wstride = a1.wstride = (size_t)M * 1024;
        a0.s = sc + tile * 32 + 2 * li;
        a1.s = a0.s + 32;
        a0.sstride = a1.sstride = (size_t)M * 32;
    } else {
        a0.w = wgu + r0 * d + lg * 8;
        a1.w = wgu + r1 * d + lg * 8;
        a0.s = sc + r0 * (d >> 5);
        a1.s = sc + r1 * (d >> 5);
        a0.wstride = a1.wstride = 64;
        a0.sstride = a1.sstride = 2;
    }

    for (int m0 = 0; m0 < n_e; m0 += 16) {
        const int mi = m0 + li;
        const bool mvalid = mi < n_e;
        // rows past the count read token 0's row and are zeroed, so no load sits under a branch
        int tok = m0 == 0 ? tok16 : perm[row0 + min(mi, n_e - 1)] / k;
        tok = mvalid ? min(max(tok, 0), T - 1) : 0;
        f32x4 acc0 = zero4(), acc1 = zero4();
        for (int sb = s0; sb < s1; sb += U) {
            uint4 wa[U], wb[U];
            uint32_t q0[U], q1[U];
            bf16x8 a[U][2][NT];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int sc_ = min(sb + u, s1 - 1);   // the tail re-reads the last super-block
                wa[u] = a0.load(sc_);
                if (GATED) wb[u] = a1.load(sc_);
                if (FMT == W_Q8_0) {
                    q0[u] = a0.scales(sc_);
                    if (GATED) q1[u] = a1.scales(sc_);
                }
            }
            const size_t xoff = (size_t)tok * d + lg * 8;
#pragma unroll
            for (int u = 0; u < U; ++u) {
                // a super-block past the wave's share re-reads the last one with zero activations,
                // so its products add exact zeros
                const int sc_ = min(sb + u, s1 - 1);
                const bool uvalid = mvalid && sb + u < s1;
                load_x8<XT, NT, PX>(x, xoff + (size_t)sc_ * 64, uvalid, a[u][0]);
                load_x8<XT, NT, PX>(x, xoff + (size_t)sc_ * 64 + 32, uvalid, a[u][1]);
            }
            // every load of the batch is issued before the first product, and no product sits
            // under a branch (the compiler otherwise sinks a later super-block's loads into the
            // branch of its products; with U = 2 the two orders measured the same)
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int u = 0; u < U; ++u) {
                {
#pragma unroll
                    for (int j = 0; j < 2; ++j) {
                        const bf16x8 b0 = j ? i8x8_to_bf16x8(wa[u].z, wa[u].w) : i8x8_to_bf16x8(wa[u].x, wa[u].y);
                        if (FMT == W_Q8_0) {
                            f32x4 c = zero4();
#pragma unroll
                            for (int t = 0; t < NT; ++t) c = mfma16x16x32_bf16(a[u][j][t], b0, c);
                            acc0 += c * half_bits_to_float(j ? (q0[u] >> 16) : (q0[u] & 0xFFFFu));
                        } else {
#pragma unroll
                            for (int t = 0; t < NT; ++t) acc0 = mfma16x16x32_bf16(a[u][j][t], b0, acc0);
                        }
                        if (GATED) {
                            const bf16x8 b1 = j ? i8x8_to_bf16x8(wb[u].z, wb[u].w) : i8x8_to_bf16x8(wb[u].x, wb[u].y);
                            if (FMT == W_Q8_0) {
                                f32x4 c = zero4();
#pragma unroll
                                for (int t = 0; t < NT; ++t) c = mfma16x16x32_bf16(a[u][j][t], b1, c);
                                acc1 += c * half_bits_to_float(j ? (q1[u] >> 16) : (q1[u] & 0xFFFFu));
                            } else {
#pragma unroll
                                for (int t = 0; t < NT; ++t) acc1 = mfma16x16x32_bf16(a[u][j][t], b1, acc1);
                            }
                        }
                    }
                }
            }
        }
        red[wave][0][lane] = acc0;
        red[wave][1][lane] = acc1;
        __syncthreads();
        if (wave == 0) {
            f32x4 g = red[0][0][lane], u = red[0][1][lane];
#pragma unroll
            for (int w = 1; w < NW; ++w) {
                g += red[w][0][lane];
                u += red[w][1][lane];
            }
            if (FMT == W_I8_ROW) {
                const float *rs = reinterpret_cast<const float *>(wgu_scales);
                g *= rs[r0];
                if (GATED) u *= rs[r1];
            }
            // lane holds C[token m0 + 4*lg + i][row f]
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int m = m0 + 4 * lg + i;
                if (m < n_e) {
                    const float hv = GATED ? silu_f32(g[i]) * u[i] : (g[i] > 0.f ? g[i] * g[i] : 0.f);
                    // h as two bf16 terms: hi + lo matches h to 2^-17 relative, and both are
                    // exact matrix-core operands for the down projection
                    const uint32_t hi = f32_to_bf16_rne(hv);
                    const uint32_t lo = f32_to_bf16_rne(hv - bf16_bits_to_f32(hi));
                    h_hi[(size_t)(row0 + m) * d_ff + f] = (uint16_t)hi;
                    h_lo[(size_t)(row0 + m) * d_ff + f] = (uint16_t)lo;
                }
            }
        }
        __syncthreads();
    }
}

// Down projection of every (token, slot) pair: y[row][o] = sum_f W_d[e][o][f] h[row][f], rows in
// permuted order.  grid.x = max_slots * ngrp; block (slot, og) has NW waves, wave w owning the
// TPW output tiles (og * NW + w) * TPW + i (16 rows each) of one active expert.  The expert's h
// rows, RM at a time, are staged in LDS in K chunks of KCS super-blocks; every thread issues its
// share of that chunk of h first and then all of its tiles' weight loads for the chunk, so one
// HBM round trip covers a wave's weights while the (L2-resident) h lands in LDS.  The A operands
// then come from LDS; rows past the expert's pair count are zero.
// The fixed-order weighted combine runs afterwards (combine_rows4_kernel).  (Letting the last
// block of each output group combine in place needs a device-scope fence per block, an L2
// write-back on this multi-XCD part, which costs far more than the extra launch.)
template <int FMT, int LAYOUT, int NW, int TPW, int RM, int KCS>
__global__ __launch_bounds__(64 * NW) void down_int8_kernel(
    const uint16_t *__restrict__ h_hi, const uint16_t *__restrict__ h_lo, int d_ff,
    const int8_t *__restrict__ wd, const void *__restrict__ wd_scales, int d,
    const int4 *__restrict__ slots, const int32_t *__restrict__ n_active, float *__restrict__ ybuf)
{
    constexpr int NT = 64 * NW;
    constexpr int RS = KCS * 64 + 8;                       // LDS row stride in bf16 (+16 B: banks)
    constexpr int HPT = (2 * RM * KCS * 8 + NT - 1) / NT;  // 16-byte h pieces per thread per chunk
    __shared__ uint4 hs4[2 * RM * RS / 8];
    uint16_t *hs = reinterpret_cast<uint16_t *>(hs4);

    const int OT = d >> 4;
    const int ngrp = (OT + NW * TPW - 1) / (NW * TPW);
    const int slot = blockIdx.x / ngrp, og = blockIdx.x - slot * ngrp;
    // count and record in one round trip (see gateup_int8_kernel); uniform across the block
    const int nact = *n_active;
    const int4 si = slots[(size_t)slot * SLOT_INT4];
    if ((slot >= nact) | (si.z < 1)) return;
    const int e = si.x, row0 = si.y, n_e = si.z;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int li = lane & 15, lg = lane >> 4;
    const int S = d_ff >> 6;
    const uint16_t *sc = reinterpret_cast<const uint16_t *>(wd_scales);

    WAddr<LAYOUT> ad[TPW];
    int otv[TPW];
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
        const int ot = (og * NW + wave) * TPW + i;
        otv[i] = ot;
        const int otc = ot < OT ? ot : OT - 1;           // a tile past the end reads the last one
        if (LAYOUT == L_TILED) {
            const size_t tile = ((size_t)e * OT + otc) * S;
            ad[i].w = wd + tile * 1024 + lane * 16;
            ad[i].s = sc + tile * 32 + 2 * li;
            ad[i].wstride = 1024;
            ad[i].sstride = 32;
        } else {
            const size_t wr = (size_t)e * d + otc * 16 + li;
            ad[i].w = wd + wr * d_ff + lg * 8;
            ad[i].s = sc + wr * (d_ff >> 5);
            ad[i].wstride = 64;
            ad[i].sstride = 2;
        }
    }

    for (int m0 = 0; m0 < n_e; m0 += RM) {
        const int nr = min(RM, n_e - m0);
        f32x4 acc[TPW];
#pragma unroll
        for (int i = 0; i < TPW; ++i) acc[i] = zero4();
        for (int c0 = 0; c0 < S; c0 += KCS) {
            const int ns = min(KCS, S - c0);
            // h pieces of this chunk: (plane, row r < nr, 16-byte column q < 8 ns)
            const int per_row = ns * 8, per_plane = nr * per_row;
            // (only pieces that exist are loaded: lanes past them are masked off, and a wave with
            // none skips the load; the loads are all issued up front)
            // (held in one vector value rather than an array, which keeps it out of scratch)
            typedef uint32_t hvec __attribute__((ext_vector_type(4 * HPT)));
            hvec hv;
#pragma unroll
            for (int j = 0; j < HPT; ++j) {
                const int idx0 = tid + j * NT;
                const int idx = min(idx0, 2 * per_plane - 1);
                const int p = idx >= per_plane;
                const int rem = idx - p * per_plane;
                const int r = rem / per_row, q = rem - r * per_row;
                const uint16_t *src = (p ? h_lo : h_hi) + (size_t)(row0 + m0 + r) * d_ff + c0 * 64 + q * 8;
                uint4 v = make_uint4(0, 0, 0, 0);
                if (idx0 < 2 * per_plane) v = *reinterpret_cast<const uint4 *>(src);
                hv[4 * j] = v.x; hv[4 * j + 1] = v.y; hv[4 * j + 2] = v.z; hv[4 * j + 3] = v.w;
            }
            __builtin_amdgcn_sched_barrier(0x000F);           // h loads before the weight loads
            uint4 wv[TPW][KCS];
            uint32_t qs[TPW][KCS];
#pragma unroll
            for (int i = 0; i < TPW; ++i)
#pragma unroll
                for (int u = 0; u < KCS; ++u) {
                    const int sb = c0 + min(u, ns - 1);        // the tail re-reads the last one
                    wv[i][u] = ad[i].load(sb);
                    if (FMT == W_Q8_0) qs[i][u] = ad[i].scales(sb);
                }
#pragma unroll
            for (int j = 0; j < HPT; ++j) {
                const int idx0 = tid + j * NT;
                const int idx = min(idx0, 2 * per_plane - 1);
                const int p = idx >= per_plane;
                const int rem = idx - p * per_plane;
                const int r = rem / per_row, q = rem - r * per_row;
                if (idx0 == idx)
                    *reinterpret_cast<uint4 *>(hs + (p * RM + r) * RS + q * 8) =
                        make_uint4(hv[4 * j], hv[4 * j + 1], hv[4 * j + 2], hv[4 * j + 3]);
            }
            // LDS writes done; the weight loads stay in flight across the barrier
            asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
#pragma unroll
            for (int u = 0; u < KCS; ++u) {
                if (u < ns) {
#pragma unroll
                    for (int j = 0; j < 2; ++j) {
                        U4 ah, al;
                        if (li < nr) {
                            const uint16_t *hp = hs + li * RS + u * 64 + 32 * j + 8 * lg;
                            ah.u = *reinterpret_cast<const uint4 *>(hp);
                            al.u = *reinterpret_cast<const uint4 *>(hp + RM * RS);
                        } else {
                            ah.u = make_uint4(0, 0, 0, 0);
                            al.u = ah.u;
                        }
#pragma unroll
                        for (int i = 0; i < TPW; ++i) {
                            const bf16x8 b = j ? i8x8_to_bf16x8(wv[i][u].z, wv[i][u].w)
                                               : i8x8_to_bf16x8(wv[i][u].x, wv[i][u].y);
                            if (FMT == W_Q8_0) {
                                f32x4 c = mfma16x16x32_bf16(ah.v, b, zero4());
                                c = mfma16x16x32_bf16(al.v, b, c);
                                acc[i] += c * half_bits_to_float(j ? (qs[i][u] >> 16) : (qs[i][u] & 0xFFFFu));
                            } else {
                                acc[i] = mfma16x16x32_bf16(ah.v, b, acc[i]);
                                acc[i] = mfma16x16x32_bf16(al.v, b, acc[i]);
                            }
                        }
                    }
                }
            }
            // every wave's LDS reads are done before the next chunk overwrites them
            asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
        }
#pragma unroll
        for (int i = 0; i < TPW; ++i) {
            if (otv[i] < OT) {
                const int o = otv[i] * 16 + li;
                f32x4 a = acc[i];
                if (FMT == W_I8_ROW) a *= reinterpret_cast<const float *>(wd_scales)[(size_t)e * d + o];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int m = 4 * lg + r;
                    if (m < nr) ybuf[(size_t)(row0 + m0 + m) * d + o] = a[r];
                }
            }
        }
    }
}

// Repack of one expert matrix [E][R][K] (R rows in M halves of R/M rows, K the reduction
// dimension) from row-major to the tiled layout.  Row r = m * (R/M) + 16 t + n, K offset
// 64 s + 32 j + 8 g + i goes to tile ((e * (R/M/16) + t) * (K/64) + s) * M + m, byte
// 16 (n + 16 g) + 8 j + i of that tile's 1 KB; its Q8_0 scale of block 2s + j to fp16 2n + j of the
// tile's 32.  One thread writes one lane's 16 bytes (and, for lanes with g = 0, the row's scales).
__global__ __launch_bounds__(256) void repack_tiled_kernel(const int8_t *__restrict__ src,
                                                           const uint16_t *__restrict__ ssrc,
                                                           int E, int R, int K, int M,
                                                           int8_t *__restrict__ dst,
                                                           uint16_t *__restrict__ sdst)
{
    const int S = K >> 6;
    const int half = R / M;                 // rows per matrix half (gate / up), multiple of 16
    const int NTt = half >> 4;
    const size_t total = (size_t)E * NTt * S * M * 64;    // lanes
    const size_t id = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (id >= total) return;
    const int lane = (int)(id & 63);
    size_t t = id >> 6;                      // tile index = ((e*NTt + tt) * S + s) * M + m
    const int m = (int)(t % M); t /= M;
    const int s = (int)(t % S); t /= S;
    const int tt = (int)(t % NTt);
    const int e = (int)(t / NTt);
    const int n = lane & 15, g = lane >> 4;
    const size_t row = (size_t)e * R + (size_t)m * half + 16 * tt + n;
    const int8_t *p = src + row * K + 64 * s + 8 * g;
    const uint2 a = *reinterpret_cast<const uint2 *>(p);
    const uint2 b = *reinterpret_cast<const uint2 *>(p + 32);
    *reinterpret_cast<uint4 *>(dst + (id >> 6) * 1024 + lane * 16) = make_uint4(a.x, a.y, b.x, b.y);
    if (ssrc && g == 0) {
        const uint32_t sv = *reinterpret_cast<const uint32_t *>(ssrc + row * (K >> 5) + 2 * s);
        *reinterpret_cast<uint32_t *>(sdst + (id >> 6) * 32 + 2 * n) = sv;
    }
}

// out[t][o] = sum over slot groups sg = 0..7 (in order) of sum over slots j = sg, sg+8, ... (in
// order) of w[t][j] * sum over chunks c (in order) of ybuf[(inv[t*k+j] * nchunk + c) * d + o],
// then + the S shared experts' rows T k + s T + t (weight 1, in order).  A fixed order, so the
// result is reproducible bit for bit.  Block: 32 outputs x 8 slot groups (d is a multiple of 64),
// so a token's outputs take d / 32 blocks.  A thread's row indices and weights (up to 8 slots,
// k <= 64) are read first, then the loads of COMBINE_CB chunks of all of its slots go out at
// once.  (Against 64 outputs and 8 chunks per batch, tokens/s: Nemotron-shaped zero-skip T = 1
// 29.2k -> 29.7k, T = 8 68.7k -> 68.7k, Gemma-shaped E2M1 T = 8 124.2k -> 124.8k, MiniMax-M3-shaped
// E2M1 T = 1 20.3k -> 20.6k.)
constexpr int COMBINE_CB = 12;    // partial-sum chunks per batch of loads
__global__ __launch_bounds__(256) void combine_rows_kernel(const float *__restrict__ ybuf,
                                                           const int32_t *__restrict__ inv,
                                                           const float *__restrict__ topk_w, int k,
                                                           int d, int nchunk, int T, int S,
                                                           float *__restrict__ out)
{
    __shared__ float red[8][32];
    const int t = blockIdx.y;
    const int ol = threadIdx.x & 31, sg = threadIdx.x >> 5;
    const int o = blockIdx.x * 32 + ol;
    const int nj = (k - sg + 7) / 8;                 // slots j = sg + 8 i, i < nj (nj <= 8)
    int row[8];
    float w[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int p = t * k + min(sg + 8 * i, k - 1);
        row[i] = inv[p];
        w[i] = topk_w[p];
    }
    // every slot's loads of a batch of CB chunks go out together, then are added in chunk order
    constexpr int CB = COMBINE_CB;
    float y[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) y[i] = 0.f;
    for (int c0 = 0; c0 < nchunk; c0 += CB) {
        float v[8][CB];
#pragma unroll
        for (int i = 0; i < 8; ++i)
            if (i < nj) {
                const float *yr = ybuf + (size_t)row[i] * nchunk * d + o;
#pragma unroll
                for (int u = 0; u < CB; ++u) v[i][u] = yr[(size_t)min(c0 + u, nchunk - 1) * d];
            }
#pragma unroll
        for (int i = 0; i < 8; ++i)
            if (i < nj) {
#pragma unroll
                for (int u = 0; u < CB; ++u)
                    if (c0 + u < nchunk) y[i] += v[i][u];
            }
    }
    float a = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i)
        if (i < nj) a += w[i] * y[i];
    red[sg][ol] = a;
    __syncthreads();
    if (sg == 0) {
        float r = red[0][ol];
#pragma unroll
        for (int g = 1; g < 8; ++g) r += red[g][ol];
        for (int sh = 0; sh < S; ++sh) {
            const float *yr = ybuf + (size_t)(T * k + sh * T + t) * nchunk * d + o;
            float y = 0.f;
            for (int c = 0; c < nchunk; ++c) y += yr[(size_t)c * d];
            r += y;
        }
        out[(size_t)t * d + o] = r;
    }
}

// out[t][4c..4c+3] = sum_{j = 0..k-1} w[t][j] * ybuf[inv[t*k+j]][4c..4c+3], slots in order,
// then + the S shared experts' rows T k + s T + t (weight 1, in order).  Eight slots at a time:
// their row indices and weights first, then their eight row loads, then the sums in slot order
// (a slot past k re-reads slot k - 1 and is not added).
__global__ __launch_bounds__(256) void combine_rows4_kernel(const float *__restrict__ ybuf,
                                                            const int32_t *__restrict__ inv,
                                                            const float *__restrict__ topk_w, int k,
                                                            int d, int T, int S, float *__restrict__ out)
{
    const int t = blockIdx.y;
    const int c = blockIdx.x * 256 + threadIdx.x;
    if (4 * c >= d) return;
    float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int j0 = 0; j0 < k; j0 += 8) {
        int row[8];
        float w[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int p = t * k + min(j0 + u, k - 1);
            row[u] = inv[p];
            w[u] = topk_w[p];
        }
        float4 y[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) y[u] = *reinterpret_cast<const float4 *>(ybuf + (size_t)row[u] * d + 4 * c);
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            if (j0 + u < k) {
                a.x = fmaf(w[u], y[u].x, a.x);
                a.y = fmaf(w[u], y[u].y, a.y);
                a.z = fmaf(w[u], y[u].z, a.z);
                a.w = fmaf(w[u], y[u].w, a.w);
            }
        }
    }
    for (int sh = 0; sh < S; ++sh) {
        const float4 y = *reinterpret_cast<const float4 *>(ybuf + (size_t)(T * k + sh * T + t) * d + 4 * c);
        a.x += y.x;
        a.y += y.y;
        a.z += y.z;
        a.w += y.w;
    }
    *reinterpret_cast<float4 *>(out + (size_t)t * d + 4 * c) = a;
}

// ------------------------------------------------------------------------------------------

// Waves per gate/up block and super-blocks per load batch.  Small batches keep the kernel at 80
// VGPRs, i.e. three 8-wave blocks per CU, and are the fastest at every batch size measured, even
// where few blocks run (so more bytes in flight per wave do not pay here): Gemma-shaped decode
// (Q8_0 tiled, us per layer) T = 1: U = 1 -> 25.1, 2 -> 26.0, 3 -> 29.8, 4 -> 27.5, 6 -> 30.5;
// T = 8: U = 1 -> 75.5, 2 -> 74.0, 3 -> 84.8; MiniMax-M3-shaped T = 1: U = 2 -> 64.5, 4 -> 65.2,
// 6 -> 72.7; T = 32: U = 1 -> 762, 2 -> 761 (4 waves per block: 41.4 - 42.6 us for the T = 8
// gate/up against 40.2; 2 waves: 44.7).
// Super-blocks per load batch (U) and masked activation loads (PX).  T > 2: U = 2, loads
// unmasked.  T <= 2: masked (73 instead of 121 VGPRs at U = 2), and U = 2 for grids of at least
// GU_U2_BLOCKS blocks, else 1.  Tokens/s against the earlier fixed U = 1 with unmasked loads:
// Gemma-shaped T = 1 (352 blocks) 42.1k with U = 1 / 40.5k with U = 2, T = 2 (704 blocks) 58.9k ->
// 60.2k with U = 2, MiniMax-M3-shaped T = 1 (768 blocks) 16.5k -> 17.2k with U = 2; at T = 8
// masking measured 107.7k -> 107.5k, so larger batches keep unmasked loads.
constexpr int GU_NW = 8, GU_U = 2, GU_U2_BLOCKS = 512;

template <int FMT, int LAYOUT, int ACT, int XT>
static void launch_gateup_t(dim3 g, hipStream_t s, const void *x, int T, int d, int k, const ExpertsDev &ex,
                            const PermuteOut &po, uint16_t *h_hi, uint16_t *h_lo, const RouteIn &ri)
{
#define GU(U, R, P) hipLaunchKernelGGL((gateup_int8_kernel<FMT, LAYOUT, ACT, XT, GU_NW, U, R, P>), g, dim3(64 * GU_NW), 0, s, \
                                       x, T, d, k, reinterpret_cast<const int8_t *>(ex.gate_up), ex.gate_up_scales, \
                                       ex.d_ff, po.perm, po.slots, po.n_active, h_hi, h_lo, ri)
    const bool u2 = g.x >= (unsigned)GU_U2_BLOCKS;
    if (ri.logits) {                                 // (in-block routing runs at T <= 2 only)
        if (u2) GU(2, true, true);
        else GU(1, true, true);
    } else if (T <= 2) {
        if (u2) GU(2, false, true);
        else GU(1, false, true);
    } else {
        GU(GU_U, false, false);
    }
#undef GU
}

template <int FMT, int LAYOUT>
static void dispatch_gateup(dim3 g, hipStream_t s, const void *x, int xtype, int T, int d, int k,
                            const ExpertsDev &ex, int act, const PermuteOut &po, uint16_t *hh,
                            uint16_t *hl, const RouteIn &ri)
{
    if (act == ACT_SWIGLU) {
        if (xtype == X_BF16) launch_gateup_t<FMT, LAYOUT, ACT_SWIGLU, X_BF16>(g, s, x, T, d, k, ex, po, hh, hl, ri);
        else launch_gateup_t<FMT, LAYOUT, ACT_SWIGLU, X_F32>(g, s, x, T, d, k, ex, po, hh, hl, ri);
    } else {
        if (xtype == X_BF16) launch_gateup_t<FMT, LAYOUT, ACT_RELU2, X_BF16>(g, s, x, T, d, k, ex, po, hh, hl, ri);
        else launch_gateup_t<FMT, LAYOUT, ACT_RELU2, X_F32>(g, s, x, T, d, k, ex, po, hh, hl, ri);
    }
}

// (the rule of up_e2m1_can_route: two tokens over more than 256 experts take two selection passes)
bool gateup_can_route(int T, int k, int E) { return (T == 1 || (T == 2 && E <= 256)) && T * k <= 64 && E <= MAX_E; }

hipError_t launch_gateup_int8(const void *x, int xtype, int T, int k, const ExpertsDev &ex, int act,
                              const PermuteOut &po, uint16_t *h_hi, uint16_t *h_lo, const RouteIn &ri,
                              hipStream_t s)
{
    if (ri.logits && !gateup_can_route(T, k, ex.E)) return hipErrorInvalidValue;
    const int max_slots = min(ex.E, T * k) + ex.S;   // routed slots, then the shared ones
    const dim3 g(max_slots * (ex.d_ff / 16));
    const int d = ex.d_model;
    ProfScope ps(K_GATEUP_I8, s);
    switch (ex.fmt) {
    case W_Q8_0: dispatch_gateup<W_Q8_0, L_PLAIN>(g, s, x, xtype, T, d, k, ex, act, po, h_hi, h_lo, ri); break;
    case W_I8_ROW: dispatch_gateup<W_I8_ROW, L_PLAIN>(g, s, x, xtype, T, d, k, ex, act, po, h_hi, h_lo, ri); break;
    case W_Q8_0_TILED: dispatch_gateup<W_Q8_0, L_TILED>(g, s, x, xtype, T, d, k, ex, act, po, h_hi, h_lo, ri); break;
    default: dispatch_gateup<W_I8_ROW, L_TILED>(g, s, x, xtype, T, d, k, ex, act, po, h_hi, h_lo, ri); break;
    }
    return hipGetLastError();
}

template <int FMT, int LAYOUT, int RM, int KCS>
static void launch_down_rm(hipStream_t s, const uint16_t *hh, const uint16_t *hl, const ExpertsDev &ex,
                           int max_slots, const PermuteOut &po, float *ybuf)
{
    constexpr int NW = 4, TPW = 1;
    const int ngrp = (ex.d_model / 16 + NW * TPW - 1) / (NW * TPW);
    hipLaunchKernelGGL((down_int8_kernel<FMT, LAYOUT, NW, TPW, RM, KCS>), dim3(max_slots * ngrp),
                       dim3(64 * NW), 0, s, hh, hl, ex.d_ff, reinterpret_cast<const int8_t *>(ex.down),
                       ex.down_scales, ex.d_model, po.slots, po.n_active, ybuf);
}

// h rows staged per pass: at most T pairs share an expert.  Super-blocks per h chunk (us per
// layer, down kernel alone in brackets): Gemma-shaped T = 8, 12 -> 74.5 (24.4), 6 -> 74.6 (24.6),
// 3 -> 76.1 (26.2); MiniMax-M3-shaped T = 32, 8 -> 761 (259), 4 -> 754 (254).  (8 waves per block
// or two output tiles per wave: 76.5 / 78.4 at Gemma T = 8.)
template <int FMT, int LAYOUT>
static void launch_down_t(hipStream_t s, const uint16_t *hh, const uint16_t *hl, const ExpertsDev &ex,
                          int T, int k, const PermuteOut &po, float *ybuf)
{
    const int max_slots = min(ex.E, T * k) + ex.S;   // routed slots, then the shared ones
    if (T <= 2) launch_down_rm<FMT, LAYOUT, 2, 12>(s, hh, hl, ex, max_slots, po, ybuf);
    else if (T <= 8) launch_down_rm<FMT, LAYOUT, 8, 12>(s, hh, hl, ex, max_slots, po, ybuf);
    else launch_down_rm<FMT, LAYOUT, 16, 4>(s, hh, hl, ex, max_slots, po, ybuf);
}

// Small batches: the down projection and the weighted combine in one pass, so neither the per-pair
// y buffer nor the combine launch is needed.  Block (ot, t) produces outputs 16 ot .. 16 ot + 15
// of token t; its 8 waves take the token's slots j = w, w + 8, ... (the k routed slots, then the
// shared experts, weight 1), or, when the token has at most 4 slots, WPS = 8 / slots (rounded down
// to a power of two) waves share slot w / WPS, wave w taking part w % WPS of its super-blocks, so
// that no wave idles while the others stream.  The token's h rows (hi + lo, exact in fp32) are
// staged in LDS while each wave's weight loads for its first slot are already in flight.  Lane (n, g) multiplies the
// 16 weights of row n it holds per 64-wide super-block (K offsets 8g..8g+7 and 32+8g..32+8g+7,
// the tiled lane order) by the matching h values on the VALU; the four g lanes of a row are added
// (xor 16, then xor 32), each slot's y is scaled by its routing weight into the wave's sum, and
// the waves' sums are added in wave order: a fixed order, so the output is deterministic.
// Each token's blocks read their experts' weights themselves, so an expert shared by several
// tokens is read once per token (from L2 after the first); measured on the Gemma-shaped decode,
// tokens/s against down + combine: T = 1 34.0k vs 31.7k, T = 2 50.8k vs 50.4k, T = 3 60.1k vs
// 61.8k, T = 6 84.3k vs 89.2k, hence T <= 2.
constexpr int DC_NW = 8;          // waves per block
constexpr int DC_MAX_H = 12288;   // (k + S) * d_ff bound: the token's h rows in LDS (48 KB)
// Super-blocks of weights in flight per wave: 6 while a wave's share is at most 12 super-blocks,
// else 4 (us per layer, Gemma-shaped T = 1 with 11 per wave / MiniMax-M3-shaped T = 1 with 24:
// 3 -> 26.2 / 60.5, 4 -> 25.8 / 59.2, 6 -> 25.4 / 60.1, 12 -> 26.1 / 64.7, 24 -> 33.0 / 75.2).
// (a template parameter of the kernel)

template <int FMT, int LAYOUT, int DC_KC>
__global__ __launch_bounds__(64 * DC_NW) void down_combine_kernel(
    const uint16_t *__restrict__ h_hi, const uint16_t *__restrict__ h_lo, int d_ff,
    const int8_t *__restrict__ wd, const void *__restrict__ wd_scales, int d,
    const int32_t *__restrict__ topk_idx, const float *__restrict__ topk_w,
    const int32_t *__restrict__ inv, int T, int k, int E, int S, float *__restrict__ out)
{
    constexpr int NT = 64 * DC_NW;
    constexpr int HU = (DC_MAX_H / 8 + NT - 1) / NT;   // 8-column h units per thread, at most
    __shared__ __attribute__((aligned(16))) float hs[DC_MAX_H];
    __shared__ float part[DC_NW][16];
    __shared__ int s_row[MAX_K + MAX_SHARED], s_exp[MAX_K + MAX_SHARED];
    __shared__ float s_wt[MAX_K + MAX_SHARED];
    const int OT = d >> 4;
    const int ot = blockIdx.x, t = blockIdx.y;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int n = lane & 15, g = lane >> 4;
    const int ns = k + S;                              // slots of the token
    const int P = T * k;
    const int SB = d_ff >> 6;                          // super-blocks
    const uint16_t *sc = reinterpret_cast<const uint16_t *>(wd_scales);

    // the permuted h row, expert and weight of each slot of token t, read once into LDS: every
    // weight and h address below needs them, and reading them from global memory behind the
    // weight loads would make each read wait for those loads (loads complete in order)
    if (tid < ns) {
        const int jj = tid;
        s_row[jj] = jj < k ? inv[t * k + jj] : P + (jj - k) * T + t;
        s_exp[jj] = jj < k ? clamp_id(topk_idx[t * k + jj], E) : E + (jj - k);
        s_wt[jj] = jj < k ? topk_w[t * k + jj] : 1.0f;
    }
    __syncthreads();
    auto slot_row = [&](int j) { return s_row[j]; };
    auto slot_expert = [&](int j) { return s_exp[j]; };
    auto slot_weight = [&](int j) { return s_wt[j]; };
    auto waddr = [&](int e) {
        WAddr<LAYOUT> a;
        if (LAYOUT == L_TILED) {
            const size_t tile = ((size_t)e * OT + ot) * SB;
            a.w = wd + tile * 1024 + lane * 16;
            a.s = sc + tile * 32 + 2 * n;
            a.wstride = 1024;
            a.sstride = 32;
        } else {
            const size_t wr = (size_t)e * d + ot * 16 + n;
            a.w = wd + wr * d_ff + g * 8;
            a.s = sc + wr * (d_ff >> 5);
            a.wstride = 64;
            a.sstride = 2;
        }
        return a;
    };

    // waves per slot, this wave's first slot and its share [sb0, sb1) of the super-blocks
    // (the largest power of two with ns * wps <= 8)
    const int wps = ns > DC_NW / 2 ? 1 : (ns > DC_NW / 4 ? 2 : (ns > 1 ? 4 : 8));
    int j = wave / wps;
    const int part_i = wave - j * wps;
    const int sb0 = part_i * SB / wps, sb1 = (part_i + 1) * SB / wps;
    // the token's h rows go out first (unit i = (slot i / (d_ff / 8), 8 columns); lanes past the
    // last unit are masked off and a wave with none skips the load, so the loads go out together),
    // then this wave's first slot's weights for the first DC_KC super-blocks (a wave without a
    // slot re-reads slot 0's and discards them), so that waiting for h (from L2) leaves the weight
    // loads in flight
    const int upr = d_ff >> 3, total = ns * upr;
    uint4 hv[HU], lv[HU];
#pragma unroll
    for (int i = 0; i < HU; ++i) {
        const int u0 = tid + i * NT, u = min(u0, total - 1);
        const int js = u / upr, c = (u - js * upr) * 8;
        const size_t off = (size_t)slot_row(js) * d_ff + c;
        hv[i] = lv[i] = make_uint4(0, 0, 0, 0);
        if (u0 < total) {
            hv[i] = *reinterpret_cast<const uint4 *>(h_hi + off);
            lv[i] = *reinterpret_cast<const uint4 *>(h_lo + off);
        }
    }
    WAddr<LAYOUT> ad = waddr(slot_expert(j < ns ? j : 0));
    uint4 wv[DC_KC];
    uint32_t qs[DC_KC];
#pragma unroll
    for (int u = 0; u < DC_KC; ++u) {
        const int sb = max(min(sb0 + u, sb1 - 1), 0);  // an empty share re-reads super-block 0
        wv[u] = ad.load(sb);
        if (FMT == W_Q8_0) qs[u] = ad.scales(sb);
    }
    __builtin_amdgcn_sched_barrier(0);                 // (keep that order)
    {
#pragma unroll
        for (int i = 0; i < HU; ++i) {
            const int u0 = tid + i * NT, u = min(u0, total - 1);
            if (u0 != u) continue;
            const int js = u / upr, c = (u - js * upr) * 8;
            float *dst = hs + js * d_ff + c;
            const uint32_t hw[4] = {hv[i].x, hv[i].y, hv[i].z, hv[i].w};
            const uint32_t lw[4] = {lv[i].x, lv[i].y, lv[i].z, lv[i].w};
            float f[8];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                f[2 * q] = bf16_bits_to_f32(hw[q] & 0xFFFFu) + bf16_bits_to_f32(lw[q] & 0xFFFFu);
                f[2 * q + 1] = bf16_bits_to_f32(hw[q] >> 16) + bf16_bits_to_f32(lw[q] >> 16);
            }
            *reinterpret_cast<float4 *>(dst) = make_float4(f[0], f[1], f[2], f[3]);
            *reinterpret_cast<float4 *>(dst + 4) = make_float4(f[4], f[5], f[6], f[7]);
        }
    }
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");   // h in LDS; weights in flight

    float acc_w = 0.f;                                 // sum over this wave's slots of w_j y_j[n]
    for (; j < ns; j += DC_NW) {                       // (wps > 1: one slot per wave, ns * wps <= 8)
        const int e = slot_expert(j);
        const float wj = slot_weight(j);
        if (j != wave / wps) {                         // a later slot: its first weights now
            ad = waddr(e);
#pragma unroll
            for (int u = 0; u < DC_KC; ++u) {
                const int sb = max(min(sb0 + u, sb1 - 1), 0);
                wv[u] = ad.load(sb);
                if (FMT == W_Q8_0) qs[u] = ad.scales(sb);
            }
        }
        const float *hr = hs + j * d_ff;
        float y = 0.f;
        for (int c0 = sb0; c0 < sb1; c0 += DC_KC) {
            if (c0 > sb0) {                            // the next DC_KC super-blocks
#pragma unroll
                for (int u = 0; u < DC_KC; ++u) {
                    const int sb = min(c0 + u, sb1 - 1);
                    wv[u] = ad.load(sb);
                    if (FMT == W_Q8_0) qs[u] = ad.scales(sb);
                }
            }
#pragma unroll
            for (int u = 0; u < DC_KC; ++u) {
                {
                    // a super-block past the share re-reads the last one with zero h (no branch:
                    // the compiler would sink the weight loads into it)
                    const bool uv = c0 + u < sb1;
                    const float *h0 = hr + max(min(c0 + u, sb1 - 1), 0) * 64 + 8 * g;
                    const float4 a0 = *reinterpret_cast<const float4 *>(h0);
                    const float4 a1 = *reinterpret_cast<const float4 *>(h0 + 4);
                    const float4 b0 = *reinterpret_cast<const float4 *>(h0 + 32);
                    const float4 b1 = *reinterpret_cast<const float4 *>(h0 + 36);
                    const float ha[8] = {uv ? a0.x : 0.f, uv ? a0.y : 0.f, uv ? a0.z : 0.f, uv ? a0.w : 0.f,
                                         uv ? a1.x : 0.f, uv ? a1.y : 0.f, uv ? a1.z : 0.f, uv ? a1.w : 0.f};
                    const float hb[8] = {uv ? b0.x : 0.f, uv ? b0.y : 0.f, uv ? b0.z : 0.f, uv ? b0.w : 0.f,
                                         uv ? b1.x : 0.f, uv ? b1.y : 0.f, uv ? b1.z : 0.f, uv ? b1.w : 0.f};
                    float p0 = 0.f, p1 = 0.f;          // K offsets 8g.. (block 2sb), 32+8g.. (2sb+1)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        p0 = fmaf(i8_to_f32(wv[u].x, i), ha[i], p0);
                        p0 = fmaf(i8_to_f32(wv[u].y, i), ha[4 + i], p0);
                        p1 = fmaf(i8_to_f32(wv[u].z, i), hb[i], p1);
                        p1 = fmaf(i8_to_f32(wv[u].w, i), hb[4 + i], p1);
                    }
                    if (FMT == W_Q8_0) {
                        y = fmaf(half_bits_to_float(qs[u] & 0xFFFFu), p0, y);
                        y = fmaf(half_bits_to_float(qs[u] >> 16), p1, y);
                    } else {
                        y += p0 + p1;
                    }
                }
            }
        }
        y += __shfl_xor(y, 16);
        y += __shfl_xor(y, 32);
        if (FMT == W_I8_ROW) y *= reinterpret_cast<const float *>(wd_scales)[(size_t)e * d + ot * 16 + n];
        acc_w = fmaf(wj, y, acc_w);
    }
    if (lane < 16) part[wave][lane] = acc_w;
    __syncthreads();
    if (tid < 16) {
        float o = 0.f;
#pragma unroll
        for (int w = 0; w < DC_NW; ++w) o += part[w][tid];
        out[(size_t)t * d + ot * 16 + tid] = o;
    }
}

bool down_combine_fits(int T, int k, const ExpertsDev &ex)
{
    return T <= 2 && (size_t)(k + ex.S) * ex.d_ff <= (size_t)DC_MAX_H && ex.fmt != W_E2M1;
}

hipError_t launch_down_combine(const uint16_t *h_hi, const uint16_t *h_lo, const ExpertsDev &ex, int T, int k,
                               const PermuteOut &po, const int32_t *topk_idx, const float *topk_w, float *out,
                               hipStream_t s)
{
    ProfScope ps(K_DOWN_I8, s);
    const dim3 g(ex.d_model / 16, T);
    // a wave's share of the super-blocks (the kernel's waves-per-slot rule)
    const int ns = k + ex.S, sbs = ex.d_ff / 64;
    const int wps = ns > DC_NW / 2 ? 1 : (ns > DC_NW / 4 ? 2 : (ns > 1 ? 4 : 8));
    const bool long_share = (sbs + wps - 1) / wps > 12;
#define DC1(F, L, KC) hipLaunchKernelGGL((down_combine_kernel<F, L, KC>), g, dim3(64 * DC_NW), 0, s, h_hi, h_lo, \
                                         ex.d_ff, reinterpret_cast<const int8_t *>(ex.down), ex.down_scales, \
                                         ex.d_model, topk_idx, topk_w, po.inv, T, k, ex.E, ex.S, out)
#define DC(F, L) do { if (long_share) DC1(F, L, 4); else DC1(F, L, 6); } while (0)
    switch (ex.fmt) {
    case W_Q8_0: DC(W_Q8_0, L_PLAIN); break;
    case W_I8_ROW: DC(W_I8_ROW, L_PLAIN); break;
    case W_Q8_0_TILED: DC(W_Q8_0, L_TILED); break;
    default: DC(W_I8_ROW, L_TILED); break;
    }
#undef DC
#undef DC1
    return hipGetLastError();
}

hipError_t launch_down_int8(const uint16_t *h_hi, const uint16_t *h_lo, const ExpertsDev &ex, int T,
                            int k, const PermuteOut &po, const int32_t *topk_idx, const float *topk_w, float *out,
                            float *ybuf, hipStream_t s)
{
    if (down_combine_fits(T, k, ex)) return launch_down_combine(h_hi, h_lo, ex, T, k, po, topk_idx, topk_w, out, s);
    {
        ProfScope ps(K_DOWN_I8, s);
        switch (ex.fmt) {
        case W_Q8_0: launch_down_t<W_Q8_0, L_PLAIN>(s, h_hi, h_lo, ex, T, k, po, ybuf); break;
        case W_I8_ROW: launch_down_t<W_I8_ROW, L_PLAIN>(s, h_hi, h_lo, ex, T, k, po, ybuf); break;
        case W_Q8_0_TILED: launch_down_t<W_Q8_0, L_TILED>(s, h_hi, h_lo, ex, T, k, po, ybuf); break;
        default: launch_down_t<W_I8_ROW, L_TILED>(s, h_hi, h_lo, ex, T, k, po, ybuf); break;
        }
    }
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    return launch_combine_rows(ybuf, po.inv, topk_w, T, k, ex.d_model, 1, ex.S, out, s);
}

hipError_t launch_repack_tiled(const int8_t *src, const uint16_t *ssrc, int E, int R, int K, int M,
                               int8_t *dst, uint16_t *sdst, hipStream_t s)
{
    const size_t lanes = (size_t)E * (R / M / 16) * (K / 64) * M * 64;
    hipLaunchKernelGGL(repack_tiled_kernel, dim3((unsigned)((lanes + 255) / 256)), dim3(256), 0, s,
                       src, ssrc, E, R, K, M, dst, sdst);
    return hipGetLastError();
}

hipError_t launch_combine_rows(const float *ybuf, const int32_t *inv, const float *topk_w, int T,
                               int k, int d, int nchunk, int S, float *out, hipStream_t s)
{
    ProfScope ps(K_COMBINE, s);
    if (nchunk == 1)
        hipLaunchKernelGGL(combine_rows4_kernel, dim3((d / 4 + 255) / 256, T), dim3(256), 0, s, ybuf, inv,
                           topk_w, k, d, T, S, out);
    else
        hipLaunchKernelGGL(combine_rows_kernel, dim3(d / 32, T), dim3(256), 0, s, ybuf, inv,
                           topk_w, k, d, nchunk, T, S, out);
    return hipGetLastError();
}

}  // namespace moe
