// Host-side launchers of the gfx950 kernels (internal to the library; the public interface is
// include/moe.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

constexpr int MAX_E = 512;       // experts per layer
constexpr int MAX_E_BITS = 9;
constexpr int MAX_K = 64;        // experts per token
constexpr int MAX_SHARED = 4;    // shared experts per layer

// Kernel kinds for the opt-in HIP-event timer (names in prof.hip).
enum KernelKind {
    K_ROUTER = 0, K_TOPK, K_PERMUTE, K_GATEUP_I8, K_DOWN_I8, K_COMBINE, K_UP_E2M1, K_DOWN_E2M1,
    K_QUANT, K_GG_GATEUP, K_GG_DOWN, K_COUNT
};

// Brackets one kernel launch with HIP events on its stream while timing is enabled.
class ProfScope {
  public:
    ProfScope(int kind, hipStream_t s);
    ~ProfScope();
    ProfScope(const ProfScope &) = delete;
    ProfScope &operator=(const ProfScope &) = delete;

  private:
    int kind_;
    hipStream_t stream_;
    void *start_;
};

// Per-active-expert record written by the permute step, SLOT_INT4 int4 (128 bytes) each:
// int4 0 = {expert, first permuted row, pair count, 0}; ints 4 .. 4 + SLOT_TOKS - 1 = the token of
// the expert's pairs 0 .. SLOT_TOKS - 1 (0 past the count).  Expert kernels read it with one load.
constexpr int SLOT_INT4 = 8;
constexpr int SLOT_TOKS = 16;

__device__ __forceinline__ int slot_token(const int4 *slots, int slot, int m)
{
    return reinterpret_cast<const int *>(slots + (size_t)slot * SLOT_INT4)[4 + m];
}

// Device arrays the permute step writes.
struct PermuteOut {
    int32_t *counts;    // [E]
    int32_t *offsets;   // [E+1]
    int32_t *perm;      // [P]
    int32_t *inv;       // [P]
    int4 *slots;        // [E][SLOT_INT4] per active expert, ascending (see below)
    int32_t *n_active;  // [1]
    int32_t *tile_off;  // [E+1] prefix of ceil(count / BM), or nullptr
    int32_t *scratch;   // [permute_scratch_ints(P, E)] for the multi-block permute, or nullptr
    int4 *tiles;        // [prefill_tile_bound(P, E)] per BM-row tile {expert, first row, rows, 0},
                        // tiles 0 .. tile_off[E] - 1 written when BM > 0, or nullptr
};

int permute_scratch_ints(int P, int E);

// Read-only view of the experts, as the kernels take it.
struct ExpertsDev {
    int fmt, E, S, d_model, d_ff;     // E routed experts, then S shared ones in the arrays
    const void *gate_up, *gate_up_scales, *down, *down_scales;
};

hipError_t launch_router_logits(const void *x, int xtype, int T, int d, const float *Wr,
                                const float *bias, int E, double *logits, hipStream_t s);
hipError_t launch_topk(const double *logits, int T, int E, int k, int32_t *idx, float *w,
                       hipStream_t s);
// S shared experts: slot records, permuted rows P .. P + S T - 1 and tiles after the routed ones
hipError_t launch_select_permute(const double *logits, const int32_t *idx_in, int T, int k, int E,
                                 int32_t *topk_idx, float *topk_w, const PermuteOut &po, int BM, int S,
                                 hipStream_t s);

// Q8_0 / I8_ROW experts on the bf16 matrix cores.
// Inputs and outputs of the gate/up kernel's own routing (logits == nullptr: the permute step's
// records are read instead); see route_slot.
struct RouteIn {
    const double *logits;   // [T][E] fp64 router logits
    int E, S;               // routed and shared experts
    int32_t *topk_idx;      // [T k] written: selected experts per token, best first
    float *topk_w;          // [T k] written: their renormalised weights
    int32_t *perm, *inv;    // written for the pairs (and the shared rows) as the permute step does
    int4 *slots;            // written: one record per active slot
    int32_t *n_active;      // written: active routed experts + S
};
bool gateup_can_route(int T, int k, int E);
hipError_t launch_gateup_int8(const void *x, int xtype, int T, int k, const ExpertsDev &ex, int act,
                              const PermuteOut &po, uint16_t *h_hi, uint16_t *h_lo, const RouteIn &ri,
                              hipStream_t s);
// topk_idx: the routing in use (ids clamped to [0, E) as the permute clamps them)
hipError_t launch_down_int8(const uint16_t *h_hi, const uint16_t *h_lo, const ExpertsDev &ex, int T,
                            int k, const PermuteOut &po, const int32_t *topk_idx, const float *topk_w, float *out,
                            float *ybuf, hipStream_t s);
// T <= 2 with the token's h rows within the LDS budget: down and the weighted combine in one
// kernel, writing out directly (no y buffer)
bool down_combine_fits(int T, int k, const ExpertsDev &ex);
hipError_t launch_down_combine(const uint16_t *h_hi, const uint16_t *h_lo, const ExpertsDev &ex, int T, int k,
                               const PermuteOut &po, const int32_t *topk_idx, const float *topk_w, float *out,
                               hipStream_t s);
hipError_t launch_repack_tiled(const int8_t *src, const uint16_t *ssrc, int E, int R, int K, int M,
                               int8_t *dst, uint16_t *sdst, hipStream_t s);
hipError_t launch_combine_rows(const float *ybuf, const int32_t *inv, const float *topk_w, int T,
                               int k, int d, int nchunk, int S, float *out, hipStream_t s);

// E2M1 experts (VALU decode).  ri.logits != nullptr: the up blocks route the batch themselves
// (route_slot_any), when up_e2m1_can_route allows it.
// gmask: [E + S][2][d_ff / 16] bytes (e2m1_mask_bytes), the zero-skip masks of each slot's first
// two pairs, written by the lane-group up kernel and read by the zero-skip down projection.
bool up_e2m1_can_route(int T, int k, int E, int d_model);
size_t e2m1_mask_bytes(int E, int S, int d_ff);
hipError_t launch_up_e2m1(const void *x, int xtype, int T, int k, const ExpertsDev &ex, int act,
                          const PermuteOut &po, float *h, const RouteIn &ri, uint8_t *gmask, hipStream_t s);
hipError_t launch_down_e2m1(const float *h, const ExpertsDev &ex, int T, int k, bool zero_skip,
                            const PermuteOut &po, float *partial, int nchunk, const uint8_t *gmask, hipStream_t s);
int e2m1_down_chunks(int d_ff, int T);   // partial sums per pair row (the down block shape depends on T)

// int8-activation prefill path (int8 matrix cores), and its E4M3 twin (fp8 matrix cores): the
// grouped GEMMs pick the kind from the weight format.
// h of the permuted pairs quantised per row into the down GEMM's 128-row A tiles
// (prefill_h_tiles_bytes of codes; rows past a tile's pair count are left unwritten)
size_t prefill_h_tiles_bytes(int P, int E, int d_ff);
// fp8: E4M3 codes by rule Q8 instead of int8 codes by rule Q (prefill_i8.hip)
hipError_t launch_quantize_h_tiles(const float *h, int T, int k, int E, int S, int d_ff, const PermuteOut &po,
                                   int8_t *q, float *scale, bool fp8, hipStream_t s);
// slot_order: codes of each 64-column block in the grouped GEMMs' lane order (see prefill_i8.hip)
hipError_t launch_quantize_rows(const void *v, int xtype, int rows, int cols, int8_t *q,
                                float *scale, bool slot_order, bool fp8, hipStream_t s);
int prefill_tile_rows();
// bound on the number of BM-row tiles of P pairs over E experts (rounded up to 8)
int prefill_tile_bound(int P, int E);
hipError_t launch_ggemm_gateup_i8(const int8_t *xq, const float *sx, int T, int k, const ExpertsDev &ex,
                                  const PermuteOut &po, float *h, hipStream_t s);
hipError_t launch_ggemm_down_i8(const int8_t *hq, const float *sh, int T, int k, const ExpertsDev &ex,
                                const PermuteOut &po, float *ybuf, hipStream_t s);

// Diagnostics (diag.hip): the workspace's intermediate activations in pair order.
// h32 != nullptr: fp32 h rows; otherwise the sum of the two bf16 planes.
hipError_t launch_unpermute_h(const float *h32, const uint16_t *h_hi, const uint16_t *h_lo, const int32_t *perm,
                              int P, int rows, int d_ff, float *out, hipStream_t s);
// prefill h codes and scales out of the down GEMM's tiles (tile_bound blocks; tile count at tile_off[E])
hipError_t launch_untile_hq(const int8_t *q, const float *sh, const PermuteOut &po, int E, int tile_bound, int P,
                            int d_ff, int8_t *out_q, float *out_s, hipStream_t s);

}  // namespace moe
