/*
 * moe.h - C ABI of a HIP (gfx950 / MI355X) library for the inference forward pass of one sparse
 * Mixture-of-Experts FFN layer.
 *
 * The layer, per token t (x[t] has d_model values):
 *   1. router:  l[e] = x[t] . W_router[e] + b[e];  p = softmax(l) over all E experts;
 *               S = the k experts ranked by (l descending, expert index ascending);
 *               w_j = p[S_j] / sum_j' p[S_j'].
 *      (Squeezing a 26B MoE onto the cheapest Inferentia instance, "Memory math": top-8 of 128;
 *       Why very large MoEs can be served scattered, sections 1 and 4: top-4 of 128, the router
 *       picks the experts first.)
 *   2. gather:  each (token, slot) pair is multiplied by the expert its id names (mul_mat_id)
 *      (Running Gemma 4 26B at 5 tokens/s on a 13-year-old Xeon, "Three-part fix").
 *   3. gate/up + activation: SwiGLU on the stacked gate_up matrix, gate rows first,
 *      h = silu(W_gate x) * (W_up x) (same page, "Broken op path in non-AVX2 builds" and
 *      "Three-part fix"); or ungated ReLU^2 on an up-only matrix, h = max(W_up x, 0)^2
 *      (Running NVIDIA's 120B Nemotron-3.5-Super on an 8 GB GPU, "bytes per token").
 *   4. down:    y_j = W_down[S_j] h_j.  With MOE_F_ZERO_SKIP (E2M1 experts) only the 16-neuron
 *      groups of h holding a nonzero value are read, from a neuron-major down matrix (same
 *      Nemotron page, "How the engine works", step 4).
 *   5. combine: out[t] = sum_{j=0..k-1} w_j y_j, summed in a fixed order without atomics (slot
 *      order; for batches of at most 2 tokens, slots j, j+8, ... first, then those sums in order
 *      of j), so the result is bitwise reproducible (same Nemotron page, "How correctness is
 *      checked").
 *
 * Conventions for every entry point:
 *  - Array pointers are DEVICE pointers owned by the caller, 16-byte aligned.  The library never
 *    allocates, frees or keeps them.  Structs passed by pointer are host memory, read during the
 *    call only.
 *  - `stream` is a hipStream_t (NULL = the null stream).  All work is enqueued on it and the call
 *    returns without waiting: outputs are valid once the caller synchronises the stream.  No
 *    device-to-host synchronisation happens inside a call.
 *  - Argument checks are synchronous and happen before any launch; a failed check launches
 *    nothing.  Kernel launch failures return MOE_EHIP; faults during execution surface at the
 *    caller's synchronisation.  No C++ exception crosses this interface.
 *  - The workspace `ws` (ws_bytes >= moe_workspace_bytes(...)) is caller-owned device memory;
 *    its contents on return are unspecified.  Calls that share a workspace must be ordered
 *    (same stream); the library keeps no other state, so calls on different streams with
 *    different workspaces may overlap.
 *  - Results are deterministic: the same inputs give bitwise-identical outputs.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_ABI_VERSION 1

typedef enum {
    MOE_OK = 0,
    MOE_EINVAL = -1,        /* bad argument: null / misaligned pointer, bad size, k > E, ... */
    MOE_EUNSUPPORTED = -2,  /* valid arguments but a combination this library does not run */
    MOE_EWORKSPACE = -3,    /* ws_bytes < moe_workspace_bytes(...) */
    MOE_EHIP = -4,          /* a HIP runtime call failed (launch error) */
    MOE_ESCRATCH = -5       /* moe_layer_forward_static: the call needs more than its static buffer */
} moe_status;

/* Element type of the activations x [T][d_model], row-major. */
typedef enum { MOE_X_F32 = 0, MOE_X_BF16 = 1 } moe_xtype;

/* Expert weight formats.
 *  MOE_W_Q8_0:   blocks of 32 int8 values along the reduction dimension K with one fp16 scale
 *                each, value = q * scale (Gemma on a Xeon page, summary: Q8_0).
 *  MOE_W_I8_ROW: int8 values with one fp32 scale per output row, value = q * scale (Inferentia
 *                page, "Memory math": per-channel int8).
 *  MOE_W_E2M1_G16: 4-bit E2M1 codes (OCP MX v1.0 FP4), two per byte, element 2i in the low
 *                nibble, one fp16 scale per 16 contiguous values; the down matrix neuron-major
 *                (Nemotron page, "bytes per token" and "How the engine works" step 4; that page
 *                uses 1-byte scales, this format fp16 ones).
 *  MOE_W_FP8_ROW: 8-bit E4M3 codes (OCP 8-bit Floating Point Specification v1.0: sign, 4
 *                exponent bits with bias 7, 3 mantissa bits; 0x7F / 0xFF are NaN, largest finite
 *                magnitude 448) with one fp32 scale per output row, value = e4m3(q) * scale; the
 *                same arrays as MOE_W_I8_ROW.  Runs only with MOE_F_PREFILL_FP8.  The
 *                Inferentia page's fp4 section names INT8 and FP8 as the two quantised types its
 *                inference stack runs; this is the FP8 one at the per-row granularity. */
typedef enum {
    MOE_W_Q8_0 = 0, MOE_W_I8_ROW = 1, MOE_W_E2M1_G16 = 2,
    MOE_W_Q8_0_TILED = 3, MOE_W_I8_ROW_TILED = 4,  /* same values, tiled layout (below) */
    MOE_W_FP8_ROW = 5, MOE_W_FP8_ROW_TILED = 6
} moe_wformat;

typedef enum { MOE_ACT_SWIGLU = 0, MOE_ACT_RELU2 = 1 } moe_act;

enum {
    /* E2M1 experts: the down projection reads only 16-neuron groups of h holding a nonzero
     * value.  The output equals the dense down projection's bit for bit. */
    MOE_F_ZERO_SKIP = 1u,
    /* I8_ROW or Q8_0 (plain or tiled) + SwiGLU only: batched-prefill definition.  x is
     * quantised per token and h per (token, slot) pair to int8 by the rule
     * q = clamp(rne(fp32(v * fp32(127/max|v|))), +-127), scale = fp32(max|v| / 127); both
     * projections are int8 x int8 -> int32 products on the matrix cores, rescaled in fp32 (see
     * moe_quantize_rows_i8): by the row scale (I8_ROW), or per 32-wide Q8_0 block by its fp16
     * scale, blocks added in K order (Q8_0). */
    MOE_F_PREFILL_I8 = 4u,
    /* FP8_ROW (plain or tiled) + SwiGLU only, and the only way FP8_ROW experts run: the same
     * batched-prefill definition with E4M3 codes in place of int8 ones.  x per token and h per
     * pair: a = max|v|; a = 0 gives codes 0 and scale 0; otherwise q = E4M3 code of fp32(v *
     * fp32(448 / a)), round to nearest, ties to even, and scale = fp32(a / 448) (see
     * moe_quantize_rows_fp8).  Both projections are E4M3 x E4M3 products (each exact in fp32)
     * summed in fp32 on the matrix cores, then rescaled by the two row scales.  Not combinable
     * with MOE_F_PREFILL_I8 (MOE_EINVAL). */
    MOE_F_PREFILL_FP8 = 8u
};

/*
 * The E experts of one layer.  rows = 2*d_ff for SwiGLU (gate rows 0..d_ff-1, then up rows),
 * d_ff for ReLU^2 (up rows only).
 *   gate_up:        Q8_0 / I8_ROW: int8 [E][rows][d_model];  E2M1: uint8 [E][rows][d_model/2];
 *                   FP8_ROW: uint8 E4M3 [E][rows][d_model]
 *   gate_up_scales: Q8_0: fp16 [E][rows][d_model/32];  I8_ROW / FP8_ROW: fp32 [E][rows];
 *                   E2M1: fp16 [E][rows][d_model/16]
 *   down:           Q8_0 / I8_ROW: int8 [E][d_model][d_ff];  FP8_ROW: uint8 E4M3 [E][d_model][d_ff];
 *                   E2M1: neuron-major uint8 [E][d_ff][d_model/2] (neuron f's d_model codes
 *                   contiguous, output 2i in the low nibble)
 *   down_scales:    Q8_0: fp16 [E][d_model][d_ff/32];  I8_ROW / FP8_ROW: fp32 [E][d_model];
 *                   E2M1: fp16 [E][d_ff/16][d_model] (scale of output o for neurons 16g..16g+15
 *                   at [g][o])
 *
 * Tiled layout (MOE_W_Q8_0_TILED, MOE_W_I8_ROW_TILED, MOE_W_FP8_ROW_TILED; made by
 * moe_repack_experts).  A matrix of
 * R rows by K columns (gate_up: R = rows, K = d_model, in M = 2 halves gate/up for SwiGLU or
 * M = 1; down: R = d_model, K = d_ff, M = 1) is cut into tiles of 16 rows by 64 columns, 1 KB
 * each.  Row r = m * (R/M) + 16 t + n (0 <= n < 16), column 64 s + 32 j + 8 g + i (j, g, i in
 * 0..1, 0..3, 0..7) is byte 16 (n + 16 g) + 8 j + i of tile ((e * (R/M/16) + t) * (K/64) + s) *
 * M + m: one 16-byte slice per lane of a 64-lane wavefront, so a wave streams whole tiles.  Q8_0
 * scales follow the tiles: 32 fp16 per tile, the scale of row n's block 2s + j at 2n + j.
 * I8_ROW and FP8_ROW scales keep the plain [E][rows] / [E][d_model] fp32 arrays.  The arrays have exactly the
 * sizes of the plain ones.
 *
 * Shared experts (n_shared = S, 0 <= S <= 4): the arrays hold E + S experts, the routed ones
 * first; experts E .. E+S-1 are the shared experts (the dense MLP of a dual-path FFN, Inferentia
 * page "all-int8 squeeze"; the shared experts beside the routed ones, Nemotron page "bytes per
 * token").  Every token also goes through each of them and their outputs are added with weight 1
 * as slots k .. k+S-1 of the combine.  Routing (E experts) is unaffected.
 */
typedef struct {
    int32_t fmt;            /* moe_wformat */
    int32_t E, d_model, d_ff;   /* E routed experts */
    const void *gate_up;
    const void *gate_up_scales;
    const void *down;
    const void *down_scales;
    int32_t n_shared;       /* shared experts after the E routed ones (see above) */
} moe_experts;

/* Size limits checked by every entry point (MOE_EINVAL beyond them):
 *   1 <= T <= 32768;  1 <= E <= 512;  1 <= k <= min(E, 64);
 *   d_model a multiple of 64, 64 <= d_model <= 16384;  d_ff a multiple of 32, 32 <= d_ff <= 16384,
 *   and a multiple of 64 for the int8 and fp8 formats (plain and tiled);  0 <= n_shared <= 4.
 */

/* Bytes of workspace the given call needs (0 if the arguments are invalid).  T, k, the expert
 * shapes, act and flags decide it; pointers inside *ex are not read. */
size_t moe_workspace_bytes(int32_t T, int32_t k, const moe_experts *ex, int32_t act, uint32_t flags);

/* Bytes of workspace moe_route needs for T tokens and E experts. */
size_t moe_route_workspace_bytes(int32_t T, int32_t E);

/*
 * Router only (step 1).  x [T][d_model] (xtype), w_router fp32 [E][d_model], router_bias fp32 [E]
 * or NULL.  Writes topk_idx int32 [T][k] in rank order (logit descending, ties to the lower
 * index) and topk_w fp32 [T][k] (renormalised, sums to 1).  Logits are accumulated in fp64, so
 * the selection is the exact-arithmetic one except for logits closer than ~1e-12 relative.
 */
moe_status moe_route(const void *x, int32_t xtype, int32_t T, int32_t d_model,
                     const float *w_router, const float *router_bias, int32_t E, int32_t k,
                     int32_t *topk_idx, float *topk_w, void *ws, size_t ws_bytes, void *stream);

/*
 * Permutation of the P = T*k (token, slot) pairs into expert groups (the gather's index
 * arrays).  topk_idx int32 [T][k], each id in [0, E).  The ids live on the device and are not
 * checked on the host: an id outside [0, E) is clamped into that range on the device, so it
 * cannot cause an out-of-bounds access, and the pair is then treated as routed to the clamped
 * id.  The same holds for moe_experts_forward.
 * Writes counts int32 [E] (pairs per expert), offsets int32 [E+1] (exclusive prefix sum),
 * perm int32 [P] (perm[r] = pair id placed at row r, pairs sorted by (expert, pair id)) and
 * inv int32 [P] (inv[perm[r]] = r).  Needs no workspace.
 */
moe_status moe_permute(const int32_t *topk_idx, int32_t T, int32_t k, int32_t E,
                       int32_t *counts, int32_t *offsets, int32_t *perm, int32_t *inv,
                       void *stream);

/*
 * The whole layer (steps 1-5).  x [T][ex->d_model]; w_router fp32 [E][d_model]; router_bias
 * fp32 [E] or NULL; out fp32 [T][d_model].  topk_idx_out / topk_w_out: optional ([T][k]) copies
 * of the routing, or NULL.
 * Supported: Q8_0 / I8_ROW with SwiGLU or ReLU^2; E2M1 with ReLU^2 (flags 0 or ZERO_SKIP) or
 * SwiGLU (flags 0); PREFILL_I8 with Q8_0 or I8_ROW + SwiGLU; PREFILL_FP8 with FP8_ROW + SwiGLU.
 * Other combinations: MOE_EUNSUPPORTED.
 */
moe_status moe_layer_forward(const void *x, int32_t xtype, int32_t T, const float *w_router,
                             const float *router_bias, const moe_experts *ex, int32_t k,
                             int32_t act, uint32_t flags, float *out, int32_t *topk_idx_out,
                             float *topk_w_out, void *ws, size_t ws_bytes, void *stream);

/*
 * moe_layer_forward without a caller workspace, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).  The
 * workspace is a static device buffer of MOE_STATIC_WORKSPACE_BYTES (64 MiB) inside the library:
 * each GPU the library runs on holds one copy until the process ends, its address looked up
 * (hipGetSymbolAddress) on the first call for that device.  The call itself allocates nothing
 * and frees nothing.  Arguments, checks, outputs and results are those of moe_layer_forward
 * (bit for bit); a call whose workspace (moe_workspace_bytes) exceeds the buffer returns
 * MOE_ESCRATCH before anything is launched (decode batches fit, e.g. T <= 64 on the Gemma-4 and
 * MiniMax-M3 shapes; the large prefill batches do not).  Every call on one GPU shares that GPU's
 * buffer and nothing in it needs to start cleared: calls on one GPU must not overlap (order them
 * on one stream), or they race.  The work runs on the device of `stream` (the current device for
 * the null stream).
 */
#define MOE_STATIC_WORKSPACE_BYTES ((size_t)64 << 20)
moe_status moe_layer_forward_static(const void *x, int32_t xtype, int32_t T, const float *w_router,
                                    const float *router_bias, const moe_experts *ex, int32_t k,
                                    int32_t act, uint32_t flags, float *out, int32_t *topk_idx_out,
                                    float *topk_w_out, void *stream);

/*
 * Steps 2-5 with the routing given: topk_idx int32 [T][k] (ids in [0, E)), topk_w fp32 [T][k].
 * Same formats, flags and output as moe_layer_forward; lets the expert FFN be checked with a
 * routing fixed from outside.
 */
moe_status moe_experts_forward(const void *x, int32_t xtype, int32_t T, const int32_t *topk_idx,
                               const float *topk_w, const moe_experts *ex, int32_t k, int32_t act,
                               uint32_t flags, float *out, void *ws, size_t ws_bytes,
                               void *stream);

/*
 * Re-lays plain Q8_0 / I8_ROW / FP8_ROW experts out in the tiled layout (a pure byte permutation,
 * done once when the weights are loaded).  src->fmt is MOE_W_Q8_0, MOE_W_I8_ROW or MOE_W_FP8_ROW
 * (the last with act = SwiGLU only); dst->fmt must be the
 * matching *_TILED value with the same E, n_shared, d_model, d_ff, and dst's four arrays (same
 * sizes as src's, not overlapping them) receive the tiled bytes of all E + n_shared experts.  act
 * decides the gate/up halves.
 */
moe_status moe_repack_experts(const moe_experts *src, int32_t act, const moe_experts *dst,
                              void *stream);

/*
 * The activation quantiser of the PREFILL_I8 path, per row of a [rows][cols] matrix v (xtype):
 * a = max|v|; a = 0 gives q = 0, scale = 0; otherwise q = clamp(round_half_even(fp32(v *
 * fp32(127 / a))), -127, 127) and scale = fp32(a / 127).  q int8 [rows][cols], scale fp32
 * [rows].  cols a multiple of 64, 64 <= cols <= 16384.
 */
moe_status moe_quantize_rows_i8(const void *v, int32_t xtype, int32_t rows, int32_t cols,
                                int8_t *q, float *scale, void *stream);

/*
 * The activation quantiser of the PREFILL_FP8 path, per row of a [rows][cols] matrix v (xtype):
 * a = max|v|; a = 0 gives codes 0 and scale 0; otherwise q = E4M3 code (OCP 8-bit Floating Point
 * v1.0) of fp32(v * fp32(448 / a)) by round to nearest, ties to the even code, and scale =
 * fp32(a / 448).  q uint8 [rows][cols], scale fp32 [rows].  cols a multiple of 64, 64 <= cols <=
 * 16384.  A value that is NaN or infinite leaves its row's codes and scale unspecified.
 */
moe_status moe_quantize_rows_fp8(const void *v, int32_t xtype, int32_t rows, int32_t cols,
                                 uint8_t *q, float *scale, void *stream);

/*
 * Diagnostics: the intermediate activations h (step 3's output, the down projection's input)
 * that the last moe_layer_forward (with_router = 1) or moe_experts_forward (with_router = 0)
 * call on workspace ws left there.  T, k, *ex, act and flags must be that call's; the stream must
 * be ordered after it, with nothing else run on ws in between (otherwise the contents are
 * unspecified, though every access stays inside ws and the outputs).  Writes, in pair order
 * (row t k + j for slot j of token t, then row T k + s T + t for shared expert s):
 *   h  fp32 [T k + S T][d_ff]: the h the down projection used (int8 experts outside the prefill
 *      flags: the sum of the two bf16 terms it multiplies);
 *   with MOE_F_PREFILL_I8 or MOE_F_PREFILL_FP8 only (otherwise both NULL, else MOE_EINVAL):
 *   hq [T k + S T][d_ff] the codes of h by rule Q (int8) or Q8 (E4M3 bytes), column order, and
 *   sh fp32 [T k + S T] their row scales.
 * Not part of the layer's path: for checking the layer against a reference and for counting the
 * 16-neuron groups a zero-skip down projection reads.
 */
moe_status moe_read_intermediates(int32_t T, int32_t k, const moe_experts *ex, int32_t act, uint32_t flags,
                                  int32_t with_router, const void *ws, size_t ws_bytes, float *h, void *hq,
                                  float *sh, void *stream);

/*
 * Diagnostics: opt-in per-kernel timing.  While enabled (process-wide), every kernel the library
 * launches is bracketed by hipEventRecord on the launch's stream, which adds small gaps between
 * kernels; use it in a pass of its own.  moe_profile_collect waits for the recorded events and
 * adds each kernel's elapsed time to its kind's totals; moe_profile_get reads kind `kind`
 * (0 <= kind < moe_profile_kinds()): a static name, the launch count and the total milliseconds
 * since the last moe_profile_reset.  Thread-safe; not for use inside HIP graph capture.
 */
moe_status moe_profile_enable(int32_t on);
moe_status moe_profile_collect(void);
void moe_profile_reset(void);
int32_t moe_profile_kinds(void);
moe_status moe_profile_get(int32_t kind, const char **name, int64_t *launches, double *total_ms);

/* A static string naming a status code. */
const char *moe_status_str(int32_t status);

/* MOE_ABI_VERSION of the built library. */
int32_t moe_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */
