/*
 * moe_oracle.c - plain, slow, CPU reference of the inference forward pass of one sparse
 * Mixture-of-Experts FFN layer, in fp64.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's CPU-baseline leg
 * load this library.  The HIP product library neither links nor calls it, and the two share no
 * code: this file has its own fp16 / bf16 / E2M1 / E4M3 decoders, its own routing and its own loops.
 *
 * What it computes, and where the pages say so:
 *
 *  1. Router (top-k of E experts, softmax weights, renormalised to sum 1): "Squeezing a 26B MoE
 *     onto the cheapest Inferentia instance" (molayo1419.me), section "Memory math" (top-8 of 128);
 *     "Why very large MoEs can be served scattered" (tony.banya.ai), section 1 (top-4 of 128) and
 *     section 4 (the router picks the experts first, then their weights are read).  Ties go to the
 *     lower expert index.
 *  2. Gather: each token is multiplied by the experts its ids pick (mul_mat_id): "Running Gemma 4
 *     26B at 5 tokens/s on a 13-year-old Xeon without a GPU" (amuse.peoplentools.com), section
 *     "Three-part fix".
 *  3. Gate/up: the stacked [n_embd, 2*n_ff, n_experts] tensor has gate as its first half and up
 *     as its second; h = silu(gate) * up (same page, "Broken op path in non-AVX2 builds" and
 *     "Three-part fix").  Ungated ReLU^2 experts (up only, h = max(u, 0)^2): "Running NVIDIA's
 *     new 120B Nemotron-3.5-Super on an 8 GB GPU" (molayo1419.me), section "bytes per token".
 *  4. Down: y = W_down h per (token, expert).  Zero-skip form: neurons grouped by 16, a group is
 *     read only if it holds a nonzero activation; down stored neuron-major with one scale per 16
 *     neurons: same Nemotron page, "How the engine works", step 4.
 *  5. Combine: out[t] = sum over the k slots of w * y, through a per-(token, expert) buffer summed
 *     in a fixed order: same Nemotron page, "How correctness is checked".
 *
 * Weight formats: Q8_0 = 32 int8 along K plus one fp16 scale (Gemma on a Xeon page, summary);
 * per-row int8 with an fp32 per-output-channel scale (Inferentia page, "Memory math"); E2M1 with
 * one scale per 16 contiguous values (Nemotron page, "bytes per token", "How the engine works"),
 * here with fp16 scales.  E2M1 values: OCP Microscaling Formats v1.0, FP4 E2M1.
 *
 * The int8-activation variant (quantise x per token and h per pair by absmax/127, int32
 * accumulate, then rescale) is the batched-prefill definition; its rounding rule ("rule Q") is
 * fixed in IEEE fp32 with correctly rounded division and round-half-even, the precision the GPU
 * takes the same integer decisions in.  Its fp8 twin (the Inferentia page's fp4 section names
 * INT8 and FP8 as the quantised types its stack runs) replaces the integers by E4M3 codes (OCP
 * 8-bit Floating Point Specification v1.0) and 127 by 448 ("rule Q8"), with per-row E4M3 weights;
 * every E4M3 x E4M3 product is exact and the sums are exact in fp64.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { OX_F32 = 0, OX_BF16 = 1 };
enum { OW_Q8_0 = 0, OW_I8_ROW = 1, OW_E2M1_G16 = 2, OW_FP8_ROW = 5 };
enum { OA_SWIGLU = 0, OA_RELU2 = 1 };

typedef struct {
    int32_t fmt, E, d_model, d_ff;
    const void *gate_up;        /* Q8_0 / I8_ROW: int8 [E][rows][d_model]; E2M1: uint8 [E][rows][d_model/2] */
    const void *gate_up_scales; /* Q8_0: fp16 [E][rows][d_model/32]; I8_ROW: fp32 [E][rows];
                                   E2M1: fp16 [E][rows][d_model/16] */
    const void *down;           /* Q8_0 / I8_ROW: int8 [E][d_model][d_ff];
                                   E2M1 neuron-major: uint8 [E][d_ff][d_model/2] */
    const void *down_scales;    /* Q8_0: fp16 [E][d_model][d_ff/32]; I8_ROW: fp32 [E][d_model];
                                   E2M1: fp16 [E][d_ff/16][d_model] */
    int32_t n_shared;           /* shared experts E .. E+n_shared-1 beside the E routed ones (the
                                   arrays then hold E + n_shared experts) */
} oracle_experts;

/*
 * Shared experts (the dense MLP beside the routed experts in Gemma 4's dual-path FFN: Inferentia
 * page, "all-int8 squeeze" item 2; the shared experts Nemotron keeps on the GPU: Nemotron page,
 * "bytes per token"): every token also goes through each shared expert, whose output is added
 * with weight 1 after the k routed slots, in shared-expert order.  The functions below take the
 * routed (idx, w) and treat the shared experts as k + s extra slots of every token.
 * Returns the extended arrays (caller frees) and fills *k2.
 */
static int with_shared(const int32_t *idx, const double *w, int T, int k, const oracle_experts *ex,
                       int32_t **idx2, double **w2, int *k2)
{
    int S = ex->n_shared, kk = k + S;
    *idx2 = (int32_t *)malloc(sizeof(int32_t) * (size_t)(T > 0 ? T : 1) * kk);
    *w2 = (double *)malloc(sizeof(double) * (size_t)(T > 0 ? T : 1) * kk);
    if (!*idx2 || !*w2) {
        free(*idx2); free(*w2);
        return -2;
    }
    for (int t = 0; t < T; ++t) {
        for (int j = 0; j < k; ++j) {
            (*idx2)[(long)t * kk + j] = idx[(long)t * k + j];
            (*w2)[(long)t * kk + j] = w[(long)t * k + j];
        }
        for (int sh = 0; sh < S; ++sh) {
            (*idx2)[(long)t * kk + k + sh] = ex->E + sh;
            (*w2)[(long)t * kk + k + sh] = 1.0;
        }
    }
    *k2 = kk;
    return 0;
}

/* ------------------------------------------------------------------------------------------ */
/* Scalar decoders, from the format definitions.                                              */
/* ------------------------------------------------------------------------------------------ */

/* IEEE 754 binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits. */
double oracle_half_to_double(uint16_t h)
{
    int sign = (h >> 15) & 1, ex = (h >> 10) & 31, fr = h & 1023;
    double v;
    if (ex == 0)
        v = ldexp((double)fr, -24);                    /* subnormal: fr * 2^-14 / 1024 */
    else if (ex == 31)
        v = fr ? NAN : INFINITY;
    else
        v = ldexp(1.0 + fr / 1024.0, ex - 15);
    return sign ? -v : v;
}

/* bfloat16: the upper 16 bits of an IEEE binary32. */
double oracle_bf16_to_double(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

/* OCP MX FP4 E2M1: bit 3 sign, bits 2..1 exponent (bias 1), bit 0 mantissa; exponent 0 is the
 * subnormal 0 / 0.5. */
double oracle_e2m1_value(unsigned code)
{
    int sign = (code >> 3) & 1, ex = (code >> 1) & 3, m = code & 1;
    double v = ex == 0 ? 0.5 * m : ldexp(1.0 + 0.5 * m, ex - 1);
    return sign ? -v : v;
}

/* OCP 8-bit floating point E4M3 (OCP 8-bit Floating Point Specification v1.0, "E4M3"): bit 7
 * sign, bits 6..3 exponent (bias 7), bits 2..0 mantissa; exponent 0 holds the subnormals m/8 *
 * 2^-6; S.1111.111 is NaN; no infinities; the largest finite magnitude is 1.75 * 2^8 = 448. */
double oracle_e4m3_value(unsigned code)
{
    int sign = (code >> 7) & 1, ex = (code >> 3) & 15, m = code & 7;
    if (ex == 15 && m == 7)
        return NAN;
    double v = ex == 0 ? ldexp((double)m, -9) : ldexp(1.0 + m / 8.0, ex - 7);
    return sign ? -v : v;
}

/* The E4M3 code of an fp32 value by round-to-nearest, ties to the even code; magnitudes from
 * 464 (the midpoint above 448) on have no finite code and give NaN. */
unsigned oracle_e4m3_encode(float f)
{
    double v = fabs((double)f);
    unsigned sign = signbit(f) ? 0x80u : 0u;
    if (v != v || v > 464.0)   /* 464 itself ties to 448, the even code */
        return sign | 0x7Fu;
    int e;
    frexp(v, &e);                         /* v = fr * 2^e, fr in [0.5, 1) */
    e -= 1;                               /* v in [2^e, 2^(e+1)) */
    if (v < ldexp(1.0, -6)) {             /* subnormal step 2^-9 */
        double q = nearbyint(ldexp(v, 9)); /* exact scaling; default rounding: ties to even */
        return sign | (unsigned)q;        /* q == 8 is the smallest normal, code 8 */
    }
    double q = nearbyint(ldexp(v, 3 - e));    /* in [8, 16] */
    if (q == 16.0) {
        q = 8.0;
        e += 1;
    }
    return sign | (unsigned)((e + 7) << 3) | (unsigned)(q - 8.0);
}

static double x_at(const void *x, int xtype, long i)
{
    if (xtype == OX_F32)
        return (double)((const float *)x)[i];
    return oracle_bf16_to_double(((const uint16_t *)x)[i]);
}

static int gate_up_rows(const oracle_experts *ex, int act)
{
    return act == OA_SWIGLU ? 2 * ex->d_ff : ex->d_ff;
}

/* Dequantised gate/up weight of expert e, row n (0..rows-1), column i (0..d_model-1). */
static double w_gate_up(const oracle_experts *ex, int act, int e, int n, int i)
{
    long rows = gate_up_rows(ex, act), d = ex->d_model;
    long row = (long)e * rows + n;
    if (ex->fmt == OW_Q8_0) {
        int8_t q = ((const int8_t *)ex->gate_up)[row * d + i];
        uint16_t s = ((const uint16_t *)ex->gate_up_scales)[row * (d / 32) + i / 32];
        return (double)q * oracle_half_to_double(s);
    }
    if (ex->fmt == OW_I8_ROW) {
        int8_t q = ((const int8_t *)ex->gate_up)[row * d + i];
        return (double)q * (double)((const float *)ex->gate_up_scales)[row];
    }
    {
        uint8_t byte = ((const uint8_t *)ex->gate_up)[row * (d / 2) + i / 2];
        unsigned code = (i & 1) ? (byte >> 4) : (byte & 15);
        uint16_t s = ((const uint16_t *)ex->gate_up_scales)[row * (d / 16) + i / 16];
        return oracle_e2m1_value(code) * oracle_half_to_double(s);
    }
}

/* Dequantised down weight of expert e: output o (0..d_model-1), neuron f (0..d_ff-1). */
static double w_down(const oracle_experts *ex, int e, int o, int f)
{
    long d = ex->d_model, dff = ex->d_ff;
    if (ex->fmt == OW_Q8_0) {
        long row = (long)e * d + o;
        int8_t q = ((const int8_t *)ex->down)[row * dff + f];
        uint16_t s = ((const uint16_t *)ex->down_scales)[row * (dff / 32) + f / 32];
        return (double)q * oracle_half_to_double(s);
    }
    if (ex->fmt == OW_I8_ROW) {
        long row = (long)e * d + o;
        int8_t q = ((const int8_t *)ex->down)[row * dff + f];
        return (double)q * (double)((const float *)ex->down_scales)[row];
    }
    {
        /* neuron-major: neuron f's d_model codes are contiguous; scale S[g][o], g = f / 16 */
        uint8_t byte = ((const uint8_t *)ex->down)[((long)e * dff + f) * (d / 2) + o / 2];
        unsigned code = (o & 1) ? (byte >> 4) : (byte & 15);
        uint16_t s = ((const uint16_t *)ex->down_scales)[((long)e * (dff / 16) + f / 16) * d + o];
        return oracle_e2m1_value(code) * oracle_half_to_double(s);
    }
}

/* ------------------------------------------------------------------------------------------ */
/* Router                                                                                     */
/* ------------------------------------------------------------------------------------------ */

/* Neumaier-compensated dot product of x row t with router row e, plus bias.  Every product of
 * an fp32 (or bf16) by an fp32 is exact in fp64; the compensated sum is accurate to a few ulp. */
static double router_logit(const void *x, int xtype, int t, int d, const float *Wr,
                           const float *bias, int e)
{
    double sum = 0.0, comp = 0.0;
    for (int i = 0; i < d; ++i) {
        double p = x_at(x, xtype, (long)t * d + i) * (double)Wr[(long)e * d + i];
        double s = sum + p;
        if (fabs(sum) >= fabs(p))
            comp += (sum - s) + p;
        else
            comp += (p - s) + sum;
        sum = s;
    }
    sum += comp;
    if (bias)
        sum += (double)bias[e];
    return sum;
}

/* a ranks before b: higher logit first, equal logits -> lower index first */
static int ranks_before(double la, int a, double lb, int b)
{
    return la > lb || (la == lb && a < b);
}

/*
 * Route T tokens.  For each token: logits l[e] = x . W_r[e] + b[e]; softmax p over all E;
 * S = the k experts ranked by (l descending, index ascending); w_j = p[S_j] / sum_j' p[S_j'].
 * Outputs idx [T][k] (rank order), w [T][k]; optionally logits [T][E] and, per token, the
 * smallest gap between adjacent logits among ranks 1..k+1 (a diagnostic for near ties).
 */
int oracle_route(const void *x, int xtype, int T, int d, const float *Wr, const float *bias,
                 int E, int k, int32_t *idx, double *w, double *logits_out, double *min_gap)
{
    if (T < 0 || d < 1 || E < 1 || k < 1 || k > E)
        return -1;
    int rc = 0;
#pragma omp parallel for schedule(dynamic, 1)
    for (int t = 0; t < T; ++t) {
        double *l = (double *)malloc(sizeof(double) * E);
        int *order = (int *)malloc(sizeof(int) * E);
        double *p = (double *)malloc(sizeof(double) * E);
        if (!l || !order || !p) {
            rc = -2;
            free(l); free(order); free(p);
            continue;
        }
        for (int e = 0; e < E; ++e)
            l[e] = router_logit(x, xtype, t, d, Wr, bias, e);
        /* softmax over all E, max-subtracted */
        double mx = l[0];
        for (int e = 1; e < E; ++e)
            if (l[e] > mx) mx = l[e];
        double z = 0.0;
        for (int e = 0; e < E; ++e) {
            p[e] = exp(l[e] - mx);
            z += p[e];
        }
        for (int e = 0; e < E; ++e)
            p[e] /= z;
        /* rank: insertion sort by (l desc, index asc) */
        for (int e = 0; e < E; ++e) {
            int pos = e;
            while (pos > 0 && ranks_before(l[e], e, l[order[pos - 1]], order[pos - 1])) {
                order[pos] = order[pos - 1];
                --pos;
            }
            order[pos] = e;
        }
        double psum = 0.0;
        for (int j = 0; j < k; ++j)
            psum += p[order[j]];
        for (int j = 0; j < k; ++j) {
            idx[(long)t * k + j] = order[j];
            w[(long)t * k + j] = p[order[j]] / psum;
        }
        if (logits_out)
            for (int e = 0; e < E; ++e)
                logits_out[(long)t * E + e] = l[e];
        if (min_gap) {
            int last = k < E ? k : E - 1;
            double g = INFINITY;
            for (int j = 0; j < last; ++j) {
                double gap = l[order[j]] - l[order[j + 1]];
                if (gap < g) g = gap;
            }
            min_gap[t] = g;
        }
        free(l); free(order); free(p);
    }
    return rc;
}

/*
 * Permutation of the P = T*k (token, slot) pairs into expert groups: counts[e] = number of
 * pairs routed to e, offsets = exclusive prefix sum (E+1 entries), perm[r] = the pair placed at
 * row r when pairs are sorted by (expert, pair id), inv[p] = the row of pair p.
 */
int oracle_permute(const int32_t *idx, int P, int E, int32_t *counts, int32_t *offsets,
                   int32_t *perm, int32_t *inv)
{
    for (int e = 0; e < E; ++e)
        counts[e] = 0;
    for (int p = 0; p < P; ++p) {
        if (idx[p] < 0 || idx[p] >= E)
            return -1;
        counts[idx[p]]++;
    }
    offsets[0] = 0;
    for (int e = 0; e < E; ++e)
        offsets[e + 1] = offsets[e] + counts[e];
    int32_t *next = (int32_t *)malloc(sizeof(int32_t) * (E > 0 ? E : 1));
    if (!next)
        return -2;
    for (int e = 0; e < E; ++e)
        next[e] = offsets[e];
    for (int p = 0; p < P; ++p) {
        int r = next[idx[p]]++;
        perm[r] = p;
        inv[p] = r;
    }
    free(next);
    return 0;
}

/* ------------------------------------------------------------------------------------------ */
/* Expert FFN in fp64                                                                         */
/* ------------------------------------------------------------------------------------------ */

static double silu(double g) { return g / (1.0 + exp(-g)); }

/* h for one (token, expert): length d_ff */
static void expert_hidden(const oracle_experts *ex, int act, int e, const void *x, int xtype,
                          int t, double *h)
{
    int d = ex->d_model, dff = ex->d_ff;
    for (int f = 0; f < dff; ++f) {
        if (act == OA_SWIGLU) {
            double g = 0.0, u = 0.0;
            for (int i = 0; i < d; ++i) {
                double xv = x_at(x, xtype, (long)t * d + i);
                g += w_gate_up(ex, act, e, f, i) * xv;
                u += w_gate_up(ex, act, e, dff + f, i) * xv;
            }
            h[f] = silu(g) * u;
        } else {
            double u = 0.0;
            for (int i = 0; i < d; ++i)
                u += w_gate_up(ex, act, e, f, i) * x_at(x, xtype, (long)t * d + i);
            h[f] = u > 0.0 ? u * u : 0.0;
        }
    }
}

/*
 * out [T][d_model] = sum_j w[t][j] * W_down[e_j] h(t, e_j), slots in order j = 0..k-1.
 * Routing is an input (idx, w).  If o_list is non-NULL only the n_o output columns it names are
 * computed, and out is [T][n_o].  If h_out is non-NULL it receives h per pair, [T*k][d_ff].
 */
int oracle_experts_forward(const void *x, int xtype, int T, const int32_t *idx, const double *w,
                           int k, const oracle_experts *ex, int act, const int32_t *o_list,
                           int n_o, double *out, double *h_out)
{
    if (ex->n_shared > 0) {                   /* h_out then holds T * (k + n_shared) rows */
        int32_t *idx2; double *w2; int k2;
        if (with_shared(idx, w, T, k, ex, &idx2, &w2, &k2)) return -2;
        oracle_experts e2 = *ex;
        e2.E += e2.n_shared;
        e2.n_shared = 0;
        int rc = oracle_experts_forward(x, xtype, T, idx2, w2, k2, &e2, act, o_list, n_o, out, h_out);
        free(idx2); free(w2);
        return rc;
    }
    int d = ex->d_model, dff = ex->d_ff;
    int no = o_list ? n_o : d;
    long P = (long)T * k;
    double *h = (double *)malloc(sizeof(double) * (P > 0 ? P : 1) * dff);
    if (!h)
        return -2;
    for (long p = 0; p < P; ++p)
        if (idx[p] < 0 || idx[p] >= ex->E) {
            free(h);
            return -1;
        }
#pragma omp parallel for schedule(dynamic, 1)
    for (long p = 0; p < P; ++p)
        expert_hidden(ex, act, idx[p], x, xtype, (int)(p / k), h + p * dff);
#pragma omp parallel for collapse(2) schedule(static)
    for (int t = 0; t < T; ++t)
        for (int oi = 0; oi < no; ++oi) {
            int o = o_list ? o_list[oi] : oi;
            double acc = 0.0;
            for (int j = 0; j < k; ++j) {
                long p = (long)t * k + j;
                int e = idx[p];
                double y = 0.0;
                for (int f = 0; f < dff; ++f)
                    y += w_down(ex, e, o, f) * h[p * dff + f];
                acc += w[p] * y;
            }
            out[(long)t * no + oi] = acc;
        }
    if (h_out)
        memcpy(h_out, h, sizeof(double) * P * dff);
    free(h);
    return 0;
}

/*
 * The zero-skip form of the down projection, for E2M1 neuron-major experts: neurons are taken in
 * groups of 16 and a group is read only when one of its 16 activations is nonzero.  Given h per
 * pair ([T*k][d_ff], as returned by oracle_experts_forward), writes out [T][d_model] and the
 * number of groups read per pair (active_groups [T*k]).
 */
int oracle_zero_skip_down(const double *h, int T, const int32_t *idx, const double *w, int k,
                          const oracle_experts *ex, double *out, int32_t *active_groups)
{
    if (ex->n_shared > 0) {                   /* h and active_groups: T * (k + n_shared) rows */
        int32_t *idx2; double *w2; int k2;
        if (with_shared(idx, w, T, k, ex, &idx2, &w2, &k2)) return -2;
        oracle_experts e2 = *ex;
        e2.E += e2.n_shared;
        e2.n_shared = 0;
        int rc = oracle_zero_skip_down(h, T, idx2, w2, k2, &e2, out, active_groups);
        free(idx2); free(w2);
        return rc;
    }
    int d = ex->d_model, dff = ex->d_ff, G = dff / 16;
    long P = (long)T * k;
    for (long p = 0; p < P; ++p) {
        int n = 0;
        for (int g = 0; g < G; ++g) {
            int any = 0;
            for (int f = 16 * g; f < 16 * g + 16; ++f)
                any |= h[p * dff + f] != 0.0;
            n += any;
        }
        active_groups[p] = n;
    }
#pragma omp parallel for collapse(2) schedule(static)
    for (int t = 0; t < T; ++t)
        for (int o = 0; o < d; ++o) {
            double acc = 0.0;
            for (int j = 0; j < k; ++j) {
                long p = (long)t * k + j;
                int e = idx[p];
                double y = 0.0;
                for (int g = 0; g < G; ++g) {
                    int any = 0;
                    for (int f = 16 * g; f < 16 * g + 16; ++f)
                        any |= h[p * dff + f] != 0.0;
                    if (!any)
                        continue;
                    for (int f = 16 * g; f < 16 * g + 16; ++f)
                        y += w_down(ex, e, o, f) * h[p * dff + f];
                }
                acc += w[p] * y;
            }
            out[(long)t * d + o] = acc;
        }
    return 0;
}

/* ------------------------------------------------------------------------------------------ */
/* int8-activation (batched prefill) variant                                                  */
/* ------------------------------------------------------------------------------------------ */

/*
 * Rule Q, in IEEE fp32: a = max |v|; a == 0 gives q = 0, s = 0; otherwise inv = fp32(127 / a),
 * q_i = clamp(round_half_even(fp32(v_i * inv)), -127, 127) and s = fp32(a / 127).
 */
void oracle_rule_q(const float *v, int n, int8_t *q, float *s)
{
    float a = 0.0f;
    for (int i = 0; i < n; ++i) {
        float m = fabsf(v[i]);
        if (m > a) a = m;
    }
    if (a == 0.0f) {
        for (int i = 0; i < n; ++i)
            q[i] = 0;
        *s = 0.0f;
        return;
    }
    volatile float inv = 127.0f / a;     /* volatile: keep each step a separate fp32 rounding */
    for (int i = 0; i < n; ++i) {
        volatile float prod = v[i] * inv;
        float r = rintf(prod);           /* default rounding mode: to nearest, ties to even */
        if (r > 127.0f) r = 127.0f;
        if (r < -127.0f) r = -127.0f;
        q[i] = (int8_t)r;
    }
    *s = a / 127.0f;
}

/*
 * The batched-prefill layer with int8 activations, SwiGLU, per-row int8 weights (I8_ROW):
 *   (xq, s_x) = rule Q of x[t] (x read as fp32);
 *   g_f = s_x * s_gu[f] * sum_i xq_i q_gu[f][i]  (integer sum exact in int64), u_f likewise;
 *   h_f = fp32(silu(g_f) * u_f);  (hq, s_h) = rule Q of the fp32 row h;
 *   y_o = s_h * s_down[o] * sum_f hq_f q_down[o][f];  out[t] = sum_j w_j y^(j) in slot order.
 * With Q8_0 weights each 32-wide block b of a weight row keeps its own fp16 scale, applied to
 * that block's exact integer sum, and the blocks add in K order:
 *   g_f = s_x * sum_b s_gu[f][b] * sum_{i in b} xq_i q_gu[f][i],  y_o likewise over f.
 * o_list / n_o / h_out as in oracle_experts_forward (h_out receives the fp32 h as doubles).
 * Optionally returns xq [T][d_model] and s_x [T].
 */

/* sum over the weight row of q_x * q_w with the row's scale(s): per-row fp32 or Q8_0 blocks */
static double i8_row_dot(const int8_t *xq, const int8_t *qw, int n, int q8, const void *scales, long row)
{
    if (!q8) {
        int64_t a = 0;
        for (int i = 0; i < n; ++i)
            a += (int64_t)xq[i] * qw[i];
        return (double)((const float *)scales)[row] * (double)a;
    }
    const uint16_t *s16 = (const uint16_t *)scales + row * (long)(n / 32);
    double acc = 0.0;
    for (int b = 0; b < n / 32; ++b) {
        int64_t a = 0;
        for (int i = 32 * b; i < 32 * b + 32; ++i)
            a += (int64_t)xq[i] * qw[i];
        acc += oracle_half_to_double(s16[b]) * (double)a;
    }
    return acc;
}
int oracle_experts_forward_i8act(const void *x, int xtype, int T, const int32_t *idx,
                                 const double *w, int k, const oracle_experts *ex,
                                 const int32_t *o_list, int n_o, double *out, double *h_out,
                                 int8_t *xq_out, float *sx_out)
{
    if (ex->n_shared > 0) {
        int32_t *idx2; double *w2; int k2;
        if (with_shared(idx, w, T, k, ex, &idx2, &w2, &k2)) return -2;
        oracle_experts e2 = *ex;
        e2.E += e2.n_shared;
        e2.n_shared = 0;
        int rc = oracle_experts_forward_i8act(x, xtype, T, idx2, w2, k2, &e2, o_list, n_o, out, h_out,
                                              xq_out, sx_out);
        free(idx2); free(w2);
        return rc;
    }
    if (ex->fmt != OW_I8_ROW && ex->fmt != OW_Q8_0)
        return -3;
    const int q8 = ex->fmt == OW_Q8_0;
    int d = ex->d_model, dff = ex->d_ff;
    int no = o_list ? n_o : d;
    long P = (long)T * k;
    int8_t *xq = (int8_t *)malloc((size_t)(T > 0 ? T : 1) * d);
    float *sx = (float *)malloc(sizeof(float) * (T > 0 ? T : 1));
    float *hrow = (float *)malloc(sizeof(float) * (P > 0 ? P : 1) * dff);
    int8_t *hq = (int8_t *)malloc((size_t)(P > 0 ? P : 1) * dff);
    float *sh = (float *)malloc(sizeof(float) * (P > 0 ? P : 1));
    if (!xq || !sx || !hrow || !hq || !sh) {
        free(xq); free(sx); free(hrow); free(hq); free(sh);
        return -2;
    }
    const int8_t *qgu = (const int8_t *)ex->gate_up, *qdn = (const int8_t *)ex->down;

#pragma omp parallel for schedule(static)
    for (int t = 0; t < T; ++t) {
        float *row = (float *)malloc(sizeof(float) * d);
        for (int i = 0; i < d; ++i)
            row[i] = (float)x_at(x, xtype, (long)t * d + i);   /* exact: x is fp32 or bf16 */
        oracle_rule_q(row, d, xq + (long)t * d, sx + t);
        free(row);
    }
    for (long p = 0; p < P; ++p)
        if (idx[p] < 0 || idx[p] >= ex->E) {
            free(xq); free(sx); free(hrow); free(hq); free(sh);
            return -1;
        }
#pragma omp parallel for schedule(dynamic, 1)
    for (long p = 0; p < P; ++p) {
        int t = (int)(p / k), e = idx[p];
        const int8_t *xr = xq + (long)t * d;
        for (int f = 0; f < dff; ++f) {
            long rg = (long)e * 2 * dff + f, ru = (long)e * 2 * dff + dff + f;
            double g = (double)sx[t] * i8_row_dot(xr, qgu + rg * d, d, q8, ex->gate_up_scales, rg);
            double u = (double)sx[t] * i8_row_dot(xr, qgu + ru * d, d, q8, ex->gate_up_scales, ru);
            hrow[p * dff + f] = (float)(silu(g) * u);
        }
        oracle_rule_q(hrow + p * dff, dff, hq + p * dff, sh + p);
    }
#pragma omp parallel for collapse(2) schedule(static)
    for (int t = 0; t < T; ++t)
        for (int oi = 0; oi < no; ++oi) {
            int o = o_list ? o_list[oi] : oi;
            double acc = 0.0;
            for (int j = 0; j < k; ++j) {
                long p = (long)t * k + j;
                long row = (long)idx[p] * d + o;
                double y = (double)sh[p] * i8_row_dot(hq + p * dff, qdn + row * dff, dff, q8, ex->down_scales, row);
                acc += w[p] * y;
            }
            out[(long)t * no + oi] = acc;
        }
    if (h_out)
        for (long i = 0; i < P * dff; ++i)
            h_out[i] = (double)hrow[i];
    if (xq_out)
        memcpy(xq_out, xq, (size_t)T * d);
    if (sx_out)
        memcpy(sx_out, sx, sizeof(float) * T);
    free(xq); free(sx); free(hrow); free(hq); free(sh);
    return 0;
}

/*
 * Rule Q8 (the fp8 counterpart of rule Q), in IEEE fp32: a = max |v|; a == 0 gives codes 0 and
 * s = 0; otherwise inv = fp32(448 / a), q_i = E4M3 code of fp32(v_i * inv) (nearest, ties to even)
 * and s = fp32(a / 448).
 */
void oracle_rule_q8(const float *v, int n, uint8_t *q, float *s)
{
    float a = 0.0f;
    for (int i = 0; i < n; ++i) {
        float m = fabsf(v[i]);
        if (m > a) a = m;
    }
    if (a == 0.0f) {
        for (int i = 0; i < n; ++i)
            q[i] = 0;
        *s = 0.0f;
        return;
    }
    volatile float inv = 448.0f / a;
    for (int i = 0; i < n; ++i) {
        volatile float prod = v[i] * inv;
        q[i] = (uint8_t)oracle_e4m3_encode(prod);
    }
    *s = a / 448.0f;
}

/*
 * The batched-prefill layer with fp8 activations and fp8 weights (FP8_ROW: E4M3 codes with one
 * fp32 scale per output row), SwiGLU: as the int8 variant with rule Q8 in place of rule Q,
 *   g_f = s_x * s_gu[f] * sum_i e4m3(xq_i) e4m3(q_gu[f][i])   (every product exact; fp64 sum),
 *   u_f likewise; h_f = fp32(silu(g_f) * u_f); (hq, s_h) = rule Q8 of the fp32 row h;
 *   y_o = s_h * s_down[o] * sum_f e4m3(hq_f) e4m3(q_down[o][f]);  out[t] = sum_j w_j y^(j).
 */
static double f8_row_dot(const uint8_t *a, const uint8_t *b, int n, double scale)
{
    double acc = 0.0;
    for (int i = 0; i < n; ++i)
        acc += oracle_e4m3_value(a[i]) * oracle_e4m3_value(b[i]);
    return scale * acc;
}

int oracle_experts_forward_f8act(const void *x, int xtype, int T, const int32_t *idx,
                                 const double *w, int k, const oracle_experts *ex,
                                 const int32_t *o_list, int n_o, double *out, double *h_out,
                                 uint8_t *xq_out, float *sx_out)
{
    if (ex->n_shared > 0) {
        int32_t *idx2; double *w2; int k2;
        if (with_shared(idx, w, T, k, ex, &idx2, &w2, &k2)) return -2;
        oracle_experts e2 = *ex;
        e2.E += e2.n_shared;
        e2.n_shared = 0;
        int rc = oracle_experts_forward_f8act(x, xtype, T, idx2, w2, k2, &e2, o_list, n_o, out, h_out,
                                              xq_out, sx_out);
        free(idx2); free(w2);
        return rc;
    }
    if (ex->fmt != OW_FP8_ROW)
        return -3;
    int d = ex->d_model, dff = ex->d_ff;
    int no = o_list ? n_o : d;
    long P = (long)T * k;
    uint8_t *xq = (uint8_t *)malloc((size_t)(T > 0 ? T : 1) * d);
    float *sx = (float *)malloc(sizeof(float) * (T > 0 ? T : 1));
    float *hrow = (float *)malloc(sizeof(float) * (P > 0 ? P : 1) * dff);
    uint8_t *hq = (uint8_t *)malloc((size_t)(P > 0 ? P : 1) * dff);
    float *sh = (float *)malloc(sizeof(float) * (P > 0 ? P : 1));
    if (!xq || !sx || !hrow || !hq || !sh) {
        free(xq); free(sx); free(hrow); free(hq); free(sh);
        return -2;
    }
    const uint8_t *qgu = (const uint8_t *)ex->gate_up, *qdn = (const uint8_t *)ex->down;
    const float *sgu = (const float *)ex->gate_up_scales, *sdn = (const float *)ex->down_scales;
#pragma omp parallel for schedule(static)
    for (int t = 0; t < T; ++t) {
        float *row = (float *)malloc(sizeof(float) * d);
        for (int i = 0; i < d; ++i)
            row[i] = (float)x_at(x, xtype, (long)t * d + i);
        oracle_rule_q8(row, d, xq + (long)t * d, sx + t);
        free(row);
    }
    for (long p = 0; p < P; ++p)
        if (idx[p] < 0 || idx[p] >= ex->E) {
            free(xq); free(sx); free(hrow); free(hq); free(sh);
            return -1;
        }
#pragma omp parallel for schedule(dynamic, 1)
    for (long p = 0; p < P; ++p) {
        int t = (int)(p / k), e = idx[p];
        const uint8_t *xr = xq + (long)t * d;
        for (int f = 0; f < dff; ++f) {
            long rg = (long)e * 2 * dff + f, ru = (long)e * 2 * dff + dff + f;
            double g = (double)sx[t] * f8_row_dot(xr, qgu + rg * d, d, (double)sgu[rg]);
            double u = (double)sx[t] * f8_row_dot(xr, qgu + ru * d, d, (double)sgu[ru]);
            hrow[p * dff + f] = (float)(silu(g) * u);
        }
        oracle_rule_q8(hrow + p * dff, dff, hq + p * dff, sh + p);
    }
#pragma omp parallel for collapse(2) schedule(static)
    for (int t = 0; t < T; ++t)
        for (int oi = 0; oi < no; ++oi) {
            int o = o_list ? o_list[oi] : oi;
            double acc = 0.0;
            for (int j = 0; j < k; ++j) {
                long p = (long)t * k + j;
                long row = (long)idx[p] * d + o;
                double y = (double)sh[p] * f8_row_dot(hq + p * dff, qdn + row * dff, dff, (double)sdn[row]);
                acc += w[p] * y;
            }
            out[(long)t * no + oi] = acc;
        }
    if (h_out)
        for (long i = 0; i < P * dff; ++i)
            h_out[i] = (double)hrow[i];
    if (xq_out)
        memcpy(xq_out, xq, (size_t)T * d);
    if (sx_out)
        memcpy(sx_out, sx, sizeof(float) * T);
    free(xq); free(sx); free(hrow); free(hq); free(sh);
    return 0;
}

void oracle_set_threads(int n)
{
#ifdef _OPENMP
    if (n > 0)
        omp_set_num_threads(n);
#else
    (void)n;
#endif
}

int oracle_get_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
