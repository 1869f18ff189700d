/*
 * fp64 CPU oracle for the activation-sparse MoE expert FFN.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the plain, slow definition of what
 * the GPU library computes.  Only the test-suite, the smoke check and the CPU
 * baseline leg of the benchmark load it.  It shares no code, header, table or
 * constant with the HIP library (activation_sparse_expert_amd/csrc) and
 * includes nothing from it.
 *
 * Sources (the pages are reviews of the papers; citations name page + section):
 *   [FloE-fwd]   FloE review, "三、技术架构 / MoE 专家前向计算": each SwiGLU
 *                expert computes a_E(x) = (SiLU(x W^gate) (.) x W^up) W^down.
 *   [FloE-comp]  FloE review, "混合压缩策略": gate and down are activation-
 *                sparsified, up is quantised to INT2; the compressed expert is
 *                {W^S(gate), W^S(down), W^Q(up)}.
 *   [FloE-intra] FloE review, "双稀疏预测器 / Intra-expert Predictor": the
 *                active channels are predicted, parameter-free, from the hidden
 *                state times the (re-used) up projection.
 *   [FloE-alg1]  FloE review, "系统协同优化 / 高效稀疏 GEMV 内核", Algorithm 1:
 *                v = x W^up; mask = |v| > t_ij; x' = SiLU(x W^gate[mask]) (.)
 *                v[mask]; output = x' W^down_T, with W^down stored transposed
 *                (column-major) so only the selected rows are loaded, and
 *                SiLU fused with the product.
 *   [MoEInf-A3]  MoE-Infinity review, "A3 背景": a router picks the top-k
 *                experts of each token (Mixtral: 8 experts, top-2).
 *   [MoEInf-4.3] MoE-Infinity review, "4.3": the iteration-level expert
 *                activation matrix counts the tokens routed to each expert.
 *   [MoEInf-4.5] MoE-Infinity review, "4.5": the collection of past request-
 *                level EAMs is searched for the one closest to the current
 *                EAM, both flattened, by cosine distance.
 *   [MoEL-arch]  MoE-Lightning review, "三、技术架构 / MoE 模型架构": a gating
 *                network selects the top-k expert FFNs of each token.
 *
 * Readings where the pages leave a step open (each is also listed with the
 * design notes of the library):
 *   R1  Algorithm 1's last line multiplies the selected values by the selected
 *       rows of W^down only: y = sum_{j in mask} x'_j W^down[j, :].
 *   R2  W^gate[mask] selects the columns j in mask of W^gate (d x f); stored
 *       f-major ("gate_t"), they are rows of gate_t.
 *   R3  W^down "transposed, column-major" is stored [f][d]: row j holds
 *       channel j's d outputs contiguously.
 *   R4  One scalar threshold per (layer, expert); strict comparison |v| > t.
 *       t < 0 keeps every channel (dense expert), t = +inf keeps none.
 *   R5  INT2 up: groups of 64 consecutive inputs k per output channel j,
 *       asymmetric, w = s * (q - z) with fp16 s and fp16 (fractional) z.  Row j
 *       is d/16 little-endian 32-bit words; word i holds the 16 codes of inputs
 *       16i..16i+15, the code of input 16i + 2m + h (m in 0..7, h in {0,1}) in
 *       bits 16h + 2m: even inputs in the low half-word, odd ones in the high.
 *   R6  The dequantised INT2 up weights feed both the mask and the product.
 *   R7  Router: logits = x R^T (+ bias); top-k by (-logit, index) so ties go to
 *       the lowest index; weights are the softmax over the k chosen logits when
 *       renormalising, else the full softmax evaluated at the chosen experts.
 *   R8  Layer: y_t = sum_s w_{t,s} a_{e(t,s)}(x_t) + sum_shared a_sh(x_t).
 *   R9  Dense grouped-GEMM path: the same layer at t < 0 with the up weights
 *       materialised once as bf16_rne(dequant(INT2)) next to bf16 gate/down.
 *   R21 EAM matching: the cosine distance of two flattened count vectors is
 *       1 - <a, b> / sqrt(|a|^2 |b|^2); it is 1 when either vector is zero (no
 *       direction).  Counts outside [0, 2^22) make a stored EAM unusable (NaN,
 *       never the match); a query with one matches nothing (index -1).  The
 *       smallest distance wins, the lowest index among equal ones.
 *   R22 Request-level EAM: after each iteration the iteration's per-layer
 *       counts are added into the request's matrix, row = layer.
 *   R23 Other up widths (8, 4, 1 bits): the INT2 group-64 min-max scheme with
 *       2^bits - 1 levels, codes packed plainly at bit k*bits of the row.
 *
 * Everything below is straight loops in double precision.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { ODT_F16 = 0, ODT_BF16 = 1, ODT_F32 = 2 };

/* ---------------------------------------------------------------- scalars */

/* IEEE binary16 bit pattern -> double (exact). */
double oracle_half_to_double(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1F;
    int m = h & 0x3FF;
    double v;
    if (e == 0)
        v = ldexp((double)m, -24);               /* subnormal: m * 2^-24 */
    else if (e == 31)
        v = m ? NAN : INFINITY;
    else
        v = ldexp((double)(m + 1024), e - 25);    /* (1 + m/1024) * 2^(e-15) */
    return sign ? -v : v;
}

/* bfloat16 bit pattern -> double (exact): bf16 is the top half of a float. */
double oracle_bf16_to_double(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

static double load_typed(const void *p, int dt, size_t i)
{
    if (dt == ODT_F16) return oracle_half_to_double(((const uint16_t *)p)[i]);
    if (dt == ODT_BF16) return oracle_bf16_to_double(((const uint16_t *)p)[i]);
    return (double)((const float *)p)[i];
}

/* Round a double to the nearest binary16 value, ties to even; returns bits.
 * Overflow saturates to infinity as IEEE rounding does. */
uint16_t oracle_double_to_half_rne(double v)
{
    uint16_t sign = 0;
    if (v != v) return 0x7E00;
    if (signbit(v)) { sign = 0x8000; v = -v; }
    if (v == 0.0) return sign;
    /* candidates are multiples of the spacing at v's binade */
    int e;
    frexp(v, &e);                  /* v = f * 2^e, f in [0.5, 1) */
    int ex = e - 1;                /* v in [2^ex, 2^(ex+1)) */
    if (ex < -14) ex = -14;        /* subnormal range shares spacing 2^-24 */
    double ulp = ldexp(1.0, ex - 10);
    double n = v / ulp;            /* exact: power-of-two scaling */
    double fl = floor(n);
    double r = n - fl;
    double q;
    if (r > 0.5) q = fl + 1;
    else if (r < 0.5) q = fl;
    else q = (fmod(fl, 2.0) == 0.0) ? fl : fl + 1;
    double rv = q * ulp;
    if (rv >= 65520.0) return sign | 0x7C00;   /* rounds past max finite */
    /* encode rv */
    if (rv < ldexp(1.0, -14)) {
        return sign | (uint16_t)(rv / ldexp(1.0, -24));
    }
    frexp(rv, &e);
    ex = e - 1;
    int mant = (int)(rv / ldexp(1.0, ex - 10)) - 1024;
    return sign | (uint16_t)(((ex + 15) << 10) | mant);
}

/* Round a double to the nearest bfloat16 value, ties to even; returns bits. */
uint16_t oracle_double_to_bf16_rne(double v)
{
    uint16_t sign = 0;
    if (v != v) return 0x7FC0;
    if (signbit(v)) { sign = 0x8000; v = -v; }
    if (v == 0.0) return sign;
    int e;
    frexp(v, &e);
    int ex = e - 1;
    if (ex < -126) ex = -126;
    double ulp = ldexp(1.0, ex - 7);
    double n = v / ulp;
    double fl = floor(n);
    double r = n - fl;
    double q;
    if (r > 0.5) q = fl + 1;
    else if (r < 0.5) q = fl;
    else q = (fmod(fl, 2.0) == 0.0) ? fl : fl + 1;
    double rv = q * ulp;
    /* largest finite bf16 is (2 - 2^-7) * 2^127; the next step would be 2^128 */
    if (rv >= ldexp(1.0, 128)) return sign | 0x7F80;
    float f = (float)rv;          /* exact: rv has <= 8 significant bits */
    uint32_t u;
    memcpy(&u, &f, 4);
    return sign | (uint16_t)(u >> 16);
}

/* ------------------------------------------------------ C0: INT2 up format */

/* Bit position of input k's code inside row j (reading R5): word k/16,
 * half-word k%2, pair slot (k%16)/2.  Words are little-endian. */
static size_t code_bit(size_t k)
{
    return 32 * (k / 16) + 16 * (k % 2) + 2 * ((k % 16) / 2);
}

static void put_code(uint8_t *up_q, int d, int j, size_t k, int q)
{
    size_t b = code_bit(k);
    uint8_t *byte = up_q + (size_t)j * (d / 4) + b / 8;
    *byte = (uint8_t)((*byte & ~(3u << (b % 8))) | ((unsigned)q << (b % 8)));
}

/*
 * Quantiser for the INT2 up projection ([FloE-comp], reading R5).  Input is
 * the fp32 up weights stored channel-major, w_t[j][k] = W^up[k][j], f x d.
 * Per channel j and group g of 64 inputs, in float32 arithmetic:
 *   mn, mx = min, max of the 64 weights
 *   s = fp16((mx - mn) / 3), replaced by 1 when it rounds to 0
 *   z = fp16(-mn / s)
 *   q = clamp(round_half_even(w / s + z), 0, 3)
 * Outputs: up_q [f][d/4] bytes holding the codes in the word order of R5,
 *          up_sz [f][d/64][2] fp16 bits {s, z}.
 * The float32 steps are written out one operation at a time; the compiler is
 * told not to contract or reassociate (built with -ffp-contract=off).
 */
void oracle_pack_up_int2(const float *w_t, int d, int f, uint8_t *up_q, uint16_t *up_sz)
{
    int G = d / 64;
    for (int j = 0; j < f; ++j) {
        for (int g = 0; g < G; ++g) {
            const float *w = w_t + (size_t)j * d + (size_t)g * 64;
            float mn = w[0], mx = w[0];
            for (int i = 1; i < 64; ++i) {
                if (w[i] < mn) mn = w[i];
                if (w[i] > mx) mx = w[i];
            }
            volatile float range = mx - mn;
            volatile float third = range / 3.0f;
            uint16_t sb = oracle_double_to_half_rne((double)third);
            float s = (float)oracle_half_to_double(sb);
            if (s == 0.0f) { sb = 0x3C00; s = 1.0f; }
            volatile float negmn = -mn;
            volatile float zq = negmn / s;
            uint16_t zb = oracle_double_to_half_rne((double)zq);
            float z = (float)oracle_half_to_double(zb);
            up_sz[((size_t)j * G + g) * 2 + 0] = sb;
            up_sz[((size_t)j * G + g) * 2 + 1] = zb;
            for (int i = 0; i < 64; ++i) {
                volatile float a = w[i] / s;
                volatile float b = a + z;
                float r = rintf(b);              /* default mode: ties to even */
                int q = (int)r;
                if (r < 0.0f) q = 0;
                if (r > 3.0f) q = 3;
                size_t k = (size_t)g * 64 + i;
                put_code(up_q, d, j, k, q);
            }
        }
    }
}

/* The INT2 code of input k of channel j. */
static int code_at(const uint8_t *up_q, int d, int j, int k)
{
    size_t b = code_bit((size_t)k);
    return (up_q[(size_t)j * (d / 4) + b / 8] >> (b % 8)) & 3;
}

/* Dequantised up weight w'_{k,j} = s_{g,j} * (q_{k,j} - z_{g,j}) (exact in double). */
static double up_weight(const uint8_t *up_q, const uint16_t *up_sz, int d, int j, int k)
{
    int G = d / 64;
    int g = k / 64;
    double s = oracle_half_to_double(up_sz[((size_t)j * G + g) * 2 + 0]);
    double z = oracle_half_to_double(up_sz[((size_t)j * G + g) * 2 + 1]);
    return s * ((double)code_at(up_q, d, j, k) - z);
}

/*
 * Other up widths (FloE review, "三、技术架构 / 敏感度分析": the up projection
 * is also quantised to 8, 4 and 1 bits; reading R23).  The same per-channel,
 * per-64-input-group asymmetric min-max scheme as the INT2 format with
 * L = 2^bits - 1 levels: s = fp16((mx - mn) / L) (1 when 0), z = fp16(-mn / s),
 * q = clamp(round_half_even(w / s + z), 0, L).  Codes are packed plainly:
 * input k of channel j sits at bit k*bits of row j (rows of d*bits/8 bytes,
 * least significant bits first within a byte).
 */
static int code_at_bits(const uint8_t *up_q, int d, int bits, int j, int k)
{
    size_t bit = (size_t)k * bits;
    const uint8_t *row = up_q + (size_t)j * ((size_t)d * bits / 8);
    return (row[bit / 8] >> (bit % 8)) & ((1 << bits) - 1);
}

void oracle_pack_up_bits(const float *w_t, int d, int f, int bits, uint8_t *up_q, uint16_t *up_sz)
{
    if (bits == 2) { oracle_pack_up_int2(w_t, d, f, up_q, up_sz); return; }
    const int G = d / 64, L = (1 << bits) - 1;
    const size_t rb = (size_t)d * bits / 8;
    memset(up_q, 0, rb * (size_t)f);
    for (int j = 0; j < f; ++j) {
        for (int g = 0; g < G; ++g) {
            const float *w = w_t + (size_t)j * d + (size_t)g * 64;
            float mn = w[0], mx = w[0];
            for (int i = 1; i < 64; ++i) {
                if (w[i] < mn) mn = w[i];
                if (w[i] > mx) mx = w[i];
            }
            volatile float range = mx - mn;
            volatile float step = range / (float)L;
            uint16_t sb = oracle_double_to_half_rne((double)step);
            float s = (float)oracle_half_to_double(sb);
            if (s == 0.0f) { sb = 0x3C00; s = 1.0f; }
            volatile float negmn = -mn;
            volatile float zq = negmn / s;
            uint16_t zb = oracle_double_to_half_rne((double)zq);
            float z = (float)oracle_half_to_double(zb);
            up_sz[((size_t)j * G + g) * 2 + 0] = sb;
            up_sz[((size_t)j * G + g) * 2 + 1] = zb;
            for (int i = 0; i < 64; ++i) {
                volatile float a = w[i] / s;
                volatile float b = a + z;
                float r = rintf(b);
                int q = (int)r;
                if (r < 0.0f) q = 0;
                if (r > (float)L) q = L;
                size_t bit = ((size_t)g * 64 + i) * bits;
                up_q[(size_t)j * rb + bit / 8] |= (uint8_t)(q << (bit % 8));
            }
        }
    }
}

/* w'_{k,j} = s (q - z) for any supported width (exact in double). */
static double up_weight_bits(const uint8_t *up_q, const uint16_t *up_sz, int d, int bits,
                             int j, int k)
{
    if (bits == 2) return up_weight(up_q, up_sz, d, j, k);
    int G = d / 64;
    int g = k / 64;
    double s = oracle_half_to_double(up_sz[((size_t)j * G + g) * 2 + 0]);
    double z = oracle_half_to_double(up_sz[((size_t)j * G + g) * 2 + 1]);
    return s * ((double)code_at_bits(up_q, d, bits, j, k) - z);
}

void oracle_dequant_up_bits(const uint8_t *up_q, const uint16_t *up_sz, int d, int f, int bits,
                            double *out)
{
    for (int j = 0; j < f; ++j)
        for (int k = 0; k < d; ++k)
            out[(size_t)j * d + k] = up_weight_bits(up_q, up_sz, d, bits, j, k);
}

/* Full dequantisation into double, out[j][k] = w'_{k,j}. */
void oracle_dequant_up(const uint8_t *up_q, const uint16_t *up_sz, int d, int f, double *out)
{
    for (int j = 0; j < f; ++j)
        for (int k = 0; k < d; ++k)
            out[(size_t)j * d + k] = up_weight(up_q, up_sz, d, j, k);
}

/* Up weights for the dense path (reading R9): bf16_rne of the exact dequantised
 * value, out[j][k] as bf16 bits. */
void oracle_materialize_up_bf16(const uint8_t *up_q, const uint16_t *up_sz, int d, int f,
                                uint16_t *out)
{
    for (int j = 0; j < f; ++j)
        for (int k = 0; k < d; ++k)
            out[(size_t)j * d + k] = oracle_double_to_bf16_rne(up_weight(up_q, up_sz, d, j, k));
}

/* The same for fp16 layers (reading R9 in the layer's own 16-bit type):
 * fp16_rne of the exact dequantised value, out[j][k] as fp16 bits. */
void oracle_materialize_up_f16(const uint8_t *up_q, const uint16_t *up_sz, int d, int f,
                               uint16_t *out)
{
    for (int j = 0; j < f; ++j)
        for (int k = 0; k < d; ++k)
            out[(size_t)j * d + k] = oracle_double_to_half_rne(up_weight(up_q, up_sz, d, j, k));
}

/* ------------------------------------------------------ C1: one expert */

static double silu(double g) { return g / (1.0 + exp(-g)); }

/*
 * One compressed expert on T tokens ([FloE-fwd], [FloE-alg1], [FloE-intra]).
 * Per token t, independently:
 *   1. v_j = sum_k x_k w'_{k,j}                 (Algorithm 1, step 1)
 *   2. mask_j = |v_j| > t   (or the fed mask)   (step 2)
 *   3. for j in mask: g_j = sum_k x_k W^gate[k][j];
 *      h_j = SiLU(g_j) * v_j                    (step 3, SiLU fused with (.))
 *   4. y_c = scale_t * sum_{j in mask} h_j W^down[j][c]      (step 4, R1)
 * Inputs: x [T][d] in xdt; gate_t, down [f][d] in wdt; up_q/up_sz per C0;
 *         thr is the float32 threshold; scale [T] or NULL (=1);
 *         mask_in [T][f] u8 or NULL (NULL: compute the mask from v).
 * Outputs (all optional): v_out [T][f], mask_out [T][f], y_out [T][d]
 *         (y_out is accumulated into when accumulate != 0).
 */
void oracle_expert_forward_bits(int bits, const void *x, int xdt, int T, int d, int f,
                                const uint8_t *up_q, const uint16_t *up_sz,
                                const void *gate_t, const void *down, int wdt,
                                float thr, const double *scale, const uint8_t *mask_in,
                                double *v_out, uint8_t *mask_out, double *y_out, int accumulate)
{
    double *xr = (double *)malloc(sizeof(double) * (size_t)T * d);
    double *yr = (double *)calloc((size_t)T * d, sizeof(double));
    double *wu = (double *)malloc(sizeof(double) * (size_t)d);
    double *wg = (double *)malloc(sizeof(double) * (size_t)d);
    double *wd = (double *)malloc(sizeof(double) * (size_t)d);
    for (size_t i = 0; i < (size_t)T * d; ++i) xr[i] = load_typed(x, xdt, i);
    /* channel by channel; each token's arithmetic is independent of the others */
    for (int j = 0; j < f; ++j) {
        for (int k = 0; k < d; ++k) {
            wu[k] = up_weight_bits(up_q, up_sz, d, bits, j, k);
            wg[k] = load_typed(gate_t, wdt, (size_t)j * d + k);
            wd[k] = load_typed(down, wdt, (size_t)j * d + k);
        }
        for (int t = 0; t < T; ++t) {
            const double *xt = xr + (size_t)t * d;
            double v = 0.0;
            for (int k = 0; k < d; ++k) v += xt[k] * wu[k];                     /* step 1 */
            int m = mask_in ? (mask_in[(size_t)t * f + j] != 0) : (fabs(v) > (double)thr); /* 2 */
            if (v_out) v_out[(size_t)t * f + j] = v;
            if (mask_out) mask_out[(size_t)t * f + j] = (uint8_t)m;
            if (!m) continue;
            double g = 0.0;
            for (int k = 0; k < d; ++k) g += xt[k] * wg[k];
            double h = silu(g) * v;                                             /* step 3 */
            double *yt = yr + (size_t)t * d;
            for (int c = 0; c < d; ++c) yt[c] += h * wd[c];                     /* step 4 */
        }
    }
    for (int t = 0; t < T; ++t) {
        double sc = scale ? scale[t] : 1.0;
        if (y_out)
            for (int c = 0; c < d; ++c) {
                double o = sc * yr[(size_t)t * d + c];
                y_out[(size_t)t * d + c] = accumulate ? y_out[(size_t)t * d + c] + o : o;
            }
    }
    free(xr); free(yr); free(wu); free(wg); free(wd);
}

/* The INT2 expert (C0 format). */
void oracle_expert_forward(const void *x, int xdt, int T, int d, int f,
                           const uint8_t *up_q, const uint16_t *up_sz,
                           const void *gate_t, const void *down, int wdt,
                           float thr, const double *scale, const uint8_t *mask_in,
                           double *v_out, uint8_t *mask_out, double *y_out, int accumulate)
{
    oracle_expert_forward_bits(2, x, xdt, T, d, f, up_q, up_sz, gate_t, down, wdt, thr, scale,
                               mask_in, v_out, mask_out, y_out, accumulate);
}

/* ------------------------------------------------------ C2: router */

/*
 * Top-k router ([MoEInf-A3], [MoEL-arch], reading R7) and the grouping of the
 * T*k (token, slot) pairs by expert ([MoEInf-4.3]: expert_count is one row of
 * the iteration-level expert activation matrix).
 *   logits[t][e] = sum_k x[t][k] R[e][k] + bias[e]
 *   topk_idx[t][s], s = 0..k-1: experts by decreasing logit, ties to the lower
 *   index.  topk_w: softmax over the chosen logits (renormalize != 0) or the
 *   full softmax at the chosen experts.
 *   expert_count[e], expert_offset[e] (exclusive prefix, offset[E] = T*k),
 *   pair_by_expert[offset[e] + i] = the i-th pair p = t*k + s (ascending p)
 *   routed to e.
 */
void oracle_route_topk(const void *x, int xdt, int T, int d, const void *router_w, int rdt,
                       const float *bias, int E, int k, int renormalize,
                       int32_t *topk_idx, double *topk_w, double *logits_out,
                       int32_t *expert_count, int32_t *expert_offset, int32_t *pair_by_expert)
{
    double *l = (double *)malloc(sizeof(double) * (size_t)E);
    char *taken = (char *)malloc((size_t)E);
    for (int t = 0; t < T; ++t) {
        for (int e = 0; e < E; ++e) {
            double a = 0.0;
            for (int i = 0; i < d; ++i)
                a += load_typed(x, xdt, (size_t)t * d + i) * load_typed(router_w, rdt, (size_t)e * d + i);
            if (bias) a += (double)bias[e];
            l[e] = a;
            if (logits_out) logits_out[(size_t)t * E + e] = a;
        }
        memset(taken, 0, (size_t)E);
        for (int s = 0; s < k; ++s) {
            int best = -1;
            for (int e = 0; e < E; ++e) {
                if (taken[e]) continue;
                if (best < 0 || l[e] > l[best]) best = e;   /* strict: keeps the lower index on ties */
            }
            taken[best] = 1;
            topk_idx[(size_t)t * k + s] = best;
        }
        double m = -INFINITY;
        if (renormalize) {
            for (int s = 0; s < k; ++s) {
                double a = l[topk_idx[(size_t)t * k + s]];
                if (a > m) m = a;
            }
            double den = 0.0;
            for (int s = 0; s < k; ++s) den += exp(l[topk_idx[(size_t)t * k + s]] - m);
            for (int s = 0; s < k; ++s)
                topk_w[(size_t)t * k + s] = exp(l[topk_idx[(size_t)t * k + s]] - m) / den;
        } else {
            for (int e = 0; e < E; ++e) if (l[e] > m) m = l[e];
            double den = 0.0;
            for (int e = 0; e < E; ++e) den += exp(l[e] - m);
            for (int s = 0; s < k; ++s)
                topk_w[(size_t)t * k + s] = exp(l[topk_idx[(size_t)t * k + s]] - m) / den;
        }
    }
    if (expert_count) {
        for (int e = 0; e < E; ++e) expert_count[e] = 0;
        for (int p = 0; p < T * k; ++p) expert_count[topk_idx[p]]++;
    }
    if (expert_offset) {
        int run = 0;
        for (int e = 0; e < E; ++e) {
            expert_offset[e] = run;
            int c = 0;
            for (int p = 0; p < T * k; ++p) c += (topk_idx[p] == e);
            run += c;
        }
        expert_offset[E] = run;
    }
    if (pair_by_expert) {
        int n = 0;
        for (int e = 0; e < E; ++e)
            for (int p = 0; p < T * k; ++p)
                if (topk_idx[p] == e) pair_by_expert[n++] = p;
    }
    free(l);
    free(taken);
}

/* ------------------------------------------------------ C3/C4: layer */

/*
 * One MoE layer (reading R8): E routed experts (top-k) then S shared experts,
 * all with the same compressed format, stored at a fixed stride per expert.
 *   up_q   [E+S][f][d/4], up_sz [E+S][f][d/64][2], gate_t/down [E+S][f][d]
 *   thr    [E+S] float32 thresholds
 * topk_in [T][k] (optional): use these experts instead of the oracle's own
 *   choice (their weights still come from the oracle's logits).
 * masks_in [T][k+S][f] (optional): fed masks, slot s < k for the routed
 *   choice s of token t, slot k+i for shared expert i.
 * dense != 0 selects the dense grouped-GEMM path (reading R9): every channel
 *   active and the up weights taken as rne(dequant(INT2)) in the layer's 16-bit
 *   type (bf16 for bf16 layers, fp16 for fp16 layers); gate/down are read in
 *   wdt as for the sparse path.
 * dense_experts [E+S] (optional): the dense path for the experts flagged 1 and
 *   Algorithm 1 for the others, within one layer (a per-expert choice of path,
 *   MoE-Lightning review, "层次化屋顶模型"; both compute the same expert, the
 *   dense one with every channel active).
 * Outputs: y [T][d]; optionally topk_idx/topk_w [T][k], masks_out [T][k+S][f].
 */
void oracle_layer_forward(const void *x, int xdt, int T, int d, int f,
                          const void *router_w, int rdt, const float *bias,
                          int E, int k, int S, int renormalize,
                          const uint8_t *up_q, const uint16_t *up_sz,
                          const void *gate_t, const void *down, int wdt,
                          const float *thr, int dense, const uint8_t *dense_experts,
                          const int32_t *topk_in, const uint8_t *masks_in,
                          double *y, int32_t *topk_idx_out, double *topk_w_out,
                          uint8_t *masks_out)
{
    int32_t *idx = (int32_t *)malloc(sizeof(int32_t) * (size_t)T * k);
    double *w = (double *)malloc(sizeof(double) * (size_t)T * k);
    double *l = (double *)malloc(sizeof(double) * (size_t)T * E);
    oracle_route_topk(x, xdt, T, d, router_w, rdt, bias, E, k, renormalize, idx, w, l,
                      NULL, NULL, NULL);
    if (topk_in) {
        /* fed choice: weights from the oracle's logits at the fed experts */
        for (int t = 0; t < T; ++t) {
            double m = -INFINITY, den = 0.0;
            if (renormalize) {
                for (int s = 0; s < k; ++s) {
                    double a = l[(size_t)t * E + topk_in[(size_t)t * k + s]];
                    if (a > m) m = a;
                }
                for (int s = 0; s < k; ++s) den += exp(l[(size_t)t * E + topk_in[(size_t)t * k + s]] - m);
            } else {
                for (int e = 0; e < E; ++e) if (l[(size_t)t * E + e] > m) m = l[(size_t)t * E + e];
                for (int e = 0; e < E; ++e) den += exp(l[(size_t)t * E + e] - m);
            }
            for (int s = 0; s < k; ++s) {
                idx[(size_t)t * k + s] = topk_in[(size_t)t * k + s];
                w[(size_t)t * k + s] = exp(l[(size_t)t * E + topk_in[(size_t)t * k + s]] - m) / den;
            }
        }
    }
    if (topk_idx_out) memcpy(topk_idx_out, idx, sizeof(int32_t) * (size_t)T * k);
    if (topk_w_out) memcpy(topk_w_out, w, sizeof(double) * (size_t)T * k);

    size_t qstride = (size_t)f * (d / 4), szstride = (size_t)f * (d / 64) * 2, wstride = (size_t)f * d;
    size_t wbytes = (wdt == ODT_F32) ? 4 : 2;
    uint8_t *mbuf = (uint8_t *)malloc((size_t)f);
    uint16_t *ubf = NULL;
    int ubf_expert = -1;
    double *ytok = (double *)malloc(sizeof(double) * (size_t)d);

    for (size_t i = 0; i < (size_t)T * d; ++i) y[i] = 0.0;
    for (int t = 0; t < T; ++t) {
        for (int slot = 0; slot < k + S; ++slot) {
            int e = slot < k ? idx[(size_t)t * k + slot] : E + (slot - k);
            double sc = slot < k ? w[(size_t)t * k + slot] : 1.0;
            const uint8_t *mi = masks_in ? masks_in + ((size_t)t * (k + S) + slot) * f : NULL;
            uint8_t *mo = masks_out ? masks_out + ((size_t)t * (k + S) + slot) * f : mbuf;
            const char *gt = (const char *)gate_t + (size_t)e * wstride * wbytes;
            const char *dn = (const char *)down + (size_t)e * wstride * wbytes;
            const uint8_t *uq = up_q + (size_t)e * qstride;
            const uint16_t *us = up_sz + (size_t)e * szstride;
            const void *xt = (const char *)x + (size_t)t * d * (xdt == ODT_F32 ? 4 : 2);
            if (!(dense || (dense_experts && dense_experts[e]))) {
                oracle_expert_forward(xt, xdt, 1, d, f, uq, us, gt, dn, wdt, thr[e], &sc, mi,
                                      NULL, mo, ytok, 0);
            } else {
                /* dense SwiGLU on rne(dequant(up)) in wdt, all channels active */
                if (!ubf) ubf = (uint16_t *)malloc(sizeof(uint16_t) * wstride);
                if (ubf_expert != e) {
                    if (wdt == ODT_F16) oracle_materialize_up_f16(uq, us, d, f, ubf);
                    else oracle_materialize_up_bf16(uq, us, d, f, ubf);
                    ubf_expert = e;
                }
                double *xr = (double *)malloc(sizeof(double) * (size_t)d);
                for (int q = 0; q < d; ++q) xr[q] = load_typed(xt, xdt, (size_t)q);
                for (int c = 0; c < d; ++c) ytok[c] = 0.0;
                for (int j = 0; j < f; ++j) {
                    double v = 0.0, g = 0.0;
                    for (int q = 0; q < d; ++q) {
                        v += xr[q] * (wdt == ODT_F16 ? oracle_half_to_double(ubf[(size_t)j * d + q])
                                                     : oracle_bf16_to_double(ubf[(size_t)j * d + q]));
                        g += xr[q] * load_typed(gt, wdt, (size_t)j * d + q);
                    }
                    double h = silu(g) * v;
                    for (int c = 0; c < d; ++c) ytok[c] += h * load_typed(dn, wdt, (size_t)j * d + c);
                    mo[j] = 1;
                }
                for (int c = 0; c < d; ++c) ytok[c] *= sc;
                free(xr);
            }
            for (int c = 0; c < d; ++c) y[(size_t)t * d + c] += ytok[c];
        }
    }
    free(idx); free(w); free(l); free(mbuf); free(ytok); free(ubf);
}

/* ------------------------------------------------------ EAM / EAMC */

/*
 * [MoEInf-4.3], reading R22: ream [L][E] += this iteration's counts of layer
 * `layer` (count [E], e.g. the expert_count of oracle_route_topk).
 */
void oracle_ream_add(int32_t *ream, int E, int layer, const int32_t *count)
{
    for (int e = 0; e < E; ++e) ream[(size_t)layer * E + e] += count[e];
}

/*
 * [MoEInf-4.5], reading R21: dist[i] = cosine distance between query [len]
 * and stored EAM i (eamc [n][len]); returns the index of the smallest.
 * The dot product and squared norms are integer sums (exact: entries are
 * below 2^22 and len is small), the rest is double precision.
 */
int oracle_eamc_match(const int32_t *eamc, int n, int len, const int32_t *query, double *dist)
{
    const long long lim = 1ll << 22;
    int query_ok = 1;
    for (int c = 0; c < len; ++c)
        if (query[c] < 0 || query[c] >= lim) query_ok = 0;
    int best = -1;
    for (int i = 0; i < n; ++i) {
        const int32_t *b = eamc + (size_t)i * len;
        int ok = query_ok;
        long long ab = 0, aa = 0, bb = 0;
        for (int c = 0; c < len; ++c) {
            if (b[c] < 0 || b[c] >= lim) ok = 0;
            ab += (long long)query[c] * b[c];
            aa += (long long)query[c] * query[c];
            bb += (long long)b[c] * b[c];
        }
        if (!ok) dist[i] = NAN;
        else if (aa == 0 || bb == 0) dist[i] = 1.0;
        else dist[i] = 1.0 - (double)ab / sqrt((double)aa * (double)bb);
        if (ok && (best < 0 || dist[i] < dist[best])) best = i;   /* strict: lowest index on ties */
    }
    return best;
}
