/*
 * moe_oracle.c -- plain CPU reference of the fused Mixture-of-Experts layer forward.
 *
 * TEST INFRASTRUCTURE ONLY (see moe_oracle.h): used by the tests, the smoke check and
 * the CPU-baseline leg of the benchmark, never by the product path.
 *
 * The layer computes, per token t with hidden vector x_t:
 *     out[t] = sum over slots j of  w_{t,j} * FFN_{e_{t,j}}(x_t),
 *     FFN_e(x) = W2_e ( SiLU(W1_e x) * (W3_e x) ),   SiLU(z) = z / (1 + exp(-z)),
 * where (e_{t,j}, w_{t,j}) are the router's top-k choice for the token.  This is what the
 * pages' pipelines (fused gate -> permute -> grouped GEMMs -> unpermute and reduce, in
 * the last review comment of SGLang PR #3191 "Add deepseek_v3 fused gate") compute; the
 * permutation and padding are an implementation device and do not change the result, so
 * the oracle applies the definition directly, one token and one expert at a time.
 *
 * Build: gcc -O2 -std=c11 -pthread -fPIC -shared moe_oracle.c -lm  (no GPU headers).
 */
#include "moe_oracle.h"

#include <math.h>
#include <pthread.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------------------ */
/* number codecs                                                                         */
/* ------------------------------------------------------------------------------------ */

static uint32_t f32_bits(float x) { uint32_t u; memcpy(&u, &x, 4); return u; }
static float bits_f32(uint32_t u) { float x; memcpy(&x, &u, 4); return x; }

float orc_bf16_to_f32(uint16_t bits) { return bits_f32((uint32_t)bits << 16); }

/* bf16 keeps the upper 16 bits of the fp32 pattern; the dropped 16 bits decide rounding:
 * above half -> up, below half -> down, exactly half -> toward an even kept pattern. */
uint16_t orc_f32_to_bf16(float x)
{
    uint32_t u = f32_bits(x);
    if (isnan(x)) return (uint16_t)((u >> 16) | 0x0040u);   /* quiet NaN, same sign */
    uint32_t kept = u >> 16, dropped = u & 0xFFFFu;
    if (dropped > 0x8000u || (dropped == 0x8000u && (kept & 1u))) kept += 1u;
    return (uint16_t)kept;
}

/* IEEE binary16: 1 sign, 5 exponent (bias 15), 10 mantissa bits. */
float orc_f16_to_f32(uint16_t bits)
{
    int sign = (bits >> 15) & 1, ex = (bits >> 10) & 0x1F, man = bits & 0x3FF;
    double v;
    if (ex == 0) v = ldexp((double)man, -24);                       /* zero / subnormal */
    else if (ex == 31) v = man ? NAN : INFINITY;
    else v = ldexp(1.0 + man / 1024.0, ex - 15);
    return (float)(sign ? -v : v);
}

/* OCP 8-bit E4M3 ("FN"): 1 sign, 4 exponent (bias 7), 3 mantissa bits; no infinities;
 * exponent 1111 with mantissa 111 is NaN; largest finite magnitude 1.75 * 2^8 = 448. */
float orc_e4m3_to_f32(uint8_t code)
{
    int sign = code >> 7, ex = (code >> 3) & 0xF, man = code & 7;
    double v;
    if (ex == 15 && man == 7) return NAN;
    if (ex == 0) v = ldexp((double)man, -9);                        /* (man/8) * 2^(1-7) */
    else v = ldexp(1.0 + man / 8.0, ex - 7);
    return (float)(sign ? -v : v);
}

/* Round to the nearest E4M3 value, ties to the even code, saturating at +-448.
 * Codes 0x00..0x7E enumerate the non-negative finite values in increasing order. */
uint8_t orc_f32_to_e4m3(float x)
{
    if (isnan(x)) return 0x7F;
    uint8_t sign = signbit(x) ? 0x80 : 0x00;
    double a = fabs((double)x);
    if (a >= 448.0) return sign | 0x7E;
    int lo = 0;
    while (lo + 1 <= 0x7E && (double)orc_e4m3_to_f32((uint8_t)(lo + 1)) <= a) lo++;
    double vlo = orc_e4m3_to_f32((uint8_t)lo);
    if (vlo == a) return sign | (uint8_t)lo;
    int hi = lo + 1;                                                /* a < 448: hi <= 0x7E */
    double vhi = orc_e4m3_to_f32((uint8_t)hi);
    double dlo = a - vlo, dhi = vhi - a;                            /* exact in fp64 */
    int pick = dlo < dhi ? lo : dhi < dlo ? hi : ((lo & 1) ? hi : lo);
    return sign | (uint8_t)pick;
}

/* The logistic function evaluated in fp64 and rounded once to fp32.  Pinning the
 * evaluation precision matters because a bias added to the sigmoid makes the selection
 * key depend on its last bit. */
float orc_sigmoid(float x) { return (float)(1.0 / (1.0 + exp(-(double)x))); }

/* ------------------------------------------------------------------------------------ */
/* routing                                                                               */
/* ------------------------------------------------------------------------------------ */

/* Expert a ranks before expert b: larger key first, equal keys -> lower index first.
 * The fused-gate review (SGLang PR #3191) asks for an output order that does not vary
 * between runs; ranking by (key, index) gives exactly one order. */
static int ranks_before(float ka, int a, float kb, int b) { return ka > kb || (ka == kb && a < b); }

/* Pick the k best experts among those with allowed[e] != 0, in rank order. */
static void select_topk(const float *key, const int *allowed, int E, int k, int32_t *out)
{
    int taken[256] = {0};
    for (int j = 0; j < k; j++) {
        int best = -1;
        for (int e = 0; e < E; e++) {
            if (!allowed[e] || taken[e]) continue;
            if (best < 0 || ranks_before(key[e], e, key[best], best)) best = e;
        }
        out[j] = best;
        taken[best] = 1;
    }
}

/*
 * Router top-k for one batch of tokens.
 *  SOFTMAX: p = softmax(logits) (fp64); the k experts with the largest logits (softmax is
 *    monotone, so this is the top-k of p, decided exactly); w_j = p_{e_j}, or with
 *    renormalisation p_{e_j} / sum_sel p.
 *  SIGMOID: s_e = sigmoid(logit_e); key_e = s_e (+ bias_e in fp32 when a bias is given);
 *    w_j = s_{e_j}, or renormalised over the selection.
 *  GROUPED_SIGMOID_BIAS (the DeepSeek-V3 "biased grouped top-k" gate of SGLang PR #3191):
 *    s_e = sigmoid(logit_e); key_e = s_e + bias_e (fp32); the E experts form n_group
 *    groups of E/n_group consecutive experts; a group's score is the fp32 sum of its two
 *    largest keys (its largest key when a group has one expert); the topk_group best
 *    groups by (score, lower group index) are kept; the k best experts by key among
 *    them are chosen; w_j = s_{e_j} / sum_sel s (renormalised) or s_{e_j}.  The bias
 *    steers the choice only and never enters a weight.
 * Every mode finally multiplies the weights by routed_scaling.  Weights are formed in
 * fp64 and rounded once to fp32.
 */
int orc_route(int kind, int E, int k, int renormalize, int n_group, int topk_group,
              float routed_scaling, int logits_dtype, const void *logits, const float *bias,
              int T, int32_t *ids, float *weights)
{
    if (E < 1 || E > 256 || k < 1 || k > E || T < 0) return -1;
    if (logits_dtype != ORC_BF16 && logits_dtype != ORC_FP32) return -1;
    if (kind == ORC_ROUTE_GROUPED_SIGMOID_BIAS) {
        if (n_group < 1 || E % n_group || topk_group < 1 || topk_group > n_group) return -1;
        if (k > topk_group * (E / n_group)) return -1;
    } else if (kind != ORC_ROUTE_SOFTMAX && kind != ORC_ROUTE_SIGMOID) {
        return -1;
    }
    float x[256], s[256], key[256];
    int allowed[256];
    for (int t = 0; t < T; t++) {
        for (int e = 0; e < E; e++) {
            x[e] = logits_dtype == ORC_BF16 ? orc_bf16_to_f32(((const uint16_t *)logits)[(int64_t)t * E + e])
                                            : ((const float *)logits)[(int64_t)t * E + e];
            allowed[e] = 1;
        }
        int32_t *sel = ids + (int64_t)t * k;
        double val[256];                    /* the unnormalised weight of each expert */
        if (kind == ORC_ROUTE_SOFTMAX) {
            for (int e = 0; e < E; e++) key[e] = x[e];
            select_topk(key, allowed, E, k, sel);
            double m = x[0];
            for (int e = 1; e < E; e++) if (x[e] > m) m = x[e];
            double z = 0.0;
            for (int e = 0; e < E; e++) z += exp((double)x[e] - m);
            for (int e = 0; e < E; e++) val[e] = exp((double)x[e] - m) / z;
        } else {
            for (int e = 0; e < E; e++) {
                s[e] = orc_sigmoid(x[e]);
                key[e] = bias ? s[e] + bias[e] : s[e];
                val[e] = s[e];
            }
            if (kind == ORC_ROUTE_GROUPED_SIGMOID_BIAS) {
                int G = E / n_group;
                float score[256];
                int32_t gsel[256];
                int gall[256];
                for (int g = 0; g < n_group; g++) {
                    int32_t top[2];
                    int in_group[256] = {0};
                    for (int e = g * G; e < (g + 1) * G; e++) in_group[e] = 1;
                    int take = G < 2 ? G : 2;
                    select_topk(key, in_group, E, take, top);
                    score[g] = take == 2 ? key[top[0]] + key[top[1]] : key[top[0]];
                    gall[g] = 1;
                }
                select_topk(score, gall, n_group, topk_group, gsel);
                for (int e = 0; e < E; e++) allowed[e] = 0;
                for (int q = 0; q < topk_group; q++)
                    for (int e = gsel[q] * G; e < (gsel[q] + 1) * G; e++) allowed[e] = 1;
            }
            select_topk(key, allowed, E, k, sel);
        }
        double norm = 0.0;
        for (int j = 0; j < k; j++) norm += val[sel[j]];
        for (int j = 0; j < k; j++) {
            double w = renormalize ? val[sel[j]] / norm : val[sel[j]];
            weights[(int64_t)t * k + j] = (float)(w * (double)routed_scaling);
        }
    }
    return 0;
}

/* ------------------------------------------------------------------------------------ */
/* align / permute                                                                       */
/* ------------------------------------------------------------------------------------ */

/* Most rows the padded layout can need: every routed pair, plus up to BM-1 filler rows
 * for each expert that receives at least one pair; rounded up to a whole block. */
int64_t orc_align_capacity(int T, int k, int E, int BM)
{
    int64_t pairs = (int64_t)T * k;
    int64_t used = pairs < E ? pairs : E;
    int64_t cap = pairs + used * (BM - 1);
    return (cap + BM - 1) / BM * BM;
}

/*
 * The moe_align_block_size step named in vLLM PR #12185 (note 1): group the T*k
 * (token, slot) pairs by expert so that each expert's rows form whole blocks of BM rows
 * for the grouped GEMM.  Reading taken (the page gives only the name):
 *  - pair (t, j) has flat index t*k + j; within an expert, pairs keep ascending flat
 *    index (a stable counting sort), so the result is unique;
 *  - expert e gets P_e = ceil(c_e / BM) * BM rows starting at off_e = sum_{e'<e} P_e';
 *    rows past its c_e pairs, and all rows past sum P, hold the filler value T*k;
 *  - expert_ids[b] names the expert of block b, -1 for blocks past the last used one;
 *  - inv_pos[t*k + j] is the row that holds pair (t, j).
 */
int orc_align(int T, int k, int E, int BM, const int32_t *ids, int32_t *sorted_token_ids,
              int32_t *expert_ids, int32_t *num_tokens_post_padded, int32_t *expert_counts,
              int32_t *inv_pos)
{
    if (T < 0 || k < 1 || E < 1 || BM < 1) return -1;
    int64_t pairs = (int64_t)T * k, cap = orc_align_capacity(T, k, E, BM);
    for (int64_t i = 0; i < pairs; i++)
        if (ids[i] < 0 || ids[i] >= E) return -1;
    int64_t *off = calloc((size_t)E, sizeof(int64_t)), *next = calloc((size_t)E, sizeof(int64_t));
    for (int e = 0; e < E; e++) expert_counts[e] = 0;
    for (int64_t i = 0; i < pairs; i++) expert_counts[ids[i]]++;
    int64_t total = 0;
    for (int e = 0; e < E; e++) {
        off[e] = total;
        total += (expert_counts[e] + BM - 1) / BM * BM;
    }
    for (int64_t r = 0; r < cap; r++) sorted_token_ids[r] = (int32_t)pairs;
    for (int64_t b = 0; b < cap / BM; b++) expert_ids[b] = -1;
    for (int e = 0; e < E; e++) {
        next[e] = off[e];
        int64_t padded = (expert_counts[e] + BM - 1) / BM * BM;
        for (int64_t b = off[e] / BM; b < (off[e] + padded) / BM; b++) expert_ids[b] = e;
    }
    for (int64_t i = 0; i < pairs; i++) {
        int64_t r = next[ids[i]]++;
        sorted_token_ids[r] = (int32_t)i;
        inv_pos[i] = (int32_t)r;
    }
    *num_tokens_post_padded = (int32_t)total;
    free(off);
    free(next);
    return 0;
}

/* ------------------------------------------------------------------------------------ */
/* expert weights                                                                        */
/* ------------------------------------------------------------------------------------ */

/* Matrix m of expert e: m = 0 is w13 ([2I, H]: rows [0, I) the gate projection W1 whose
 * output goes through SiLU, rows [I, 2I) the up projection W3), m = 1 is w2 ([H, I]). */
static void mat_shape(const orc_weights *W, int m, int64_t *rows, int64_t *cols)
{
    *rows = m == 0 ? 2 * (int64_t)W->I : W->H;
    *cols = m == 0 ? W->H : W->I;
}

/*
 * Dequantised value of one weight.
 *  bf16: the value itself.
 *  fp8 (w8a8 per tensor, as served in SGLang PR #2333 and named in the FBGEMM article):
 *    E4M3 code times the expert's fp32 scale for that matrix.
 *  int4 (GPTQ/AWQ group-wise, vLLM PR #12185): unsigned nibble q, group of 128 columns
 *    sharing an fp16 scale s and an fp16 zero point z; value (q - z) * s.  Column c sits
 *    in byte c/2 of its row, in the low nibble when c is even.
 */
double orc_weight(const orc_weights *W, int m, int e, int64_t n, int64_t c)
{
    int64_t rows, cols;
    mat_shape(W, m, &rows, &cols);
    int64_t idx = ((int64_t)e * rows + n) * cols + c;
    const void *w = m == 0 ? W->w13 : W->w2;
    if (W->wdtype == ORC_BF16) return orc_bf16_to_f32(((const uint16_t *)w)[idx]);
    if (W->wdtype == ORC_FP8_E4M3) {
        const float *scale = m == 0 ? W->w13_scale : W->w2_scale;
        return (double)orc_e4m3_to_f32(((const uint8_t *)w)[idx]) * (double)scale[e];
    }
    /* int4 */
    uint8_t byte = ((const uint8_t *)w)[((int64_t)e * rows + n) * (cols / 2) + c / 2];
    int q = (c % 2 == 0) ? (byte & 0xF) : (byte >> 4);
    int64_t gidx = ((int64_t)e * (cols / 128) + c / 128) * rows + n;   /* group-major [E, cols/128, rows] */
    double s = orc_f16_to_f32((m == 0 ? W->w13_s : W->w2_s)[gidx]);
    double z = orc_f16_to_f32((m == 0 ? W->w13_z : W->w2_z)[gidx]);
    return ((double)q - z) * s;
}

/* E4M3 codes decoded once into a table of their values (from orc_e4m3_to_f32, so the table
 * holds exactly what the decoder returns): the rows of an fp8 layer are decoded with it. */
static float e4m3_value[256];
static pthread_once_t e4m3_once = PTHREAD_ONCE_INIT;
static void e4m3_fill(void)
{
    for (int c = 0; c < 256; c++) e4m3_value[c] = orc_e4m3_to_f32((uint8_t)c);
}

/* Dequantise one row of matrix m of expert e into buf (length cols): the value orc_weight
 * gives for every column, walking the row once (an int4 group's scale and zero point are
 * decoded once per group). */
static void weight_row(const orc_weights *W, int m, int e, int64_t n, double *buf)
{
    int64_t rows, cols;
    mat_shape(W, m, &rows, &cols);
    if (W->wdtype == ORC_BF16) {
        const uint16_t *row = (const uint16_t *)(m == 0 ? W->w13 : W->w2) + ((int64_t)e * rows + n) * cols;
        for (int64_t c = 0; c < cols; c++) buf[c] = orc_bf16_to_f32(row[c]);
        return;
    }
    if (W->wdtype == ORC_FP8_E4M3) {
        const uint8_t *row = (const uint8_t *)(m == 0 ? W->w13 : W->w2) + ((int64_t)e * rows + n) * cols;
        double scale = (m == 0 ? W->w13_scale : W->w2_scale)[e];
        pthread_once(&e4m3_once, e4m3_fill);
        for (int64_t c = 0; c < cols; c++) buf[c] = (double)e4m3_value[row[c]] * scale;
        return;
    }
    const uint8_t *row = (const uint8_t *)(m == 0 ? W->w13 : W->w2) + ((int64_t)e * rows + n) * (cols / 2);
    for (int64_t g = 0; g < cols / 128; g++) {
        int64_t gi = ((int64_t)e * (cols / 128) + g) * rows + n;
        double s = orc_f16_to_f32((m == 0 ? W->w13_s : W->w2_s)[gi]);
        double z = orc_f16_to_f32((m == 0 ? W->w13_z : W->w2_z)[gi]);
        for (int64_t c = g * 128; c < (g + 1) * 128; c++) {
            int q = (c % 2 == 0) ? (row[c / 2] & 0xF) : (row[c / 2] >> 4);
            buf[c] = ((double)q - z) * s;
        }
    }
}

/* Accumulation precision of the FFN.  ACC64: products and sums in fp64 (the reference the
 * tests compare against).  ACC32: the layer as the definition reads in single precision --
 * the dequantised weights and the activations taken as fp32 values, each product and
 * running sum rounded to fp32, SiLU and the slot sum in fp32 (a second instantiation that
 * the fp64 one must agree with to within fp32 rounding). */
enum { ACC64 = 0, ACC32 = 1 };

static double dot(const double *a, const double *b, int64_t n, int acc)
{
    if (acc == ACC32) {
        float s = 0.0f;
        for (int64_t i = 0; i < n; i++) s += (float)a[i] * (float)b[i];
        return s;
    }
    double s = 0.0;
    for (int64_t i = 0; i < n; i++) s += a[i] * b[i];
    return s;
}

static double silu(double z) { return z / (1.0 + exp(-z)); }
static float silu32(float z) { return z / (1.0f + expf(-z)); }

/* h = SiLU(W1_e x) * (W3_e x), length I. */
static void expert_intermediate(const orc_weights *W, int acc, int e, const double *x, double *h, double *row)
{
    for (int i = 0; i < W->I; i++) {
        weight_row(W, 0, e, i, row);
        double g = dot(row, x, W->H, acc);
        weight_row(W, 0, e, (int64_t)W->I + i, row);
        double u = dot(row, x, W->H, acc);
        if (acc == ACC32) h[i] = silu32((float)g) * (float)u;
        else h[i] = silu(g) * u;
    }
}

/* y = W2_e h, length H. */
static void expert_output(const orc_weights *W, int acc, int e, const double *h, double *y, double *row)
{
    for (int n = 0; n < W->H; n++) {
        weight_row(W, 1, e, n, row);
        y[n] = dot(row, h, W->I, acc);
    }
}

static int check_weights(const orc_weights *W)
{
    if (!W || W->E < 1 || W->H < 1 || W->I < 1) return -1;
    if (W->wdtype == ORC_INT4_G128 && (W->H % 128 || W->I % 128)) return -1;
    if (W->wdtype != ORC_BF16 && W->wdtype != ORC_FP8_E4M3 && W->wdtype != ORC_INT4_G128) return -1;
    return 0;
}

/* ------------------------------------------------------------------------------------ */
/* threads over tokens                                                                   */
/* ------------------------------------------------------------------------------------ */

/* The per-token work below is split over threads by contiguous ranges of tokens.  Each
 * token's arithmetic is the same whatever the split and every thread writes only its own
 * tokens' rows, so the results do not depend on the number of threads (bit for bit). */
typedef struct {
    const orc_weights *W;
    int acc, T, k;
    const uint16_t *hidden;
    const int32_t *ids;
    const float *weights;
    const int32_t *tokens;          /* output rows: token of row q (NULL: row q is token q) */
    const double *hall;             /* fp8: dequantised intermediate of every pair, or NULL */
    double *out;                    /* output rows, or (fp8 pass 1) the pairs' intermediates */
    float s1, inv1;                 /* fp8 pass 1: the activation scale and its inverse */
    int lo, hi;                     /* this thread's range */
} job;

/* fp8 pass 1 for tokens [lo, hi): the token's hidden row quantised with the per-tensor
 * scale and dequantised, then h of each of its k pairs into out. */
static void *fp8_pass1_range(void *arg)
{
    job *j = arg;
    const orc_weights *W = j->W;
    int H = W->H, I = W->I;
    double *x = malloc(sizeof(double) * H), *row = malloc(sizeof(double) * (H > I ? H : I));
    for (int t = j->lo; t < j->hi; t++) {
        for (int c = 0; c < H; c++) {
            float v = orc_bf16_to_f32(j->hidden[(int64_t)t * H + c]) * j->inv1;   /* fp32 product */
            x[c] = (double)orc_e4m3_to_f32(orc_f32_to_e4m3(v)) * (double)j->s1;
        }
        for (int s = 0; s < j->k; s++)
            expert_intermediate(W, j->acc, j->ids[(int64_t)t * j->k + s], x, j->out + ((int64_t)t * j->k + s) * I, row);
    }
    free(x);
    free(row);
    return NULL;
}

/* Output rows [lo, hi): out[t] = sum over slots of w_{t,j} * W2_e h_{t,j}, slots in order. */
static void *output_range(void *arg)
{
    job *jb = arg;
    const orc_weights *W = jb->W;
    int H = W->H, I = W->I, k = jb->k;
    double *x = malloc(sizeof(double) * H), *h = malloc(sizeof(double) * I);
    double *y = malloc(sizeof(double) * H), *row = malloc(sizeof(double) * (H > I ? H : I));
    for (int q = jb->lo; q < jb->hi; q++) {
        int t = jb->tokens ? jb->tokens[q] : q;
        double *o = jb->out + (int64_t)q * H;
        for (int n = 0; n < H; n++) o[n] = 0.0;
        if (!jb->hall)
            for (int c = 0; c < H; c++) x[c] = orc_bf16_to_f32(jb->hidden[(int64_t)t * H + c]);
        for (int j = 0; j < k; j++) {
            int e = jb->ids[(int64_t)t * k + j];
            const double *hj = h;
            if (jb->hall) hj = jb->hall + ((int64_t)t * k + j) * I;
            else expert_intermediate(W, jb->acc, e, x, h, row);
            expert_output(W, jb->acc, e, hj, y, row);
            double w = jb->weights[(int64_t)t * k + j];
            if (jb->acc == ACC32)
                for (int n = 0; n < H; n++) o[n] = (float)o[n] + (float)w * (float)y[n];
            else
                for (int n = 0; n < H; n++) o[n] += w * y[n];
        }
    }
    free(x); free(h); free(y); free(row);
    return NULL;
}

/* Run fn over [0, n) in nthreads contiguous ranges (n >= 0, nthreads >= 1). */
static int run_split(void *(*fn)(void *), const job *proto, int n, int nthreads)
{
    if (nthreads > n) nthreads = n > 0 ? n : 1;
    job *jobs = malloc(sizeof(job) * nthreads);
    pthread_t *th = malloc(sizeof(pthread_t) * nthreads);
    int rc = 0;
    for (int i = 0; i < nthreads; i++) {
        jobs[i] = *proto;
        jobs[i].lo = (int)((int64_t)n * i / nthreads);
        jobs[i].hi = (int)((int64_t)n * (i + 1) / nthreads);
    }
    if (nthreads == 1) {
        fn(&jobs[0]);
    } else {
        int started = 0;
        for (; started < nthreads; started++)
            if (pthread_create(&th[started], NULL, fn, &jobs[started])) { rc = -1; break; }
        for (int i = 0; i < started; i++) pthread_join(th[i], NULL);
    }
    free(jobs);
    free(th);
    return rc;
}

/* ------------------------------------------------------------------------------------ */
/* fp8 w8a8: dynamic per-tensor activation quantisation                                  */
/* ------------------------------------------------------------------------------------ */

/* Per-tensor scale from the tensor's largest magnitude: the largest element maps to the
 * largest E4M3 value 448.  Quantising uses v * (448 / amax) and dequantising code *
 * (amax / 448), both scale factors formed by one fp32 division; an all-zero tensor uses
 * scale 1. */
static void pertensor_scales(float amax, float *scale, float *inv)
{
    if (amax == 0.0f) { *scale = 1.0f; *inv = 1.0f; return; }
    *scale = amax / 448.0f;
    *inv = 448.0f / amax;
}

/* The w8a8 intermediate of every pair: pass 1 quantises all hidden rows with one scale,
 * computes h = SiLU(g) * u from the dequantised codes; pass 2 takes the largest |h| over
 * all T*k pairs (each h rounded to fp32 first) and quantises every h with it. */
static int fp8_intermediate(const orc_weights *W, int acc, int nthreads, int T, int k, const uint16_t *hidden,
                            const int32_t *ids, double *hbuf, float *h32, uint8_t *hq, float *sc)
{
    int H = W->H, I = W->I;
    float amax1 = 0.0f;
    for (int64_t i = 0; i < (int64_t)T * H; i++) {
        float a = fabsf(orc_bf16_to_f32(hidden[i]));
        if (a > amax1) amax1 = a;
    }
    float s1, inv1;
    pertensor_scales(amax1, &s1, &inv1);
    job p = {0};
    p.W = W; p.acc = acc; p.T = T; p.k = k; p.hidden = hidden; p.ids = ids; p.out = hbuf;
    p.s1 = s1; p.inv1 = inv1;
    if (run_split(fp8_pass1_range, &p, T, nthreads)) return -1;
    float amax2 = 0.0f;
    for (int64_t i = 0; i < (int64_t)T * k * I; i++) {
        float a = fabsf((float)hbuf[i]);
        if (a > amax2) amax2 = a;
    }
    float s2, inv2;
    pertensor_scales(amax2, &s2, &inv2);
    for (int64_t i = 0; i < (int64_t)T * k * I; i++) {
        float v = (float)hbuf[i];
        uint8_t code = orc_f32_to_e4m3(v * inv2);                          /* fp32 product */
        if (h32) h32[i] = v;
        if (hq) hq[i] = code;
        hbuf[i] = (double)orc_e4m3_to_f32(code) * (double)s2;
    }
    if (sc) { sc[0] = s1; sc[1] = s2; }
    return 0;
}

int orc_fp8_intermediate(const orc_weights *W, int T, int k, const uint16_t *hidden_bf16,
                         const int32_t *ids, float *h, uint8_t *hq, float *scales)
{
    if (check_weights(W) || W->wdtype != ORC_FP8_E4M3 || T < 0 || k < 1) return -1;
    double *hbuf = malloc(sizeof(double) * ((size_t)T * k * W->I + 1));
    int rc = fp8_intermediate(W, ACC64, 1, T, k, hidden_bf16, ids, hbuf, h, hq, scales);
    free(hbuf);
    return rc;
}

/* ------------------------------------------------------------------------------------ */
/* the layer                                                                             */
/* ------------------------------------------------------------------------------------ */

int orc_forward_ex(const orc_weights *W, int T, int k, const uint16_t *hidden_bf16,
                   const int32_t *ids, const float *weights, int ntok, const int32_t *tokens,
                   double *out, float *dbg, int acc32, int nthreads)
{
    if (check_weights(W) || T < 0 || k < 1 || nthreads < 1) return -1;
    int n_out = tokens ? ntok : T;
    for (int q = 0; q < n_out; q++)
        if (tokens && (tokens[q] < 0 || tokens[q] >= T)) return -1;
    for (int64_t i = 0; i < (int64_t)T * k; i++)
        if (ids[i] < 0 || ids[i] >= W->E) return -1;
    int acc = acc32 ? ACC32 : ACC64;
    double *hall = NULL;
    if (W->wdtype == ORC_FP8_E4M3) {
        float sc[2];
        hall = malloc(sizeof(double) * ((size_t)T * k * W->I + 1));
        if (fp8_intermediate(W, acc, nthreads, T, k, hidden_bf16, ids, hall, NULL, NULL, sc)) { free(hall); return -1; }
        if (dbg) { dbg[0] = sc[0]; dbg[1] = sc[1]; }
    }
    job p = {0};
    p.W = W; p.acc = acc; p.T = T; p.k = k; p.hidden = hidden_bf16; p.ids = ids; p.weights = weights;
    p.tokens = tokens; p.hall = hall; p.out = out;
    int rc = run_split(output_range, &p, n_out, nthreads);
    free(hall);
    return rc;
}

int orc_forward(const orc_weights *W, int T, int k, const uint16_t *hidden_bf16,
                const int32_t *ids, const float *weights, int ntok, const int32_t *tokens,
                double *out, float *dbg)
{
    return orc_forward_ex(W, T, k, hidden_bf16, ids, weights, ntok, tokens, out, dbg, 0, 1);
}

/* ---- grouped GEMM over pre-permuted contiguous segments ----
 * [FBGEMM]: the grouped GEMM that EP-MoE runs on tokens already grouped by expert, with
 * bf16 operands or E4M3 operands and per-tensor scales.  Reading: segment e holds rows
 * [off_e, off_e + m_sizes[e]) of X, off_e the sum of the earlier sizes; every row r of
 * segment e gets Y[r, n] = x_scale * w_scale[e] * sum_c X[r, c] * W[e, n, c] (scales 1 for
 * bf16), in fp64 on the decoded values.  Rows past the last segment are left untouched. */
static double grouped_elem(int dtype, const void *base, int64_t i)
{
    if (dtype == ORC_BF16) return orc_bf16_to_f32(((const uint16_t *)base)[i]);
    return orc_e4m3_to_f32(((const uint8_t *)base)[i]);
}

int orc_grouped_gemm(int E, int N, int K, int dtype, int M, const void *x, float x_scale,
                     const void *w, const float *w_scale, const int32_t *m_sizes, double *y)
{
    if (E < 1 || N < 1 || K < 1 || M < 0 || (dtype != ORC_BF16 && dtype != ORC_FP8_E4M3)) return -1;
    if (dtype == ORC_FP8_E4M3 && !w_scale) return -1;
    int64_t total = 0;
    for (int e = 0; e < E; e++) {
        if (m_sizes[e] < 0) return -1;
        total += m_sizes[e];
    }
    if (total > M) return -1;
    double *xr = malloc(sizeof(double) * K);
    int64_t r = 0;
    for (int e = 0; e < E; e++) {
        double scale = dtype == ORC_FP8_E4M3 ? (double)x_scale * w_scale[e] : 1.0;
        for (int i = 0; i < m_sizes[e]; i++, r++) {
            for (int c = 0; c < K; c++) xr[c] = grouped_elem(dtype, x, r * K + c);
            for (int n = 0; n < N; n++) {
                double acc = 0.0;
                int64_t wrow = ((int64_t)e * N + n) * K;
                for (int c = 0; c < K; c++) acc += xr[c] * grouped_elem(dtype, w, wrow + c);
                y[r * N + n] = scale * acc;
            }
        }
    }
    free(xr);
    return 0;
}
