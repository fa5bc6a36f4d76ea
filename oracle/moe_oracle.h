/*
 * moe_oracle.h -- plain CPU reference of the fused Mixture-of-Experts layer forward.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may include, link, load or
 * call this code; only the tests, the smoke check and the CPU-baseline leg of the
 * benchmark do.  It shares no code, header, table or helper with the GPU library.
 *
 * Everything is written for readability, not speed: one token at a time, one expert
 * at a time, fp64 accumulation on dequantised weights (an fp32-accumulation variant
 * serves as a cross-check); tokens may be spread over threads, each computing whole
 * tokens exactly as the single-threaded run does.  Where floating point decides
 * an integer (a top-k selection, an fp8 code) the decision is taken in fp32, the
 * precision the GPU kernels use for it.
 *
 * Sources (web pages; cited by title and section):
 *  [GATE]  SGLang PR #3191 "Add deepseek_v3 fused gate": the biased grouped top-k gate
 *          and its reference twin; the request that the output order be deterministic;
 *          the TensorRT-LLM pipeline fused gate -> expand_and_permute -> grouped GEMM ->
 *          unpermute_and_reduce (last review comment).
 *  [ALIGN] vLLM PR #12185 "[Kernel] add triton fused moe kernel for gptq/awq": the
 *          moe_align_block_size step (note 1 under the generation-speed table) and the
 *          int4 GPTQ/AWQ (group-wise scales and zeros) weights.
 *  [SPLITK] SGLang PR #2333 "[kernel] introduce fused_moe_triton_splitk": fp8 w8a8
 *          serving (Accuracy / GTX 4090 Performance sections), atomic-add corruption
 *          of the output (Background).
 *  [FBGEMM] aijishu article on FBGEMM's MoE grouped GEMM vs SGLang's (BBuf): per-tensor
 *          fp8 w8a8 (Limitations paragraph).
 * The pages give no formulas; the readings taken where they are silent are stated at
 * each function.
 */
#ifndef MOE_ORACLE_H
#define MOE_ORACLE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* routing modes */
enum { ORC_ROUTE_SOFTMAX = 0, ORC_ROUTE_SIGMOID = 1, ORC_ROUTE_GROUPED_SIGMOID_BIAS = 2 };
/* element encodings */
enum { ORC_BF16 = 0, ORC_FP32 = 1, ORC_FP8_E4M3 = 2, ORC_INT4_G128 = 3 };

/* ---- number codecs (own implementations, from the IEEE / OCP definitions) ---- */
float    orc_bf16_to_f32(uint16_t bits);
uint16_t orc_f32_to_bf16(float x);          /* round to nearest, ties to even */
float    orc_f16_to_f32(uint16_t bits);
float    orc_e4m3_to_f32(uint8_t code);     /* OCP E4M3FN: bias 7, no inf, S.1111.111 = NaN */
uint8_t  orc_f32_to_e4m3(float x);          /* RNE, saturating to +-448 */
float    orc_sigmoid(float x);              /* 1/(1+exp(-x)) in fp64, rounded once to fp32 */

/* ---- routing: per token, top-k experts and their weights ----
 * logits: [T,E] as bf16 bits (logits_dtype ORC_BF16) or fp32; bias: [E] fp32 or NULL.
 * ids: [T,k] int32 in slot order; weights: [T,k] fp32.  Returns 0, or -1 on bad args. */
int orc_route(int kind, int E, int k, int renormalize, int n_group, int topk_group,
              float routed_scaling, int logits_dtype, const void *logits, const float *bias,
              int T, int32_t *ids, float *weights);

/* ---- align: stable counting sort of the (token, slot) pairs by expert, padded ----
 * capacity() is the length of sorted_token_ids; expert_ids has capacity/BM entries. */
int64_t orc_align_capacity(int T, int k, int E, int BM);
int orc_align(int T, int k, int E, int BM, const int32_t *ids, int32_t *sorted_token_ids,
              int32_t *expert_ids, int32_t *num_tokens_post_padded, int32_t *expert_counts,
              int32_t *inv_pos);

/* ---- the layer's expert weights ---- */
typedef struct {
    int E, H, I;
    int wdtype;                 /* ORC_BF16, ORC_FP8_E4M3 or ORC_INT4_G128 */
    const void *w13;            /* bf16 bits / e4m3 codes [E,2I,H]; int4: uint8 [E,2I,H/2] */
    const void *w2;             /* bf16 bits / e4m3 codes [E,H,I];  int4: uint8 [E,H,I/2]  */
    const float *w13_scale;     /* fp8: [E] per-expert per-tensor scale of w13 */
    const float *w2_scale;      /* fp8: [E] */
    const uint16_t *w13_s, *w13_z;  /* int4: fp16 [E,H/128,2I] scales and zero points (group-major) */
    const uint16_t *w2_s, *w2_z;    /* int4: fp16 [E,I/128,H] */
} orc_weights;

/* Dequantised weight element of expert e, matrix m (0 = w13, 1 = w2), row n, column c. */
double orc_weight(const orc_weights *W, int m, int e, int64_t n, int64_t c);

/* ---- the layer output ----
 * out[t,:] = sum_j weights[t,j] * FFN_{ids[t,j]}(x_t) in fp64, for the tokens listed in
 * tokens[0..ntok) (all tokens when tokens == NULL; out is then [T,H], else [ntok,H]).
 * For fp8 weights the activations are quantised per tensor, dynamically, as w8a8
 * defines (two passes; the second pass needs every token's intermediate, so fp8 always
 * computes the intermediate of all T tokens).
 * dbg (nullable, fp8 only): dbg[0] = activation scale s1, dbg[1] = intermediate scale s2. */
int orc_forward(const orc_weights *W, int T, int k, const uint16_t *hidden_bf16,
                const int32_t *ids, const float *weights, int ntok, const int32_t *tokens,
                double *out, float *dbg);

/* orc_forward with its two options: acc32 = 0 accumulates in fp64 (orc_forward), 1 in fp32
 * (operands taken as fp32 values, each product and sum rounded to fp32, SiLU and the slot
 * sum in fp32); the per-token work runs on nthreads >= 1 threads over contiguous ranges of
 * tokens, with results identical bit for bit for every nthreads. */
int orc_forward_ex(const orc_weights *W, int T, int k, const uint16_t *hidden_bf16,
                   const int32_t *ids, const float *weights, int ntok, const int32_t *tokens,
                   double *out, float *dbg, int acc32, int nthreads);

/* fp8 intermediate of every (token, slot) pair, before and after its quantisation:
 * h[T*k, I] (fp32 value of the fp64 intermediate) and hq[T*k, I] (e4m3 codes). */
int orc_fp8_intermediate(const orc_weights *W, int T, int k, const uint16_t *hidden_bf16,
                         const int32_t *ids, float *h, uint8_t *hq, float *scales);

/* ---- grouped GEMM over pre-permuted contiguous per-expert segments (EP-MoE) ----
 * Segment e = rows [off_e, off_e + m_sizes[e]) of x, off_e = sum of the earlier sizes;
 * y[r, n] = x_scale * w_scale[e] * sum_c x[r, c] * w[e, n, c] in fp64 (dtype ORC_BF16:
 * bf16 bits, scales 1; ORC_FP8_E4M3: E4M3 codes and per-tensor scales).  x [M, K],
 * w [E, N, K], y [M, N]; rows past the last segment are not written.  Returns -1 for a
 * negative size or sizes summing past M. */
int orc_grouped_gemm(int E, int N, int K, int dtype, int M, const void *x, float x_scale,
                     const void *w, const float *w_scale, const int32_t *m_sizes, double *y);

#ifdef __cplusplus
}
#endif
#endif
