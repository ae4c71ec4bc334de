/*
 * moe_ref: plain, slow, single-threaded C99 oracle of one Stable-LatentMoE
 * layer with MXFP4 routed experts.
 *
 * TEST INFRASTRUCTURE ONLY.  The tests, the smoke check and the CPU-baseline
 * leg of the benchmark call it to check and to time the GPU library; the GPU
 * library never includes, links or calls it, and it shares no code, header or
 * table with the GPU library.
 *
 * Pages followed (cited by page title and section):
 *  - kimi-k3-mlx digest, architecture table: 896 routed experts, top-16 per
 *    token; routed experts work in a 3584-wide latent space instead of the
 *    7168-wide residual ("Stable LatentMoE" row, and the LatentMoE bullet
 *    under "five things implemented anew"); SiTU-GLU activation computed in
 *    fp32 (activation row and the SiTU-GLU bullet).
 *  - kimi-k3-mlx digest, quantisation tiers: the native mxfp4 mode uses the
 *    checkpoint's own encoding, low-nibble-first codes with an e8m0 scale.
 *  - kimi-k3-in-c post, "experts that are already 4-bit MXFP4": each weight is
 *    a 4-bit nibble indexing a 16-entry table, 32 consecutive weights share one
 *    8-bit exponent, 0.53125 bytes per weight, 33,030,144 weights and
 *    17,547,264 bytes per expert.
 *  - kimi-k3-mlx digest, REAP pruning: router weights are probabilities and
 *    are renormalised over the experts that remain.
 *
 * Readings where the pages are silent (each stated at its function):
 *  - the 16 E2M1 values are +-{0, .5, 1, 1.5, 2, 3, 4, 6} with bit 3 the sign
 *    (OCP Microscaling Formats v1.0, E2M1); e8m0 scale s means 2^(s-127), and
 *    s = 255 is NaN;
 *  - a record holds gate, up, down; each matrix is [out][in] row-major, codes
 *    (rows x cols/2 bytes) then scales (rows x cols/32 bytes), blocks of 32
 *    running along the input (reduction) axis;
 *  - router logits are the correctly rounded fp32 value of the exact dot
 *    product of bf16 x and bf16 router row, then an optional fp32 bias is added
 *    with one fp32 rounding; top-k orders by (logit descending, expert index
 *    ascending), +0 == -0, NaN below -inf; weights are the softmax over the k
 *    selected logits (or over all E when renormalize = 0);
 *  - rounding points: h = bf16(x W_d^T), g and u fp32, a = bf16(act(g) * u),
 *    y fp32, z = bf16(sum_j w_j y_j), out = bf16(z W_u^T); every sum is taken
 *    in fp64 (products of the operands are exact in fp64) and rounded once at
 *    the point named; round-to-nearest-even everywhere;
 *  - act = SiLU (g / (1 + exp(-g))); the SiTU formula is not given on the
 *    pages, so MOE_REF_ACT_SITU is rejected (parity unpinned).
 *
 * bf16 values travel as uint16_t bit patterns.  All pointers are host memory
 * owned by the caller.  Functions returning int give 0 on success, -1 for an
 * invalid argument, -2 for an unsupported option.
 */
#ifndef MOE_REF_H
#define MOE_REF_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { MOE_REF_OK = 0, MOE_REF_ERR_ARG = -1, MOE_REF_ERR_UNSUPPORTED = -2 };
enum { MOE_REF_ACT_SILU = 0, MOE_REF_ACT_SITU = 1 };
/* activation format at the expert GEMM inputs: the bf16 values themselves, or their
 * MXFP8 (E4M3 + e8m0 per 32) quantisation (OCP Microscaling v1.0 convention) */
enum { MOE_REF_ACT_BF16 = 0, MOE_REF_ACT_MXFP8 = 1 };

/* value of an E4M3 code (NaN for S.1111.111) */
double moe_ref_e4m3_value(int32_t code);
/* MXFP8 of one block of 32 values: codes[32] and the e8m0 scale byte */
int moe_ref_mxfp8_block(const double* v, uint8_t* codes, uint8_t* scale);

/* bytes of one expert record: 3 * d_latent * d_ffn weights at 0.53125 B */
size_t moe_ref_expert_bytes(int32_t d_latent, int32_t d_ffn);

/* the E2M1 value of a 4-bit code (bit 3 sign, bits 2..1 exponent, bit 0 mantissa) */
float moe_ref_e2m1(int32_t code);

/* one MXFP4 weight: fp32 of E2M1(code) * 2^(scale-127); NaN when scale == 255 */
float moe_ref_mxfp4_value(int32_t code, int32_t scale);

/* dequantise a [rows][cols] MXFP4 matrix (codes then scales as laid out above) */
int moe_ref_dequant_matrix(const uint8_t* codes, const uint8_t* scales, int64_t rows, int64_t cols,
                           float* out);

/* round a double to bf16 bits (nearest, ties to even; overflow to inf) */
uint16_t moe_ref_bf16_from_f64(double v);

/* correctly rounded fp32 of the exact sum of a[i]*b[i] over bf16 vectors */
float moe_ref_dot_bf16_exact(const uint16_t* a, const uint16_t* b, int64_t n);

/* logits[t][e] = RN32(exact x_t . W_r[e]) (+ bias[t*bias_stride + e], one fp32 add).
 * Each logit equals moe_ref_dot_bf16_exact of the pair: an fp64 sum with a proven
 * error bound settles the rounding when it can, the exact accumulator otherwise. */
int moe_ref_router_logits(const uint16_t* x, const uint16_t* router_w, const float* bias,
                          int64_t bias_stride, int64_t T, int32_t d, int32_t E, float* logits);

/* top-k per token, idx ascending; weights softmax over selected (renorm) or all */
int moe_ref_select(const float* logits, int64_t T, int32_t E, int32_t k, int32_t renormalize,
                   int32_t* idx, float* w);

/* stable grouping by (expert, token): counts[E], offsets[E+1], perm[T*k] = t*k+j */
int moe_ref_permute(const int32_t* idx, int64_t T, int32_t k, int32_t E, int32_t* counts,
                    int32_t* offsets, int32_t* perm);

/* out[t][o] = bf16(sum_i in[t][i] * W[o][i]) for bf16 in [T][n_in], W [n_out][n_in] */
int moe_ref_linear_bf16(const uint16_t* in, const uint16_t* W, int64_t T, int32_t n_in, int32_t n_out,
                        uint16_t* out);

/* REAP saliency sum: s[idx[t][j]] += w[t][j] * ||y[t*k+j]||_2 (fp64), accumulated */
int moe_ref_reap_saliency(const float* y, const float* w, const int32_t* idx, int64_t T, int32_t k,
                          int32_t L, int32_t E, double* s);

/* SiLU in double, the oracle's GLU activation */
double moe_ref_silu(double g);

/* one routed expert on one latent row: a (bf16 [F], nullable) and y (fp32 [L]) */
int moe_ref_expert(const uint16_t* h, const uint8_t* record, int32_t d_latent, int32_t d_ffn,
                   int32_t act, uint16_t* a_out, float* y);
/* the same with the activation format of h and a at the GEMM inputs */
int moe_ref_expert_fmt(const uint16_t* h, const uint8_t* record, int32_t d_latent, int32_t d_ffn,
                       int32_t act, int32_t act_format, uint16_t* a_out, float* y);

/* z[t][l] = bf16(sum_j w[t][j] * y[t*k+j][l]) */
int moe_ref_combine(const float* y, const float* w, int64_t T, int32_t k, int32_t d_latent,
                    uint16_t* z);

/*
 * The whole layer for the tokens listed in `tokens` (n_tokens of them; NULL
 * means tokens 0..n_tokens-1).  Row i of out/idx/w/logits/h/z belongs to token
 * tokens[i].  Tokens are independent in this layer, so a subset gives exactly
 * the rows a full run would.  idx, w, logits, h, z are nullable outputs.
 */
int moe_ref_layer_forward(int32_t d_model, int32_t d_latent, int32_t d_ffn, int32_t num_experts,
                          int32_t k, int32_t act, int32_t renormalize, const uint16_t* x,
                          const uint16_t* router_w, const float* bias, int64_t bias_stride,
                          const uint16_t* latent_down, const uint16_t* latent_up,
                          const uint8_t* expert_blob, const int32_t* tokens, int64_t n_tokens,
                          uint16_t* out, int32_t* idx, float* w, float* logits, uint16_t* h,
                          uint16_t* z);
/* the same with num_shared shared experts (records of moe_ref_expert_bytes(d_model, F_s)
 * in shared_blob, SiLU-GLU on x, weight 1, added to the latent-up product before the
 * bf16 rounding of out) */
int moe_ref_layer_forward_shared(int32_t d_model, int32_t d_latent, int32_t d_ffn, int32_t num_experts,
                                 int32_t k, int32_t act, int32_t act_format, int32_t renormalize,
                                 const uint16_t* x, const uint16_t* router_w, const float* bias,
                                 int64_t bias_stride, const uint16_t* latent_down, const uint16_t* latent_up,
                                 const uint8_t* expert_blob, const int32_t* tokens, int64_t n_tokens,
                                 uint16_t* out, int32_t* idx, float* w, float* logits, uint16_t* h,
                                 uint16_t* z, const uint8_t* shared_blob, int32_t num_shared, int32_t F_s);
/* the same with the activation format of the expert GEMM inputs */
int moe_ref_layer_forward_fmt(int32_t d_model, int32_t d_latent, int32_t d_ffn, int32_t num_experts,
                              int32_t k, int32_t act, int32_t act_format, int32_t renormalize,
                              const uint16_t* x, const uint16_t* router_w, const float* bias,
                              int64_t bias_stride, const uint16_t* latent_down, const uint16_t* latent_up,
                              const uint8_t* expert_blob, const int32_t* tokens, int64_t n_tokens,
                              uint16_t* out, int32_t* idx, float* w, float* logits, uint16_t* h,
                              uint16_t* z);

#ifdef __cplusplus
}
#endif
#endif
