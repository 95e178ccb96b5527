/*
 * oracle.h -- CPU reference for the single-GPU forward of a Mixture-of-Experts
 * layer (route -> dispatch -> expert FFN -> combine, plus the selection-bias
 * update).
 *
 * TEST INFRASTRUCTURE ONLY.  This library is the correctness oracle for the
 * HIP path.  Only the tests, the smoke entry point and the CPU-baseline leg of
 * the benchmark may load it.  It shares no code, header, table or helper with
 * the HIP library, and the HIP library never calls it.
 *
 * Everything is plain per-token / per-row loops in fp64 except where a
 * rounding point is part of the definition (logits to fp32; hidden activations,
 * expert outputs and layer outputs to the layer dtype, round-to-nearest-even).
 *
 * Sources (web pages; each function cites the passage it follows):
 *  [EP-glossary]  "Expert Parallelism", Ultralytics glossary (zh/de/ja
 *                 editions say the same): sections "How tokens travel between
 *                 GPUs" (four steps + routing snippet), "Load balancing and
 *                 capacity" (capacity factor, selection-only bias, drops pass
 *                 through the residual, node-limited routing).
 *  [EP-notes]     "专家并行" (bowenzhou.top): "MoE 的账先算清楚" (256 routed +
 *                 1 shared expert, 8 active), "机制：all-to-all 两轮"
 *                 (dispatch/combine), answer 2 of "参考答案" (per-expert buffer
 *                 = mean x capacity factor).
 *  [MLSys-ch10]   "第 10 章 模型并行与专家并行", section 10.5 (top-1 Switch,
 *                 top-2 GShard, DeepSeekMoE shared + fine-grained experts).
 *
 * Dtype codes: 0 = fp32, 1 = bf16 (raw uint16 bit patterns).
 * Score codes: 0 = softmax over the k selected logits, 1 = softmax over all E
 *              logits (not renormalised), 2 = sigmoid affinities renormalised
 *              over the k selected.
 * Activation codes: 0 = ReLU, 1 = GELU (erf), 2 = SwiGLU.
 * Return value of every int function: 0 on success, -1 on invalid arguments.
 */
#ifndef MOE_ORACLE_H
#define MOE_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct {
  int32_t num_tokens;      /* N */
  int32_t hidden;          /* d */
  int32_t num_experts;     /* E */
  int32_t top_k;           /* k */
  int32_t num_ranks;       /* R, E % R == 0 */
  float   capacity_factor; /* <= 0: no capacity limit */
  int32_t num_groups;      /* G, 1 = no group limit */
  int32_t topk_groups;     /* kg */
  int32_t score_fn;        /* 0/1/2, see above */
  int32_t dtype;           /* 0 fp32, 1 bf16 */
} oracle_desc;

/* Router logits z[N,E] (fp32) of x[N,d] against w[E,d], plus bias[E] (nullable). */
int oracle_logits(const oracle_desc* desc, const void* x, const void* w,
                  const float* router_bias, float* z);

/* Selection from given logits: topk_idx[N,k], topk_w[N,k], counts[E].
 * sel_bias[E] is nullable. affinity[N,E] (nullable) receives the fp32 score
 * f(z) before the bias (z itself for the softmax modes). */
int oracle_select(const oracle_desc* desc, const float* z, const float* sel_bias,
                  int32_t* topk_idx, float* topk_w, int32_t* counts, float* affinity);

/* Capacity, token-order admission and the expert/rank-contiguous layout.
 * token_of_row / slot_of_row have N*k entries; entries from M on are set to -1. */
int oracle_dispatch(const oracle_desc* desc, const int32_t* topk_idx,
                    int32_t* row_of_slot, int32_t* token_of_row, int8_t* slot_of_row,
                    int32_t* expert_offsets, int32_t* admitted,
                    int32_t* rank_offsets, int32_t* rank_counts);

/* The same with a choice of admission order.  admission 0: token order (as
 * oracle_dispatch).  admission 1: first choice first -- slot j = 0 of every
 * token in token order, then j = 1 of every token, and so on; rows inside an
 * expert follow that order.  MLSys ch.10, section 10.5 names GShard's top-2
 * router; the pages fix no admission priority, and this is the plainest
 * reading of a router that ranks first choices above second ones.
 * Bit 1 of admission (value 2, combinable with either order) asks for the
 * padded layout of GShard-style fixed buffers ("参考答案" answer 2 of the EP
 * notes sizes each expert's buffer as the mean load times the capacity
 * factor): expert e owns rows [e cap, (e+1) cap), expert_offsets[e] = e cap,
 * its admitted rows come first in admission order and the rest are padding
 * (token_of_row = slot_of_row = -1); rank offsets and counts follow from the
 * offsets as before.  token_of_row / slot_of_row then hold max(N k, E cap)
 * entries.  The padded layout needs a finite capacity (cf > 0).
 * Returns -1 for any other admission value. */
int oracle_dispatch_ex(const oracle_desc* desc, int32_t admission, const int32_t* topk_idx,
                       int32_t* row_of_slot, int32_t* token_of_row, int8_t* slot_of_row,
                       int32_t* expert_offsets, int32_t* admitted,
                       int32_t* rank_offsets, int32_t* rank_counts);

/* x_perm[i] = x[token_of_row[i]] for i < num_rows (a byte copy); a row with
 * token_of_row[i] < 0 (padding of the padded layout) is all zero bytes. */
int oracle_permute(int32_t num_rows, int32_t hidden, int32_t dtype, const void* x,
                   const int32_t* token_of_row, void* x_perm);

/* INT8 payload of the dispatch exchange, one symmetric scale per row (EP
 * notes, "深入推导": INT8-quantised communication halves the exchange volume;
 * the scheme is a reading).  Each step an fp32 IEEE operation rounded to
 * nearest even: amax = max |x_i|; inv = 127 / amax; q_i = clamp(rint(x_i * inv),
 * -127, 127); scale = amax / 127 (a zero row gives q = 0, scale = 0).
 * q is [num_rows, hidden] int8, scale [num_rows] fp32. */
int oracle_quantize_rows_q8(int32_t num_rows, int32_t hidden, int32_t dtype, const void* x,
                            int8_t* q, float* scale);

/* x_i = q_i * scale as an fp32 product, rounded to the dtype (bf16: nearest even). */
int oracle_dequantize_rows_q8(int32_t num_rows, int32_t hidden, int32_t dtype, const int8_t* q,
                              const float* scale, void* x);

/* One row of one expert's FFN: y = W2 act(W1 x [, W3 x]).  w1/w3 are [h,d],
 * w2 is [d,h] (row-major, out x in); w3 only for SwiGLU (gate = w1, up = w3). */
int oracle_ffn_row(int32_t hidden, int32_t ffn_hidden, int32_t act, int32_t dtype,
                   const void* x_row, const void* w1, const void* w3, const void* w2,
                   void* y_row);

/* Grouped FFN: rows [offsets[e], offsets[e+1]) of x_rows use expert e's
 * weights w1[e], w3[e], w2[e] ([E,h,d], [E,h,d], [E,d,h]). */
int oracle_expert_ffn(int32_t num_experts, int32_t hidden, int32_t ffn_hidden,
                      int32_t act, int32_t dtype, const void* x_rows,
                      const int32_t* offsets, const void* w1, const void* w3,
                      const void* w2, void* y_rows);

/* Backward of one row through one expert (chain rule through oracle_ffn_row):
 * g = dy W2, du = g act'(u) [* v], dv = g silu(u) (SwiGLU), dx = du W1 [+ dv W3];
 * du, dv and dx rounded to the dtype.  h_out/du_out/dv_out (nullable, h doubles
 * each) receive H as the forward rounds it, du and dv. */
int oracle_ffn_backward_row(int32_t hidden, int32_t ffn_hidden, int32_t act, int32_t dtype,
                            const void* x_row, const void* w1, const void* w3, const void* w2,
                            const void* dy_row, void* dx_row, double* h_out, double* du_out,
                            double* dv_out);

/* Backward of the grouped FFN: dx_rows for every row of a segment, and fp32
 * weight gradients dw1/dw3 [E,h,d] (sum over the expert's rows of du x^T,
 * dv x^T) and dw2 [E,d,h] (sum of dy H^T); zero for an expert with no rows. */
int oracle_expert_ffn_backward(int32_t num_experts, int32_t hidden, int32_t ffn_hidden,
                               int32_t act, int32_t dtype, const void* x_rows,
                               const int32_t* offsets, const void* w1, const void* w3,
                               const void* w2, const void* dy_rows, void* dx_rows, float* dw1,
                               float* dw3, float* dw2);

/* y[t] = residual[t] + shared[t] + sum_j w[t,j] y_perm[row_of_slot[t,j]]
 * (residual, shared nullable; dropped slots, row < 0, contribute nothing). */
int oracle_combine(int32_t num_tokens, int32_t hidden, int32_t top_k, int32_t dtype,
                   const void* y_perm, const int32_t* row_of_slot, const float* topk_w,
                   const void* residual, const void* shared_out, void* y);

/* Selection-bias update from pre-capacity counts. */
/* Backward of the combine's expert terms: dy_perm[r] = w * dy[t] (rounded to the
 * dtype) and dtopk_w[t, j] = <dy[t], y_perm[r]> (fp64 sum, rounded to fp32) for
 * every admitted slot; dropped slots get dtopk_w = 0.  (The permute's backward
 * is oracle_combine with unit weights and no residual.) */
int oracle_combine_backward(int32_t num_tokens, int32_t hidden, int32_t top_k, int32_t dtype,
                            const void* dy, const void* y_perm, const int32_t* row_of_slot,
                            const float* topk_w, void* dy_perm, float* dtopk_w);

int oracle_bias_update(int32_t num_experts, int32_t num_tokens, int32_t top_k,
                       const int32_t* counts, float step, float* sel_bias);

/* Backward of the router and of an auxiliary load-balancing loss (see
 * oracle.c): from the logits z, the selection and dtopk_w, the gradient dz at
 * the logits (fp32 out), dW_r [E,d] and db [E] (fp32; db nullable), the
 * router's input gradient dx [N,d] in the dtype (plus dx_in when not NULL),
 * and the loss coef * E * sum_e f_e P_e in *aux_loss (coef 0: none). */
int oracle_router_backward(const oracle_desc* desc, const void* x, const void* w_router,
                           const float* z, const int32_t* topk_idx, const float* dtopk_w,
                           const int32_t* counts, double aux_coef, const void* dx_in,
                           float* dz_out, float* dw_router, float* db, void* dx,
                           double* aux_loss);

/* Capacity for a descriptor (INT32_MAX when unlimited). */
int64_t oracle_capacity(const oracle_desc* desc);

/* Threads the route loop may use (OpenMP over tokens; 1 = sequential). */
void oracle_set_threads(int32_t n);
int32_t oracle_get_threads(void);

#ifdef __cplusplus
}
#endif
#endif
