/*
 * moe.h -- C ABI of the MI355X (gfx950) MoE-layer forward library.
 *
 * The single-GPU forward of a Mixture-of-Experts layer in the four steps the
 * "Expert Parallelism" glossary page (Ultralytics; section "How tokens travel
 * between GPUs") lists -- route, dispatch, compute, combine -- plus the
 * selection-bias update of its "Load balancing and capacity" section:
 *
 *   moe_route        router logits, top-k selection (optional group limit and
 *                    selection-only bias), combine weights, per-expert counts
 *   moe_dispatch     capacity, token-order admission, expert- and
 *                    rank-contiguous row layout, permuted hidden states
 *                    (moe_dispatch_ex: also first-choice-first admission;
 *                    moe_dispatch_q8 / moe_dequantize_q8: INT8 row payload)
 *   moe_expert_ffn   every expert's FFN over its rows as one grouped GEMM pair
 *                    (bf16 weights packed once by moe_expert_ffn_pack_weights)
 *   moe_combine      weighted sum back to token order, plus residual and an
 *                    optional shared-expert output (or, after a fused down
 *                    GEMM, the finish of its fp32 accumulator)
 *   moe_bias_update  lower the selection bias of overloaded experts, raise it
 *                    for underloaded ones
 *   moe_combine_backward, moe_permute_backward
 *                    the data path's backward: gradients of the combine's
 *                    expert terms (rows and weights) and of the permute
 *   moe_expert_ffn_backward (moe_expert_ffn_backward_packed: on the forward's
 *                    grouped GEMM, with weights packed once)
 *                    the expert FFN's backward: input gradients of every
 *                    expert's rows and the experts' weight gradients
 *
 * Conventions (all entry points):
 *  - Every tensor pointer is a DEVICE pointer owned by the caller; the library
 *    never allocates device memory.  Scratch memory comes in through `ws`
 *    (size from the matching *_workspace_size query, 256-byte aligned).
 *  - `stream` is a hipStream_t (NULL = the null stream).  Work is enqueued
 *    asynchronously; nothing synchronises the host.
 *  - Arguments are validated on the host before any launch.  A call that
 *    returns an error has enqueued nothing and written nothing.
 *  - Layouts are row-major and dense (bf16 expert weights excepted: packed,
 *    see moe_expert_ffn_pack_weights).  Hidden-state buffers must be 16-byte
 *    aligned.  dtype MOE_BF16 buffers hold bf16, MOE_F32 buffers fp32; routing
 *    tensors (logits, weights, biases) are fp32 in both cases.
 *  - Every call fully overwrites its outputs (counts included), so calls are
 *    idempotent; calls on different streams with distinct buffers are
 *    independent.
 *  - Asynchronous device faults surface at the caller's next synchronisation.
 *  - No C++ exception crosses this interface.
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = 1,    /* a size, pointer or enum is out of range */
  MOE_ERR_UNSUPPORTED = 2,    /* valid, but outside what the kernels handle */
  MOE_ERR_HIP = 3,            /* a HIP launch failed */
  MOE_ERR_WORKSPACE = 4       /* ws is NULL or smaller than the query said */
};

/* Element types of hidden states and expert weights. */
enum { MOE_F32 = 0, MOE_BF16 = 1 };

/* How combine weights come from the router logits z (selection never uses
 * these weights; it ranks z, or the sigmoid of z, plus the selection bias):
 *  MOE_SOFTMAX_TOPK  softmax over the k selected logits (GShard/Mixtral top-2)
 *  MOE_SOFTMAX_ALL   softmax over all E logits, taken at the selected experts,
 *                    not renormalised (Switch top-1)
 *  MOE_SIGMOID_NORM  sigmoid affinities, renormalised over the k selected
 *                    (DeepSeek-V3); selection ranks sigmoid(z) + bias */
enum { MOE_SOFTMAX_TOPK = 0, MOE_SOFTMAX_ALL = 1, MOE_SIGMOID_NORM = 2 };

/* Expert activation: ReLU and GELU (exact erf) FFNs are act(x W1^T) W2^T;
 * SwiGLU is (silu(x W1^T) * (x W3^T)) W2^T with W1 the gate, W3 the up. */
enum { MOE_RELU = 0, MOE_GELU = 1, MOE_SWIGLU = 2 };

/* The routing problem as the pages state it: tokens and their hidden states,
 * number of experts, number of GPUs (here simulated EP ranks, expert e on rank
 * e / (E/R), as in the glossary snippet), top-k, capacity factor (glossary
 * "Load balancing and capacity"), and the node-limited group restriction
 * (DeepSeek-V3: each token reaches experts on a bounded number of nodes). */
typedef struct {
  int32_t num_tokens;       /* N >= 0 */
  int32_t hidden;           /* d >= 1, multiple of 8 */
  int32_t num_experts;      /* E in [1, 256] */
  int32_t top_k;            /* k in [1, min(E, 8)] */
  int32_t num_ranks;        /* R >= 1, E % R == 0 */
  float   capacity_factor;  /* <= 0: unlimited; else cap = ceil(cf * N * k / E) */
  int32_t num_groups;       /* G >= 1, E % G == 0; 1 = no group limit */
  int32_t topk_groups;      /* kg in [1, G], kg * (E/G) >= k */
  int32_t score_fn;         /* MOE_SOFTMAX_TOPK / MOE_SOFTMAX_ALL / MOE_SIGMOID_NORM */
  int32_t dtype;            /* MOE_F32 / MOE_BF16 */
} moe_route_desc;

/* ------------------------------------------------------------------ route -- */

/* Workspace bytes moe_route needs (0 when N == 0). */
size_t moe_route_workspace_size(const moe_route_desc* desc);

/* Route.  Glossary "How tokens travel between GPUs", step 1: the router scores
 * each token against each expert and keeps the k highest; "Load balancing and
 * capacity": a per-expert bias added to the scores steers selection only.
 *
 *  x           [N, d]  dtype       hidden states
 *  w_router    [E, d]  dtype       router weight (Linear(d, E).weight)
 *  router_bias [E]     fp32        Linear bias, nullable
 *  sel_bias    [E]     fp32        selection-only bias, nullable
 *  logits      [N, E]  fp32  out   the router logit, defined as
 *                                  z[t,e] = fp32( fp64 sum over i = 0..d-1, in
 *                                  order, of x[t,i]*w[e,i]; then + router_bias[e]
 *                                  in fp64 ), rounded once to nearest-even.
 *                                  MOE_F32: every entry is that value.
 *                                  MOE_BF16: entries of the selected experts (and
 *                                  of any expert whose rank the selection had to
 *                                  resolve exactly) are that value; the others
 *                                  are within 2^-16 |x_t| |w_e| + 2^-22 |z| of it
 *                                  (selection is decided only on exact values)
 *  topk_idx    [N, k]  int32 out   chosen experts, best first; a token's
 *                                  selection score is sigmoid(z) (SIGMOID_NORM,
 *                                  fp64 then rounded to fp32) or z, plus
 *                                  sel_bias in fp32; ties go to the lower index;
 *                                  with G > 1 only experts in the kg groups with
 *                                  the highest group score (max selection score
 *                                  in the group; ties to the lower group) are
 *                                  eligible
 *  topk_w      [N, k]  fp32  out   combine weights (score_fn), from unbiased z
 *  counts      [E]     int32 out   assignments per expert before capacity
 *                                  (sum = N*k)
 *  ws, ws_bytes                    workspace, >= moe_route_workspace_size */
int moe_route(const moe_route_desc* desc, const void* x, const void* w_router,
              const float* router_bias, const float* sel_bias, float* logits,
              int32_t* topk_idx, float* topk_w, int32_t* counts,
              void* ws, size_t ws_bytes, void* stream);

/* Exact router logits of every (token, expert) pair, as defined for moe_route,
 * with no selection (glossary "How tokens travel between GPUs": the router is
 * a Linear(d, E) over the hidden state).  x, w_router, router_bias (nullable)
 * and logits [N, E] fp32 as for moe_route; only num_tokens, hidden,
 * num_experts and dtype of desc are used beyond validation; ws as for
 * moe_route (same size query). */
int moe_router_logits(const moe_route_desc* desc, const void* x, const void* w_router,
                      const float* router_bias, float* logits, void* ws, size_t ws_bytes,
                      void* stream);

/* --------------------------------------------------------------- dispatch -- */

/* Workspace bytes moe_dispatch needs. */
size_t moe_dispatch_workspace_size(const moe_route_desc* desc);

/* Dispatch.  Glossary step 2 (the dispatch all-to-all sends each token's hidden
 * state to the rank that holds its experts) and the capacity-factor bullet
 * (each expert takes at most cap = ceil(cf*N*k/E) assignments per batch; the
 * rest skip that expert).  Single-GPU form: the send buffer and its counts.
 *
 *  x              [N, d]    dtype  hidden states
 *  topk_idx       [N, k]    int32  from moe_route (values in [0, E))
 *  x_perm         [N*k, d]  dtype  out: rows 0..M-1 are the admitted
 *                                  assignments grouped by expert in increasing
 *                                  expert order, token order inside an expert;
 *                                  x_perm[r] = x[token_of_row[r]] bit for bit.
 *                                  Since rank = e / (E/R) is non-decreasing in
 *                                  e, the buffer is also rank-contiguous.
 *                                  Rows >= M are left untouched.
 *  row_of_slot    [N, k]    int32  out: row of slot (t,j), -1 if dropped;
 *                                  admission walks tokens in order
 *  token_of_row   [N*k]     int32  out: token of each row (entries >= M: -1)
 *  slot_of_row    [N*k]     int8   out: slot j of each row (entries >= M: -1)
 *  expert_offsets [E+1]     int32  out: exclusive scan of admitted; [E] = M
 *  admitted       [E]       int32  out: min(count_e, cap)
 *  rank_offsets   [R+1]     int32  out: expert_offsets[r * E/R]
 *  rank_counts    [R]       int32  out: rows per rank (the all-to-all's send
 *                                  counts)
 * Returns MOE_ERR_INVALID_ARG for bad sizes; out-of-range expert ids in
 * topk_idx are a caller error the kernels do not detect. */
int moe_dispatch(const moe_route_desc* desc, const void* x, const int32_t* topk_idx,
                 void* x_perm, int32_t* row_of_slot, int32_t* token_of_row,
                 int8_t* slot_of_row, int32_t* expert_offsets, int32_t* admitted,
                 int32_t* rank_offsets, int32_t* rank_counts,
                 void* ws, size_t ws_bytes, void* stream);

/* Admission orders of moe_dispatch_ex. */
typedef enum {
  MOE_ADMIT_TOKEN_ORDER = 0,  /* tokens in order, a token's slots j = 0..k-1 in turn */
  MOE_ADMIT_FIRST_CHOICE = 1, /* slot 0 of every token (in token order), then slot 1
                                 of every token, and so on */
  MOE_LAYOUT_PADDED = 2       /* flag, with either order: fixed buffers of cap rows per
                                 expert (see moe_dispatch_rows) */
} moe_admission;

/* Rows a dispatch with these admission flags lays out: N*k for the compact
 * layout; max(N*k, E*cap) with MOE_LAYOUT_PADDED.  EP notes, "参考答案" answer 2,
 * sizes each expert's buffer as the mean load times the capacity factor; the
 * padded layout is that buffer: expert e owns rows [e*cap, (e+1)*cap),
 * expert_offsets[e] = e*cap (so moe_expert_ffn runs every row of the buffer,
 * GShard's static shapes), its admitted rows come first in admission order,
 * and the rest are padding: token_of_row = slot_of_row = -1 and, from
 * moe_dispatch_ex / moe_dispatch_q8, zero rows (zero codes, scale 0), whose
 * FFN output is zero and which moe_combine never reads.  rank_counts are then
 * (E/R)*cap: an all-to-all of fixed size.  x_perm, token_of_row, slot_of_row
 * (and x_perm_q, row_scale) need this many rows.  The padded layout needs a
 * finite capacity (cf > 0).  Returns -1 for an invalid descriptor or flags. */
int64_t moe_dispatch_rows(const moe_route_desc* desc, int32_t admission);

/* Dispatch with a choice of admission order.  MLSys ch.10, section 10.5 names
 * GShard's top-2 router, whose first choices outrank second choices when an
 * expert fills up; the pages fix no admission priority, and
 * MOE_ADMIT_FIRST_CHOICE is the plainest reading of such a router: the
 * capacity is filled by walking every token's first choice (token order),
 * then every second choice, and so on.  Rows inside an expert follow the same
 * walk: by (slot, token) for MOE_ADMIT_FIRST_CHOICE, so token_of_row is not
 * monotonic inside an expert there.  Everything else -- arguments, layout,
 * admitted = min(count_e, cap), rank offsets, workspace size, errors -- is as
 * for moe_dispatch, which is moe_dispatch_ex with MOE_ADMIT_TOKEN_ORDER.  With
 * k = 1, or with no capacity limit, both orders admit the same slots.
 * admission may also carry MOE_LAYOUT_PADDED (see moe_dispatch_rows for the
 * layout and the buffer sizes).  Returns MOE_ERR_INVALID_ARG for any other
 * admission value, and for MOE_LAYOUT_PADDED without a capacity. */
int moe_dispatch_ex(const moe_route_desc* desc, int32_t admission, const void* x,
                    const int32_t* topk_idx, void* x_perm, int32_t* row_of_slot,
                    int32_t* token_of_row, int8_t* slot_of_row, int32_t* expert_offsets,
                    int32_t* admitted, int32_t* rank_offsets, int32_t* rank_counts,
                    void* ws, size_t ws_bytes, void* stream);

/* Dispatch that allocates nothing and takes no workspace, for callers that
 * cannot allocate device memory: code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc.  Arguments, outputs, layout and
 * errors are those of moe_dispatch_ex (same kernels, bit-identical results);
 * the kernels' scratch lives in a 1 MiB device array inside the library
 * instead of ws, one copy per GPU, kept until the process ends.
 *  - The call runs on the current device (the one `stream` belongs to); its
 *    first call on a device looks the array's address up (no allocation).
 *  - A batch needing more scratch than the array holds -- ceil(N*k / 1024) * E
 *    * 4 bytes > 1 MiB, i.e. more than about 2^20 slots at E = 256 -- returns
 *    MOE_ERR_UNSUPPORTED and enqueues nothing.
 *  - Every call on one GPU shares that GPU's array: calls that overlap on one
 *    GPU (different streams, or other host threads) race and give wrong
 *    layouts.  Serialise them.  No state carries over from one call to the
 *    next: every call writes each scratch entry before reading it. */
int moe_dispatch_noalloc(const moe_route_desc* desc, int32_t admission, const void* x,
                         const int32_t* topk_idx, void* x_perm, int32_t* row_of_slot,
                         int32_t* token_of_row, int8_t* slot_of_row, int32_t* expert_offsets,
                         int32_t* admitted, int32_t* rank_offsets, int32_t* rank_counts,
                         void* stream);

/* The two halves of moe_dispatch_ex / moe_dispatch_q8, for callers that schedule
 * them apart -- a multi-GPU layer exchanges the rank counts from the layout
 * before it moves the rows (glossary step 2) -- or time them apart.
 * moe_dispatch_layout: histograms, capacity, admission walk, scan and ranks --
 *   every output of moe_dispatch_ex except x_perm (arguments, workspace and
 *   errors as there; x is not read).
 * moe_permute: x_perm[row_of_slot[t, j]] = x[t] for every admitted slot (the
 *   permute of moe_dispatch; row_of_slot from moe_dispatch_layout).  It writes
 *   admitted rows only: padding rows of a padded layout are left as they are
 *   (the whole-dispatch calls zero them).
 * moe_permute_q8: the same rows as the INT8 payload (codes and scales exactly
 *   as moe_dispatch_q8).
 * A layout followed by a permute on one stream equals one moe_dispatch_ex /
 * moe_dispatch_q8 call, bit for bit. */
int moe_dispatch_layout(const moe_route_desc* desc, int32_t admission, const int32_t* topk_idx,
                        int32_t* row_of_slot, int32_t* token_of_row, int8_t* slot_of_row,
                        int32_t* expert_offsets, int32_t* admitted, int32_t* rank_offsets,
                        int32_t* rank_counts, void* ws, size_t ws_bytes, void* stream);
int moe_permute(const moe_route_desc* desc, const void* x, const int32_t* row_of_slot,
                void* x_perm, void* stream);
int moe_permute_q8(const moe_route_desc* desc, const void* x, const int32_t* row_of_slot,
                   int8_t* x_perm_q, float* row_scale, void* stream);

/* INT8 payload of the dispatch exchange.  EP notes, "深入推导" (DeepSeek-V3's EP
 * configuration): INT8-quantised communication halves the exchange volume.  The
 * pages give no scheme; this is one symmetric scale per token row, each
 * decision an fp32 IEEE operation rounded to nearest even:
 *   amax = max_i |x_ti|;  inv = 127 / amax;  q_ti = clamp(rint(x_ti * inv), -127, 127);
 *   scale_t = amax / 127   (a row of zeros: q = 0, scale = 0).
 * moe_dispatch_q8 is moe_dispatch_ex (same arguments, outputs, workspace and
 * errors) except that the permuted rows are written as that payload instead of
 * dtype rows:
 *  x_perm_q   [N*k, d]  int8   out: row r holds the codes of x[token_of_row[r]]
 *                              (rows >= M untouched); 16-byte aligned
 *  row_scale  [N*k]     fp32   out: its scale (entries >= M untouched)
 * x is read once per token.  Returns MOE_ERR_UNSUPPORTED when d exceeds 8192
 * (bf16) / 4096 (fp32), the row a wave keeps in registers. */
int moe_dispatch_q8(const moe_route_desc* desc, int32_t admission, const void* x,
                    const int32_t* topk_idx, int8_t* x_perm_q, float* row_scale,
                    int32_t* row_of_slot, int32_t* token_of_row, int8_t* slot_of_row,
                    int32_t* expert_offsets, int32_t* admitted, int32_t* rank_offsets,
                    int32_t* rank_counts, void* ws, size_t ws_bytes, void* stream);

/* Receiver side of the INT8 payload: x_perm[r, i] = q[r, i] * row_scale[r] as an
 * fp32 product, rounded to dtype (bf16: nearest even), for r < min(*num_rows,
 * max_rows).  num_rows is a DEVICE pointer (for the layer: &expert_offsets[E]),
 * so the row count never has to reach the host.  x_perm_q and x_perm
 * 16-byte aligned; d % 8 == 0 (else MOE_ERR_UNSUPPORTED). */
int moe_dequantize_q8(int32_t max_rows, int32_t hidden, int32_t dtype, const int8_t* x_perm_q,
                      const float* row_scale, const int32_t* num_rows, void* x_perm,
                      void* stream);

/* ------------------------------------------------------------- expert FFN -- */

/* Fused combine of the down GEMM (glossary step 4 folded into step 3): with
 * this argument the down GEMM does not write y_rows; each expert output row r
 * (token t = token_of_row[r], slot j = slot_of_row[r]; rows with t = -1 are
 * skipped) is rounded to dtype, as the unfused path stores it, multiplied by
 * topk_w[t, j] in fp32 and added into y_acc[t] with fp32 atomic adds.  The call
 * first zeroes y_acc (with a kernel: the call stays capturable in a graph).
 * moe_combine with y_acc then adds the residual and shared output and rounds.
 * The atomic adds of a token's k rows land in no fixed order, so with k > 1
 * the result may differ between runs in the last bits; with k = 1 each
 * element receives one add onto zero and the result is the same on every run.
 * Either way it matches the unfused path to rounding (within the layer
 * tolerance), not bit for bit: the unfused combine rounds once per fused
 * multiply-add, this path rounds the product and the sum apart.  A token whose
 * every slot was dropped keeps y_acc = 0, so its y is the residual unchanged.
 * The shared expert never takes this path. */
typedef struct {
  int32_t num_tokens;          /* N: rows of y_acc (>= every token_of_row + 1) */
  int32_t top_k;               /* k: topk_w is [N, k] */
  const float* topk_w;         /* [N, k] fp32, from moe_route */
  const int32_t* token_of_row; /* [max_rows] int32, from the dispatch (-1: no token) */
  const int8_t* slot_of_row;   /* [max_rows] int8, from the dispatch */
  float* y_acc;                /* [N, d] fp32 out, 16-byte aligned; owned by the caller */
} moe_fused_combine;

/* Workspace bytes moe_expert_ffn needs for up to max_rows rows. */
size_t moe_expert_ffn_workspace_size(int32_t num_experts, int32_t max_rows, int32_t hidden,
                                     int32_t ffn_hidden, int32_t act, int32_t dtype);

/* Expert FFN.  Glossary step 3 (each GPU runs its local experts on the tokens
 * it received); each expert is an ordinary FFN.  Rows [offsets[e],
 * offsets[e+1]) of x_rows go through expert e:
 *   H = act(X W1_e^T) (SwiGLU: silu(X W1_e^T) * (X W3_e^T)), stored in dtype;
 *   Y = H W2_e^T, stored in dtype.  fp32 accumulation.
 *
 *  num_experts   E >= 1 (1 with offsets {0, N} runs a shared expert)
 *  max_rows      rows allocated in x_rows / y_rows (offsets[E] <= max_rows)
 *  hidden        d, multiple of 64;  ffn_hidden  h, multiple of 64
 *  x_rows        [max_rows, d]  dtype
 *  group_offsets [E+1]  int32  DEVICE array, non-decreasing, [0] = 0
 *  w1            [E, h, d]  dtype  (gate for SwiGLU)
 *  w3            [E, h, d]  dtype  (up; SwiGLU only, else NULL)
 *  w2            [E, d, h]  dtype
 *                fp32: row-major as shown.  bf16: in the packed layout that
 *                moe_expert_ffn_pack_weights writes (done once, when the
 *                weights are loaded); row-major bf16 weights give wrong
 *                results, which the library cannot detect.
 *  y_rows        [max_rows, d]  dtype out (rows >= offsets[E] untouched);
 *                NULL (and not written) when fused is given
 *  fused         nullable: the fused combine above (token_of_row and
 *                slot_of_row then cover max_rows rows)
 *  ws, ws_bytes  workspace >= moe_expert_ffn_workspace_size(...) */
int moe_expert_ffn(int32_t num_experts, int32_t max_rows, int32_t hidden, int32_t ffn_hidden,
                   int32_t act, int32_t dtype, const void* x_rows,
                   const int32_t* group_offsets, const void* w1, const void* w3,
                   const void* w2, void* y_rows, const moe_fused_combine* fused, void* ws,
                   size_t ws_bytes, void* stream);

/* The three stages of moe_expert_ffn, for callers that time or overlap them.
 * They share one workspace (same size query) and must run in this order on
 * one stream with the same num_experts, max_rows, group_offsets and ws:
 *  moe_expert_ffn_plan  per-expert row-tile schedule from group_offsets
 *  moe_expert_ffn_up    H = act(X W1_e^T) (SwiGLU: silu(X W1_e^T)*(X W3_e^T)),
 *                       H kept in ws, one kernel launch
 *  moe_expert_ffn_down  Y = H W2_e^T, one kernel launch (with fused: a zeroing
 *                       launch for y_acc, then the GEMM scatter-adding into it)
 * Arguments mean what they mean for moe_expert_ffn; errors likewise. */
int moe_expert_ffn_plan(int32_t num_experts, int32_t max_rows, int32_t hidden,
                        int32_t ffn_hidden, int32_t act, int32_t dtype,
                        const int32_t* group_offsets, void* ws, size_t ws_bytes, void* stream);
int moe_expert_ffn_up(int32_t num_experts, int32_t max_rows, int32_t hidden, int32_t ffn_hidden,
                      int32_t act, int32_t dtype, const void* x_rows,
                      const int32_t* group_offsets, const void* w1, const void* w3,
                      void* ws, size_t ws_bytes, void* stream);
int moe_expert_ffn_down(int32_t num_experts, int32_t max_rows, int32_t hidden,
                        int32_t ffn_hidden, int32_t act, int32_t dtype,
                        const int32_t* group_offsets, const void* w2, void* y_rows,
                        const moe_fused_combine* fused, void* ws, size_t ws_bytes,
                        void* stream);

/* Pack one bf16 expert weight tensor for the bf16 expert FFN.
 *
 *  num_experts  E >= 1
 *  rows, cols   the tensor is [E, rows, cols] row-major bf16: rows = output
 *               features of its GEMM, cols = input features (W1, W3: rows = h,
 *               cols = d; W2: rows = d, cols = h); both multiples of 64
 *  dtype        MOE_BF16 (fp32 weights are used row-major: MOE_ERR_UNSUPPORTED)
 *  w            source, device, 16-byte aligned; not modified
 *  w_packed     destination, device, E*rows*cols bf16, 16-byte aligned, must
 *               not overlap w; owned by the caller
 *
 * Layout: rows are grouped in slabs of S rows, S = 256 if rows % 256 == 0,
 * else 64.  Element (e, n, k), with s = n / S, g = (n % S) / 16, r = n % 16,
 * t = k / 32, c = (k % 32) / 8 and L = 4r + (c XOR sw(r)),
 * sw(r) = ((r >> 1) XOR (r >> 2)) & 3, is stored at element offset
 *   ((e*(rows/S) + s)*(cols/32) + t)*S*32 + g*512 + 8*L + k % 8.
 * So each slab is cols/32 consecutive stages of S x 32 elements, and each
 * stage is S/16 blocks of 1 KB in the order the GEMM kernel stages weight
 * rows in LDS: every K step of a slab is one contiguous run of S * 64 bytes.
 * A pure permutation: the packed tensor holds the same values bit for bit.
 * Errors: MOE_ERR_INVALID_ARG (sizes, null/misaligned/overlapping pointers),
 * MOE_ERR_UNSUPPORTED (fp32, rows or cols not a multiple of 64), MOE_ERR_HIP. */
int moe_expert_ffn_pack_weights(int32_t num_experts, int32_t rows, int32_t cols, int32_t dtype,
                                const void* w, void* w_packed, void* stream);

/* The same packed layout for a matrix given transposed, as the backward on
 * the grouped GEMM needs it (moe_expert_ffn_backward_packed): per expert e the
 * [rows, cols] matrix M_e whose columns j < cols_a are row j of wa[e] and
 * whose columns j >= cols_a are row j - cols_a of wb[e]:
 *   wa [E, cols_a, rows], wb [E, cols - cols_a, rows] bf16 row-major (wb
 *   NULL exactly when cols_a == cols); w_packed [E, rows, cols] bf16.
 * The backward takes W2^T (rows = h, cols = cols_a = d, wa = w2 [E, d, h]) and
 * [W1^T | W3^T] (rows = d, cols_a = h, cols = 2h for SwiGLU with wa = w1, wb =
 * w3, both [E, h, d]; cols = h and wb = NULL otherwise).  Like the forward's
 * packing it is done once per weight update, not per step.  A permutation of
 * the values.  Errors: MOE_ERR_INVALID_ARG (sizes, cols_a > cols, wb given or
 * missing wrongly, null/misaligned/overlapping pointers), MOE_ERR_UNSUPPORTED
 * (fp32; rows or cols not a multiple of 64, cols_a not of 8), MOE_ERR_HIP. */
int moe_expert_ffn_pack_weights_t(int32_t num_experts, int32_t rows, int32_t cols_a,
                                  int32_t cols, int32_t dtype, const void* wa, const void* wb,
                                  void* w_packed, void* stream);

/* ---------------------------------------------------------------- combine -- */

/* Combine.  Glossary step 4 (outputs return to each token and are weighted by
 * the router scores and summed) and "Load balancing and capacity" (a skipped
 * token passes through the residual connection unchanged):
 *   y[t] = residual[t] + shared_out[t] + sum_j [row_of_slot[t,j] >= 0] *
 *          topk_w[t,j] * y_perm[row_of_slot[t,j]]
 * accumulated in fp32 in that order and rounded once to dtype.
 *
 *  y_perm      [>=M, d]  dtype   expert outputs by row
 *  row_of_slot [N, k]    int32   from moe_dispatch
 *  topk_w      [N, k]    fp32    from moe_route
 *  residual    [N, d]    dtype   nullable (normally x)
 *  shared_out  [N, d]    dtype   nullable (always-on shared expert output)
 *  y_acc       [N, d]    fp32    nullable: the accumulator a fused down GEMM
 *                                (moe_fused_combine) filled; then
 *                                y[t] = residual[t] + shared_out[t] + y_acc[t]
 *                                in fp32, rounded once, and y_perm,
 *                                row_of_slot and topk_w are not read (may be
 *                                NULL).  16-byte aligned.
 *  y           [N, d]    dtype   out */
int moe_combine(const moe_route_desc* desc, const void* y_perm, const int32_t* row_of_slot,
                const float* topk_w, const void* residual, const void* shared_out,
                const float* y_acc, void* y, void* stream);

/* --------------------------------------------------------------- backward -- */

/* Backward of the data path (a training step reads the glossary's four steps
 * of "How tokens travel between GPUs" in reverse).
 *
 * moe_combine_backward: given dy [N, d] (dtype), the forward's y_perm,
 * row_of_slot and topk_w, for every admitted slot (t, j) with row r:
 *   dy_perm[r]    = w_tj * dy[t]            fp32 product, rounded once to the dtype
 *   dtopk_w[t, j] = <dy[t], y_perm[r]>      exact products summed in fp64, then fp32
 * A dropped slot gets dtopk_w = 0 and writes no row; rows of dy_perm no slot
 * maps to are left untouched.  The residual and shared terms of moe_combine pass
 * dy on unchanged, so they need no call.  dy, y_perm, dy_perm 16-byte aligned.
 *
 * moe_permute_backward: dx[t] = sum over the token's admitted slots, in slot
 * order, of dx_perm[row_of_slot[t, j]] (fp32, rounded once to the dtype); a
 * token with every slot dropped gets zero.  This is the adjoint of the permute
 * (x_perm[r] = x[token_of_row[r]]).  dx_perm, dx 16-byte aligned.
 *
 * Both return MOE_ERR_INVALID_ARG for a bad descriptor, missing or misaligned
 * buffers. */
int moe_combine_backward(const moe_route_desc* desc, const void* dy, const void* y_perm,
                         const int32_t* row_of_slot, const float* topk_w, void* dy_perm,
                         float* dtopk_w, void* stream);
int moe_permute_backward(const moe_route_desc* desc, const void* dx_perm,
                         const int32_t* row_of_slot, void* dx, void* stream);

/* Backward of the expert FFN (each expert is an ordinary feed-forward block:
 * glossary "Expert Parallelism", introduction).  With the forward of
 * moe_expert_ffn, u = x W1^T, v = x W3^T, H = act(u) [* v], y = H W2^T, over
 * rows [group_offsets[e], group_offsets[e+1]) (clamped to max_rows and, when
 * group_rows is given, to the first group_rows[e] of them) of expert e:
 *   g   = dy W2                     (gradient at H)
 *   du  = g * act'(u) [* v]         rounded to bf16
 *   dv  = g * silu(u)               SwiGLU only, rounded to bf16
 *   dx  = du W1 [+ dv W3]           rounded to bf16, written to dx_rows
 *   dw1[e] = sum_r du^T x,  dw3[e] = sum_r dv^T x,  dw2[e] = sum_r dy^T H
 * u, v and H are recomputed and rounded to bf16 at the forward's rounding
 * point; products run on bf16 operands with fp32 sums.  GELU is the erf form,
 * gelu(u) = u Phi(u) and gelu'(u) = Phi(u) + u phi(u).  This entry point takes
 * Phi from the device erf, whereas the forward evaluates erf by a polynomial,
 * so its recomputed H can differ from the forward's H by one bf16 ulp;
 * moe_expert_ffn_backward_packed recomputes u (v) on the forward's grouped
 * GEMM and forms H, Phi and silu with the forward's own expressions.
 *
 *  x_rows, dy_rows, dx_rows [max_rows, d] bf16 (dy_rows: the gradient at
 *      y_rows, e.g. moe_combine_backward's dy_perm; rows outside every
 *      segment are neither read nor written);
 *  group_rows [E] int32 DEVICE array, nullable: rows of each segment that
 *      hold data.  With the capacity-padded layout pass the dispatch's
 *      admitted: the padding rows then take no part (moe_combine_backward
 *      leaves them unwritten in dy_perm, and moe_permute leaves them as they
 *      were in x_perm) and the gradients equal the compact layout's;
 *  w1, w3 [E, h, d] and w2 [E, d, h] bf16, PLAIN row-major (not the packed
 *      layout of moe_expert_ffn); w3 and dw3 only for MOE_SWIGLU (NULL else);
 *  dw1, dw3 [E, h, d] and dw2 [E, d, h] fp32, fully written (zero for an
 *      expert with no rows, also when max_rows == 0).
 * dtype must be MOE_BF16, d and h multiples of 32, E <= 1024 (else
 * MOE_ERR_UNSUPPORTED).  Workspace from moe_expert_ffn_backward_workspace_size
 * (H and [du | dv] for every row, about max_rows * 3h * 2 bytes for SwiGLU);
 * none is needed when max_rows == 0.  All buffers 16-byte aligned. */
size_t moe_expert_ffn_backward_workspace_size(int32_t num_experts, int32_t max_rows,
                                              int32_t hidden, int32_t ffn_hidden, int32_t act,
                                              int32_t dtype);
int moe_expert_ffn_backward(int32_t num_experts, int32_t max_rows, int32_t hidden,
                            int32_t ffn_hidden, int32_t act, int32_t dtype, const void* x_rows,
                            const int32_t* group_offsets, const int32_t* group_rows,
                            const void* w1, const void* w3, const void* w2, const void* dy_rows,
                            void* dx_rows, float* dw1, float* dw3, float* dw2, void* ws,
                            size_t ws_bytes, void* stream);

/* The same backward with every product on the forward's grouped GEMM
 * (moe_expert_ffn's kernel: operands streamed into LDS, packed weights) and
 * the same definitions, rounding points and outputs as moe_expert_ffn_backward:
 * u (and v) are recomputed as an fp32 GEMM, g = dy W2 runs as a GEMM whose
 * epilogue forms H, du, dv from u, v and g, and dx = [du | dv] [W1 ; W3] as
 * the forward's down GEMM over G; the weight gradients then run as in
 * moe_expert_ffn_backward.  Weights come packed:
 *   w1_packed, w3_packed  moe_expert_ffn_pack_weights of w1, w3 (rows h,
 *                         cols d), as the forward uses them;
 *   w2t_packed            moe_expert_ffn_pack_weights_t of w2 (rows h,
 *                         cols_a = cols = d);
 *   w13t_packed           moe_expert_ffn_pack_weights_t of w1 (and w3):
 *                         rows d, cols_a h, cols h (2h for SwiGLU).
 * Other arguments as in moe_expert_ffn_backward (group_rows included); d and h
 * must be multiples of 64.  The workspace (moe_expert_ffn_backward_packed_
 * workspace_size: the tile plan, G in the packed layout, u and v in fp32, G
 * and H row-major -- about max_rows * 9h * 2 bytes for SwiGLU) is needed only
 * when max_rows > 0.  Errors as moe_expert_ffn_backward's. */
size_t moe_expert_ffn_backward_packed_workspace_size(int32_t num_experts, int32_t max_rows,
                                                     int32_t hidden, int32_t ffn_hidden,
                                                     int32_t act, int32_t dtype);
int moe_expert_ffn_backward_packed(int32_t num_experts, int32_t max_rows, int32_t hidden,
                                   int32_t ffn_hidden, int32_t act, int32_t dtype,
                                   const void* x_rows, const int32_t* group_offsets,
                                   const int32_t* group_rows, const void* w1_packed,
                                   const void* w3_packed, const void* w2t_packed,
                                   const void* w13t_packed, const void* dy_rows, void* dx_rows,
                                   float* dw1, float* dw3, float* dw2, void* ws, size_t ws_bytes,
                                   void* stream);

/* Backward of the router (glossary "How tokens travel between GPUs", step 1,
 * read backwards: the router's logits decide the combine weights) and of an
 * auxiliary load-balancing loss (glossary "Load balancing and capacity",
 * auxiliary-loss bullet; MLSys ch.10 section 10.5 names it for GShard).  The
 * pages give the loss no formula; it is taken as the Switch Transformer's,
 * for k slots:
 *   L = aux_coef * E * sum_e f_e P_e,  f_e = counts[e] / (N k)  (a constant),
 *   P_e = mean over tokens of the token's router distribution over all E
 *         (softmax of z; SIGMOID_NORM: sigmoid(z) / sum over all E of sigmoid(z)).
 * From the logits z, the selection topk_idx and dtopk_w (the gradient at the
 * combine weights, moe_combine_backward's output; dropped slots carry 0):
 *   dz[t, e]  gradient at the logits: through the score function at the
 *             selected experts (the selection itself, incl. group limit and
 *             selection bias, passes no gradient) plus the loss's term
 *   dw_router = dz^T x,  drouter_bias = sum over tokens of dz  (fp32)
 *   dx[t]     = sum_e dz[t, e] w_router[e]  (+ dx[t] when accumulate_dx: the
 *             rest of the layer's input gradient; rounded once to dtype)
 * fp32 arithmetic; the loss is summed in fp64 in a fixed order.
 *
 *  x [N, d] dtype, w_router [E, d] dtype, logits [N, E] fp32 (moe_route's, or
 *  moe_router_logits'), topk_idx [N, k] int32, dtopk_w [N, k] fp32,
 *  counts [E] int32 (pre-capacity, moe_route's; needed when aux_coef != 0),
 *  aux_coef  finite; 0 = no auxiliary loss,
 *  dlogits [N, E] fp32 out, nullable;  dw_router [E, d] fp32 out;
 *  drouter_bias [E] fp32 out, nullable;  dx [N, d] dtype (in/)out, nullable,
 *  16-byte aligned;  aux_loss: one fp32 DEVICE value out, nullable;
 *  ws, ws_bytes >= moe_router_backward_workspace_size (0 when N == 0).
 * With N == 0 the gradients are zero and the loss 0.  Errors:
 * MOE_ERR_INVALID_ARG (descriptor, missing or misaligned buffers, counts
 * missing with aux_coef != 0, a non-finite aux_coef), MOE_ERR_WORKSPACE. */
size_t moe_router_backward_workspace_size(const moe_route_desc* desc);
int moe_router_backward(const moe_route_desc* desc, const void* x, const void* w_router,
                        const float* logits, const int32_t* topk_idx, const float* dtopk_w,
                        const int32_t* counts, float aux_coef, float* dlogits, float* dw_router,
                        float* drouter_bias, void* dx, int32_t accumulate_dx, float* aux_loss,
                        void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------ bias update -- */

/* Selection-bias update.  Glossary "Load balancing and capacity", bias-based
 * balancing: after each step the bias of overloaded experts goes down and that
 * of idle ones goes up.  In place, for each e:
 *   counts[e]*E > N*k  ->  sel_bias[e] -= step   (fp32)
 *   counts[e]*E < N*k  ->  sel_bias[e] += step
 *   equal              ->  unchanged
 *  counts [E] int32 (pre-capacity, from moe_route), sel_bias [E] fp32. */
int moe_bias_update(int32_t num_experts, int32_t num_tokens, int32_t top_k,
                    const int32_t* counts, float step, float* sel_bias, void* stream);

/* Human-readable name of a status code (static storage). */
const char* moe_status_string(int status);

#ifdef __cplusplus
}
#endif
#endif /* MOE_MI355X_H */
