// kernels.h -- launch interface between the C ABI (api.hip) and the kernels.
// Host-side validation happens in api.hip; these functions assume valid,
// already-checked arguments.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <algorithm>

namespace moe {

struct RouteArgs {
  int N, d, E, k, G, kg, score_fn, dtype;
  const void* x;
  const void* w_router;
  const float* router_bias;
  const float* sel_bias;
  float* logits;
  int32_t* topk_idx;
  float* topk_w;
  int32_t* counts;
  void* ws;
};

size_t route_workspace_bytes(int N, int d, int E, int dtype);
hipError_t launch_route(const RouteArgs& a, hipStream_t st);
// Exact logits for every (token, expert) pair (the fp64 definition), no selection.
hipError_t launch_router_logits(const RouteArgs& a, hipStream_t st);
// Certified path for bf16 inputs (route_mfma.hip).
size_t route_certified_workspace_bytes(int N, int d, int E);
hipError_t launch_route_certified(const RouteArgs& a, hipStream_t st);
void launch_zero_i32(int32_t* p, int n, hipStream_t st);

struct DispatchArgs {
  int N, d, E, k, R, dtype;
  int32_t cap;  // INT32_MAX when unlimited
  const void* x;
  const int32_t* topk_idx;
  void* x_perm;
  int32_t* row_of_slot;
  int32_t* token_of_row;
  int8_t* slot_of_row;
  int32_t* expert_offsets;
  int32_t* admitted;
  int32_t* rank_offsets;
  int32_t* rank_counts;
  void* ws;
  int first_choice;  // 0: token order; 1: every token's slot j before any slot j + 1
  void* xq = nullptr;          // INT8 payload rows [N*k, d] (x_perm unused when set)
  float* row_scale = nullptr;  // one scale per payload row
  int padded = 0;              // 1: expert e owns rows [e cap, (e+1) cap) (cap finite)
};

// Rows a dispatch lays out: N*k, or max(N*k, E*cap) for the padded layout.
size_t dispatch_rows(int N, int k, int E, int32_t cap, int padded);

// INT8 payload: the largest hidden size the register-resident quantiser takes,
// and the receiver-side dequantisation of rows < *num_rows.
int q8_max_hidden(int dtype);
hipError_t launch_dequantize_q8(int max_rows, int d, int dtype, const void* xq,
                                const float* row_scale, const int32_t* num_rows, void* out,
                                hipStream_t st);

size_t dispatch_workspace_bytes(int N, int k, int E);
// Stages of a dispatch: the layout (histograms, capacity, scan, ranks) and the
// permute of the rows (dtype rows, or the INT8 payload when xq is set).
enum { kDispatchLayout = 1, kDispatchPermute = 2 };
hipError_t launch_dispatch(const DispatchArgs& a, hipStream_t st,
                           int stages = kDispatchLayout | kDispatchPermute);

// Fused combine of the down GEMM: expert output row r goes, as
// topk_w[t, j] * dtype(O[r]), into y_acc[t] (t = token_of_row[r],
// j = slot_of_row[r]) by fp32 atomic adds instead of into y_rows.
struct FusedCombineArgs {
  int N, k;
  const float* topk_w;
  const int32_t* token_of_row;
  const int8_t* slot_of_row;
  float* y_acc;
};

struct FfnArgs {
  int E, max_rows, d, h, act, dtype;
  const void* x_rows;
  const int32_t* offsets;
  const void* w1;
  const void* w3;
  const void* w2;
  void* y_rows;
  void* ws;
  const FusedCombineArgs* fused = nullptr;  // down GEMM: scatter-add into y_acc
};

size_t ffn_workspace_bytes(int E, int max_rows, int d, int h, int act, int dtype);
hipError_t launch_ffn_plan(const FfnArgs& a, hipStream_t st);
hipError_t launch_ffn_up(const FfnArgs& a, hipStream_t st);
hipError_t launch_ffn_down(const FfnArgs& a, hipStream_t st);
// Zero the fused combine's accumulator (a.fused->y_acc, N x d fp32).
hipError_t launch_ffn_zero_acc(const FfnArgs& a, hipStream_t st);
hipError_t launch_pack_weights(int E, int N, int K, const void* w, void* wp, hipStream_t st);
// The packed layout of the [N, K] matrix [wa^T | wb^T] (wa [E, KA, N], wb
// [E, K - KA, N] row-major; wb unused when KA == K).
hipError_t launch_pack_weights_t(int E, int N, int KA, int K, const void* wa, const void* wb,
                                 void* wp, hipStream_t st);

// Backward of the expert FFN on the grouped GEMM (bf16, packed weights): the
// tile plan, u (v) recomputed in fp32, g = dy W2 with H, du, dv, and dx.
struct FfnBwdPackedArgs {
  int E, max_rows, d, h, act;
  const void* x_rows;
  const int32_t* offsets;
  const int32_t* group_rows;  // nullable
  const void* w1p;            // forward-packed W1 [E, h, d]
  const void* w3p;            // forward-packed W3 (SwiGLU)
  const void* w2tp;           // packed W2^T: N = h, K = d
  const void* w13tp;          // packed [W1^T | W3^T]: N = d, K = h or 2h
  const void* dy_rows;
  void* dx_rows;
  void* ws;
};
size_t ffn_bwd_packed_workspace_bytes(int E, int max_rows, int d, int h, int act);
// The GEMMs' share of it (the weight gradients' workspace follows).
size_t ffn_bwd_gemms_workspace_bytes(int E, int max_rows, int d, int h, int act);
hipError_t launch_zero_f32(float* p, size_t n, hipStream_t st);
// Enqueues the GEMMs; *g_rm and *h_rm receive the workspace's row-major G
// ([max_rows, kg]) and H ([max_rows, h]) for the weight gradients.
hipError_t launch_ffn_bwd_packed_gemms(const FfnBwdPackedArgs& a, void** g_rm, void** h_rm,
                                       hipStream_t st);
// The weight gradients on the grouped GEMM from the row-major G and H (and
// x, dy): transposed per expert into the GEMM's operand layouts, in a
// workspace of ffn_bwd_wgrad_workspace_bytes (256-aligned).
size_t ffn_bwd_wgrad_workspace_bytes(int E, int max_rows, int d, int h, int act);
hipError_t launch_ffn_bwd_wgrad(const FfnBwdPackedArgs& a, const void* g_rm, const void* h_rm,
                                void* ws, float* dw1, float* dw3, float* dw2, hipStream_t st);

struct CombineArgs {
  int N, d, k, dtype;
  const void* y_perm;
  const int32_t* row_of_slot;
  const float* topk_w;
  const void* residual;
  const void* shared_out;
  void* y;
  const float* y_acc = nullptr;  // set: finish a fused down GEMM's accumulator instead
};

hipError_t launch_combine(const CombineArgs& a, hipStream_t st);

// Backward of the combine's expert terms and of the permute (backward.hip).
struct CombineBackwardArgs {
  int N, d, k, dtype;
  const void* dy;
  const void* y_perm;
  const int32_t* row_of_slot;
  const float* topk_w;
  void* dy_perm;
  float* dtopk_w;
};
hipError_t launch_combine_backward(const CombineBackwardArgs& a, hipStream_t st);
hipError_t launch_permute_backward(int N, int d, int k, int dtype, const void* dx_perm,
                                   const int32_t* row_of_slot, void* dx, hipStream_t st);

// Backward of the expert FFN (backward_ffn.hip), bf16: plain row-major
// weights w1/w3 [E,h,d] and w2 [E,d,h]; fp32 weight gradients.
struct FfnBackwardArgs {
  int E, max_rows, d, h, act;
  const void* x_rows;
  const int32_t* offsets;
  const int32_t* group_rows;  // nullable: rows of each segment that hold data
  const void* w1;
  const void* w3;
  const void* w2;
  const void* dy_rows;
  void* dx_rows;
  float* dw1;
  float* dw3;
  float* dw2;
  void* ws;
};
size_t ffn_backward_workspace_bytes(int E, int max_rows, int d, int h, int act);
int ffn_backward_max_tiles(int E, int max_rows);
hipError_t launch_ffn_backward(const FfnBackwardArgs& a, hipStream_t st);
// The whole backward on packed weights: the GEMMs above, then the weight
// gradients from the row-major G and H.
hipError_t launch_ffn_backward_packed(const FfnBwdPackedArgs& a, float* dw1, float* dw3,
                                      float* dw2, hipStream_t st);

hipError_t launch_bias_update(int E, int N, int k, const int32_t* counts, float step,
                              float* sel_bias, hipStream_t st);

// Backward of the router and of the auxiliary load-balancing loss
// (router_backward.hip).
struct RouterBackwardArgs {
  int N, d, E, k, score_fn, dtype;
  const void* x;
  const void* w_router;
  const float* logits;
  const int32_t* topk_idx;
  const float* dtopk_w;
  const int32_t* counts;  // needed when aux_coef != 0
  float aux_coef;
  float* dlogits;         // nullable: then dz lives in ws
  float* dw_router;
  float* db;              // nullable
  void* dx;               // nullable
  int accumulate_dx;
  float* aux_loss;        // nullable
  void* ws;
};
size_t router_backward_workspace_bytes(int N, int d, int E);
hipError_t launch_router_backward(const RouterBackwardArgs& a, hipStream_t st);

}  // namespace moe
