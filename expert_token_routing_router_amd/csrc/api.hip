// api.hip -- the C ABI declared in include/moe.h: host-side validation, then
// the launches.  Nothing here allocates device memory or synchronises.
#include <math.h>

#include <mutex>

#include "../../include/moe.h"
#include "kernels.h"

namespace {

constexpr int kMaxExperts = 256;   // routing kernels: <= 4 experts per lane
constexpr int kMaxTopK = 8;        // per-token register arrays; int8 slot ids
constexpr int kMaxGroups = 64;     // group mask fits one 64-bit word
constexpr int kMaxFfnExperts = 1024;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Returns MOE_OK or the status describing what is wrong with desc.
int check_desc(const moe_route_desc* d) {
  if (!d) return MOE_ERR_INVALID_ARG;
  if (d->num_tokens < 0 || d->hidden < 1 || d->num_experts < 1 || d->top_k < 1)
    return MOE_ERR_INVALID_ARG;
  if (d->top_k > d->num_experts) return MOE_ERR_INVALID_ARG;
  if (d->num_ranks < 1 || d->num_experts % d->num_ranks != 0) return MOE_ERR_INVALID_ARG;
  if (d->num_groups < 1 || d->num_experts % d->num_groups != 0) return MOE_ERR_INVALID_ARG;
  if (d->topk_groups < 1 || d->topk_groups > d->num_groups) return MOE_ERR_INVALID_ARG;
  if ((long long)d->topk_groups * (d->num_experts / d->num_groups) < d->top_k)
    return MOE_ERR_INVALID_ARG;
  if (d->score_fn < MOE_SOFTMAX_TOPK || d->score_fn > MOE_SIGMOID_NORM) return MOE_ERR_INVALID_ARG;
  if (d->dtype != MOE_F32 && d->dtype != MOE_BF16) return MOE_ERR_INVALID_ARG;
  if (isnan(d->capacity_factor)) return MOE_ERR_INVALID_ARG;
  if ((long long)d->num_tokens * d->top_k > 0x7fffffffLL) return MOE_ERR_INVALID_ARG;
  if (d->hidden % 8 != 0) return MOE_ERR_UNSUPPORTED;
  if (d->num_experts > kMaxExperts || d->top_k > kMaxTopK || d->num_groups > kMaxGroups)
    return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

int32_t capacity_of(const moe_route_desc* d) {
  if (!(d->capacity_factor > 0.0f)) return 0x7fffffff;
  const double c = ceil((double)d->capacity_factor * ((double)d->num_tokens * d->top_k) /
                        (double)d->num_experts);
  return c > 2147483647.0 ? 0x7fffffff : (int32_t)c;
}

int status_of(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

}  // namespace

extern "C" {

const char* moe_status_string(int status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARG: return "invalid argument";
    case MOE_ERR_UNSUPPORTED: return "unsupported configuration";
    case MOE_ERR_HIP: return "HIP launch error";
    case MOE_ERR_WORKSPACE: return "workspace missing or too small";
    default: return "unknown status";
  }
}

size_t moe_route_workspace_size(const moe_route_desc* desc) {
  if (check_desc(desc) != MOE_OK) return 0;
  return moe::route_workspace_bytes(desc->num_tokens, desc->hidden, desc->num_experts,
                                    desc->dtype);
}

int moe_route(const moe_route_desc* desc, const void* x, const void* w_router,
              const float* router_bias, const float* sel_bias, float* logits,
              int32_t* topk_idx, float* topk_w, int32_t* counts, void* ws, size_t ws_bytes,
              void* stream) {
  int st = check_desc(desc);
  if (st != MOE_OK) return st;
  if (!counts) return MOE_ERR_INVALID_ARG;
  const int N = desc->num_tokens;
  if (N > 0) {
    if (!x || !w_router || !logits || !topk_idx || !topk_w) return MOE_ERR_INVALID_ARG;
    if (!aligned16(x)) return MOE_ERR_INVALID_ARG;
    const size_t need =
        moe::route_workspace_bytes(N, desc->hidden, desc->num_experts, desc->dtype);
    if (!ws || ws_bytes < need || (reinterpret_cast<uintptr_t>(ws) & 255u)) return MOE_ERR_WORKSPACE;
  }
  moe::RouteArgs a{N, desc->hidden, desc->num_experts, desc->top_k, desc->num_groups,
                   desc->topk_groups, desc->score_fn, desc->dtype, x, w_router, router_bias,
                   sel_bias, logits, topk_idx, topk_w, counts, ws};
  return status_of(moe::launch_route(a, static_cast<hipStream_t>(stream)));
}

int moe_router_logits(const moe_route_desc* desc, const void* x, const void* w_router,
                      const float* router_bias, float* logits, void* ws, size_t ws_bytes,
                      void* stream) {
  int st = check_desc(desc);
  if (st != MOE_OK) return st;
  const int N = desc->num_tokens;
  if (N == 0) return MOE_OK;
  if (!x || !w_router || !logits) return MOE_ERR_INVALID_ARG;
  if (!aligned16(x)) return MOE_ERR_INVALID_ARG;
  const size_t need = moe::route_workspace_bytes(N, desc->hidden, desc->num_experts, desc->dtype);
  if (!ws || ws_bytes < need || (reinterpret_cast<uintptr_t>(ws) & 255u)) return MOE_ERR_WORKSPACE;
  moe::RouteArgs a{N, desc->hidden, desc->num_experts, desc->top_k, desc->num_groups,
                   desc->topk_groups, desc->score_fn, desc->dtype, x, w_router, router_bias,
                   nullptr, logits, nullptr, nullptr, nullptr, ws};
  return status_of(moe::launch_router_logits(a, static_cast<hipStream_t>(stream)));
}

size_t moe_dispatch_workspace_size(const moe_route_desc* desc) {
  if (check_desc(desc) != MOE_OK) return 0;
  return moe::dispatch_workspace_bytes(desc->num_tokens, desc->top_k, desc->num_experts);
}

int moe_dispatch(const moe_route_desc* desc, const void* x, const int32_t* topk_idx,
                 void* x_perm, int32_t* row_of_slot, int32_t* token_of_row,
                 int8_t* slot_of_row, int32_t* expert_offsets, int32_t* admitted,
                 int32_t* rank_offsets, int32_t* rank_counts, void* ws, size_t ws_bytes,
                 void* stream) {
  return moe_dispatch_ex(desc, MOE_ADMIT_TOKEN_ORDER, x, topk_idx, x_perm, row_of_slot,
                         token_of_row, slot_of_row, expert_offsets, admitted, rank_offsets,
                         rank_counts, ws, ws_bytes, stream);
}

// The padded layout needs a finite capacity and E * cap rows addressable as int32.
static bool padded_layout_ok(const moe_route_desc* d) {
  if (!(d->capacity_factor > 0.f)) return false;
  return (long long)d->num_experts * capacity_of(d) <= 0x7fffffffLL;
}

// Shared by moe_dispatch_ex and moe_dispatch_q8: x_perm is the dtype rows or,
// with xq set, the INT8 payload rows (then x_perm must be NULL).
static int dispatch_common(const moe_route_desc* desc, int32_t admission, const void* x,
                           const int32_t* topk_idx, void* x_perm, int8_t* xq, float* row_scale,
                           int32_t* row_of_slot, int32_t* token_of_row, int8_t* slot_of_row,
                           int32_t* expert_offsets, int32_t* admitted, int32_t* rank_offsets,
                           int32_t* rank_counts, void* ws, size_t ws_bytes, void* stream,
                           int stages = moe::kDispatchLayout | moe::kDispatchPermute,
                           bool validate_only = false);

int moe_dispatch_ex(const moe_route_desc* desc, int32_t admission, const void* x,
                    const int32_t* topk_idx, void* x_perm, int32_t* row_of_slot,
                    int32_t* token_of_row, int8_t* slot_of_row, int32_t* expert_offsets,
                    int32_t* admitted, int32_t* rank_offsets, int32_t* rank_counts, void* ws,
                    size_t ws_bytes, void* stream) {
  return dispatch_common(desc, admission, x, topk_idx, x_perm, nullptr, nullptr, row_of_slot,
                         token_of_row, slot_of_row, expert_offsets, admitted, rank_offsets,
                         rank_counts, ws, ws_bytes, stream);
}

int moe_dispatch_q8(const moe_route_desc* desc, int32_t admission, const void* x,
                    const int32_t* topk_idx, int8_t* x_perm_q, float* row_scale,
                    int32_t* row_of_slot, int32_t* token_of_row, int8_t* slot_of_row,
                    int32_t* expert_offsets, int32_t* admitted, int32_t* rank_offsets,
                    int32_t* rank_counts, void* ws, size_t ws_bytes, void* stream) {
  if (desc && desc->num_tokens > 0) {
    if (!x_perm_q || !row_scale) return MOE_ERR_INVALID_ARG;
    if (!aligned16(x_perm_q) || (reinterpret_cast<uintptr_t>(row_scale) & 3u))
      return MOE_ERR_INVALID_ARG;
  }
  if (desc && (desc->dtype == MOE_F32 || desc->dtype == MOE_BF16) &&
      desc->hidden > moe::q8_max_hidden(desc->dtype))
    return MOE_ERR_UNSUPPORTED;
  return dispatch_common(desc, admission, x, topk_idx, nullptr, x_perm_q, row_scale, row_of_slot,
                         token_of_row, slot_of_row, expert_offsets, admitted, rank_offsets,
                         rank_counts, ws, ws_bytes, stream);
}

int moe_dequantize_q8(int32_t max_rows, int32_t hidden, int32_t dtype, const int8_t* x_perm_q,
                      const float* row_scale, const int32_t* num_rows, void* x_perm,
                      void* stream) {
  if (max_rows < 0 || hidden < 1 || (dtype != MOE_F32 && dtype != MOE_BF16))
    return MOE_ERR_INVALID_ARG;
  if (hidden % 8 != 0) return MOE_ERR_UNSUPPORTED;
  if (max_rows > 0) {
    if (!x_perm_q || !row_scale || !num_rows || !x_perm) return MOE_ERR_INVALID_ARG;
    if (!aligned16(x_perm_q) || !aligned16(x_perm) ||
        (reinterpret_cast<uintptr_t>(row_scale) & 3u) || (reinterpret_cast<uintptr_t>(num_rows) & 3u))
      return MOE_ERR_INVALID_ARG;
  }
  return status_of(moe::launch_dequantize_q8(max_rows, hidden, dtype, x_perm_q, row_scale,
                                             num_rows, x_perm, static_cast<hipStream_t>(stream)));
}

static int dispatch_common(const moe_route_desc* desc, int32_t admission, const void* x,
                           const int32_t* topk_idx, void* x_perm, int8_t* xq, float* row_scale,
                           int32_t* row_of_slot, int32_t* token_of_row, int8_t* slot_of_row,
                           int32_t* expert_offsets, int32_t* admitted, int32_t* rank_offsets,
                           int32_t* rank_counts, void* ws, size_t ws_bytes, void* stream,
                           int stages, bool validate_only) {
  int st = check_desc(desc);
  if (st != MOE_OK) return st;
  const bool layout = stages & moe::kDispatchLayout, permute = stages & moe::kDispatchPermute;
  const int N = desc->num_tokens;
  const int padded = (admission & MOE_LAYOUT_PADDED) ? 1 : 0;
  if (layout) {
    if (admission & ~(MOE_ADMIT_FIRST_CHOICE | MOE_LAYOUT_PADDED)) return MOE_ERR_INVALID_ARG;
    if (padded && !padded_layout_ok(desc)) return MOE_ERR_INVALID_ARG;
    if (!expert_offsets || !admitted || !rank_offsets || !rank_counts) return MOE_ERR_INVALID_ARG;
    if (N > 0 && (!topk_idx || !row_of_slot || !token_of_row || !slot_of_row))
      return MOE_ERR_INVALID_ARG;
  }
  if (permute && N > 0) {
    if (!x || !row_of_slot || !(x_perm || xq)) return MOE_ERR_INVALID_ARG;
    if (!aligned16(x) || (x_perm && !aligned16(x_perm))) return MOE_ERR_INVALID_ARG;
  }
  if (validate_only) return MOE_OK;  // every argument but the workspace checked
  if (layout) {
    const size_t need = moe::dispatch_workspace_bytes(N, desc->top_k, desc->num_experts);
    if (!ws || ws_bytes < need || (reinterpret_cast<uintptr_t>(ws) & 15u))
      return MOE_ERR_WORKSPACE;
  }
  moe::DispatchArgs a{N, desc->hidden, desc->num_experts, desc->top_k, desc->num_ranks,
                      desc->dtype, capacity_of(desc), x, topk_idx, x_perm, row_of_slot,
                      token_of_row, slot_of_row, expert_offsets, admitted, rank_offsets,
                      rank_counts, ws, (admission & MOE_ADMIT_FIRST_CHOICE) ? 1 : 0};
  a.xq = xq;
  a.row_scale = row_scale;
  a.padded = layout ? padded : 0;
  return status_of(moe::launch_dispatch(a, static_cast<hipStream_t>(stream), stages));
}

// ---------------------------------------------------- no-allocation dispatch --
//
// moe_dispatch_noalloc runs the dispatch kernels with their scratch (the
// per-tile, per-expert histograms and tile bases) in this file-scope device
// array instead of a caller workspace.  Each GPU the library runs on holds its
// own copy until the process ends.  Host code never passes the array's name
// to a kernel (on the host it is a stand-in, not a device address): the first
// call on a device, with that device current, looks its address up once with
// hipGetSymbolAddress and keeps it per device.  Every call on a device shares
// that device's array, so calls that overlap on one GPU race; each call
// writes every entry it reads before reading it, so nothing has to start at
// zero.
constexpr size_t kNoAllocScratchBytes = size_t(1) << 20;
constexpr int kNoAllocMaxDevices = 64;
static __device__ __align__(256) int32_t scratch[kNoAllocScratchBytes / sizeof(int32_t)];

static std::mutex g_scratch_mutex;
static void* g_scratch_ptr[kNoAllocMaxDevices];  // guarded by g_scratch_mutex

// This device's address of `scratch` (looked up on its first use), or an error.
static int noalloc_scratch(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return MOE_ERR_HIP;
  if (dev < 0 || dev >= kNoAllocMaxDevices) return MOE_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return MOE_ERR_HIP;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return MOE_OK;
}

int moe_dispatch_noalloc(const moe_route_desc* desc, int32_t admission, const void* x,
                         const int32_t* topk_idx, void* x_perm, int32_t* row_of_slot,
                         int32_t* token_of_row, int8_t* slot_of_row, int32_t* expert_offsets,
                         int32_t* admitted, int32_t* rank_offsets, int32_t* rank_counts,
                         void* stream) {
  int st = check_desc(desc);
  if (st != MOE_OK) return st;
  if (moe::dispatch_workspace_bytes(desc->num_tokens, desc->top_k, desc->num_experts) >
      kNoAllocScratchBytes)
    return MOE_ERR_UNSUPPORTED;  // the batch needs more scratch than the static array holds
  // Everything but the workspace is checked before the device is touched.
  st = dispatch_common(desc, admission, x, topk_idx, x_perm, nullptr, nullptr, row_of_slot,
                       token_of_row, slot_of_row, expert_offsets, admitted, rank_offsets,
                       rank_counts, nullptr, 0, stream,
                       moe::kDispatchLayout | moe::kDispatchPermute, true);
  if (st != MOE_OK) return st;
  void* ws = nullptr;
  if ((st = noalloc_scratch(&ws)) != MOE_OK) return st;
  return dispatch_common(desc, admission, x, topk_idx, x_perm, nullptr, nullptr, row_of_slot,
                         token_of_row, slot_of_row, expert_offsets, admitted, rank_offsets,
                         rank_counts, ws, kNoAllocScratchBytes, stream);
}

int64_t moe_dispatch_rows(const moe_route_desc* desc, int32_t admission) {
  if (check_desc(desc) != MOE_OK) return -1;
  if (admission & ~(MOE_ADMIT_FIRST_CHOICE | MOE_LAYOUT_PADDED)) return -1;
  const int padded = (admission & MOE_LAYOUT_PADDED) ? 1 : 0;
  if (padded && !padded_layout_ok(desc)) return -1;
  return (int64_t)moe::dispatch_rows(desc->num_tokens, desc->top_k, desc->num_experts,
                                     capacity_of(desc), padded);
}

int moe_dispatch_layout(const moe_route_desc* desc, int32_t admission, const int32_t* topk_idx,
                        int32_t* row_of_slot, int32_t* token_of_row, int8_t* slot_of_row,
                        int32_t* expert_offsets, int32_t* admitted, int32_t* rank_offsets,
                        int32_t* rank_counts, void* ws, size_t ws_bytes, void* stream) {
  return dispatch_common(desc, admission, nullptr, topk_idx, nullptr, nullptr, nullptr,
                         row_of_slot, token_of_row, slot_of_row, expert_offsets, admitted,
                         rank_offsets, rank_counts, ws, ws_bytes, stream,
                         moe::kDispatchLayout);
}

int moe_permute(const moe_route_desc* desc, const void* x, const int32_t* row_of_slot,
                void* x_perm, void* stream) {
  return dispatch_common(desc, MOE_ADMIT_TOKEN_ORDER, x, nullptr, x_perm, nullptr, nullptr,
                         const_cast<int32_t*>(row_of_slot), nullptr, nullptr, nullptr, nullptr,
                         nullptr, nullptr, nullptr, 0, stream, moe::kDispatchPermute);
}

int moe_permute_q8(const moe_route_desc* desc, const void* x, const int32_t* row_of_slot,
                   int8_t* x_perm_q, float* row_scale, void* stream) {
  if (desc && desc->num_tokens > 0) {
    if (!x_perm_q || !row_scale) return MOE_ERR_INVALID_ARG;
    if (!aligned16(x_perm_q) || (reinterpret_cast<uintptr_t>(row_scale) & 3u))
      return MOE_ERR_INVALID_ARG;
  }
  if (desc && (desc->dtype == MOE_F32 || desc->dtype == MOE_BF16) &&
      desc->hidden > moe::q8_max_hidden(desc->dtype))
    return MOE_ERR_UNSUPPORTED;
  return dispatch_common(desc, MOE_ADMIT_TOKEN_ORDER, x, nullptr, nullptr, x_perm_q, row_scale,
                         const_cast<int32_t*>(row_of_slot), nullptr, nullptr, nullptr, nullptr,
                         nullptr, nullptr, nullptr, 0, stream, moe::kDispatchPermute);
}

static int check_ffn(int32_t E, int32_t max_rows, int32_t d, int32_t h, int32_t act,
                     int32_t dtype) {
  if (E < 1 || max_rows < 0 || d < 1 || h < 1) return MOE_ERR_INVALID_ARG;
  if (act < MOE_RELU || act > MOE_SWIGLU) return MOE_ERR_INVALID_ARG;
  if (dtype != MOE_F32 && dtype != MOE_BF16) return MOE_ERR_INVALID_ARG;
  if (E > kMaxFfnExperts || d % 64 != 0 || h % 64 != 0) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

size_t moe_expert_ffn_workspace_size(int32_t num_experts, int32_t max_rows, int32_t hidden,
                                     int32_t ffn_hidden, int32_t act, int32_t dtype) {
  if (check_ffn(num_experts, max_rows, hidden, ffn_hidden, act, dtype) != MOE_OK) return 0;
  return moe::ffn_workspace_bytes(num_experts, max_rows, hidden, ffn_hidden, act, dtype);
}

// The fused combine argument of the down GEMM: sizes in range, every array
// present once there are rows and tokens, the accumulator 16-byte aligned.
static int check_fused(const moe_fused_combine* f, int32_t max_rows) {
  if (f->num_tokens < 0 || f->top_k < 1 || f->top_k > kMaxTopK) return MOE_ERR_INVALID_ARG;
  if (max_rows > 0 && (!f->token_of_row || !f->slot_of_row)) return MOE_ERR_INVALID_ARG;
  if (f->num_tokens > 0 && (!f->topk_w || !f->y_acc || !aligned16(f->y_acc)))
    return MOE_ERR_INVALID_ARG;
  return MOE_OK;
}

// Validation shared by moe_expert_ffn and its stages.  stage: 0 = all,
// 1 = plan, 2 = up, 3 = down.
static int check_ffn_call(int stage, int32_t E, int32_t max_rows, int32_t d, int32_t h,
                          int32_t act, int32_t dtype, const void* x_rows,
                          const int32_t* offsets, const void* w1, const void* w3,
                          const void* w2, const void* y_rows, const void* ws, size_t ws_bytes,
                          const moe_fused_combine* fused = nullptr) {
  int st = check_ffn(E, max_rows, d, h, act, dtype);
  if (st != MOE_OK) return st;
  if (!offsets) return MOE_ERR_INVALID_ARG;
  const bool up = stage == 0 || stage == 2, down = stage == 0 || stage == 3;
  if (up && (!w1 || (act == MOE_SWIGLU) != (w3 != nullptr))) return MOE_ERR_INVALID_ARG;
  if (down && !w2) return MOE_ERR_INVALID_ARG;
  if (down && fused && (st = check_fused(fused, max_rows)) != MOE_OK) return st;
  if (max_rows == 0) return MOE_OK;
  if (up && (!x_rows || !aligned16(x_rows) || !aligned16(w1) || (w3 && !aligned16(w3))))
    return MOE_ERR_INVALID_ARG;
  if (down && (!aligned16(w2) || (!fused && (!y_rows || !aligned16(y_rows)))))
    return MOE_ERR_INVALID_ARG;
  const size_t need = moe::ffn_workspace_bytes(E, max_rows, d, h, act, dtype);
  if (!ws || ws_bytes < need || (reinterpret_cast<uintptr_t>(ws) & 255u)) return MOE_ERR_WORKSPACE;
  return MOE_OK;
}

int moe_expert_ffn(int32_t num_experts, int32_t max_rows, int32_t hidden, int32_t ffn_hidden,
                   int32_t act, int32_t dtype, const void* x_rows,
                   const int32_t* group_offsets, const void* w1, const void* w3,
                   const void* w2, void* y_rows, const moe_fused_combine* fused, void* ws,
                   size_t ws_bytes, void* stream) {
  int st = check_ffn_call(0, num_experts, max_rows, hidden, ffn_hidden, act, dtype, x_rows,
                          group_offsets, w1, w3, w2, y_rows, ws, ws_bytes, fused);
  if (st != MOE_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  moe::FusedCombineArgs fc{};
  if (fused) fc = {fused->num_tokens, fused->top_k, fused->topk_w, fused->token_of_row,
                   fused->slot_of_row, fused->y_acc};
  if (max_rows == 0) {  // nothing to multiply; a fused call still leaves y_acc zeroed
    if (!fused || fused->num_tokens == 0) return MOE_OK;
    moe::FfnArgs z{num_experts, 0, hidden, ffn_hidden, act, dtype, nullptr, group_offsets,
                   nullptr, nullptr, w2, nullptr, nullptr, &fc};
    return status_of(moe::launch_ffn_zero_acc(z, s));
  }
  moe::FfnArgs a{num_experts, max_rows, hidden, ffn_hidden, act, dtype, x_rows,
                 group_offsets, w1, w3, w2, y_rows, ws, fused ? &fc : nullptr};
  hipError_t e = moe::launch_ffn_plan(a, s);
  if (e == hipSuccess) e = moe::launch_ffn_up(a, s);
  if (e == hipSuccess) e = moe::launch_ffn_down(a, s);
  return status_of(e);
}

// Backward of the expert FFN: bf16 only; d and h multiples of 32; at most
// 1024 experts; the 128-row tile list must fit a grid dimension.
static int check_ffn_backward(int32_t E, int32_t max_rows, int32_t d, int32_t h, int32_t act,
                              int32_t dtype) {
  if (E < 1 || max_rows < 0 || d < 1 || h < 1) return MOE_ERR_INVALID_ARG;
  if (act < MOE_RELU || act > MOE_SWIGLU) return MOE_ERR_INVALID_ARG;
  if (dtype != MOE_F32 && dtype != MOE_BF16) return MOE_ERR_INVALID_ARG;
  if (dtype != MOE_BF16 || E > 1024 || d % 32 != 0 || h % 32 != 0) return MOE_ERR_UNSUPPORTED;
  if (moe::ffn_backward_max_tiles(E, max_rows) > 65535) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

size_t moe_expert_ffn_backward_workspace_size(int32_t num_experts, int32_t max_rows,
                                              int32_t hidden, int32_t ffn_hidden, int32_t act,
                                              int32_t dtype) {
  if (check_ffn_backward(num_experts, max_rows, hidden, ffn_hidden, act, dtype) != MOE_OK)
    return 0;
  return moe::ffn_backward_workspace_bytes(num_experts, max_rows, hidden, ffn_hidden, act);
}

int moe_expert_ffn_backward(int32_t num_experts, int32_t max_rows, int32_t hidden,
                            int32_t ffn_hidden, int32_t act, int32_t dtype, const void* x_rows,
                            const int32_t* group_offsets, const int32_t* group_rows,
                            const void* w1, const void* w3, const void* w2, const void* dy_rows,
                            void* dx_rows, float* dw1, float* dw3, float* dw2, void* ws,
                            size_t ws_bytes, void* stream) {
  int st = check_ffn_backward(num_experts, max_rows, hidden, ffn_hidden, act, dtype);
  if (st != MOE_OK) return st;
  const bool swiglu = act == MOE_SWIGLU;
  if (!group_offsets || !w1 || !w2 || !dw1 || !dw2) return MOE_ERR_INVALID_ARG;
  if (swiglu != (w3 != nullptr) || swiglu != (dw3 != nullptr)) return MOE_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(group_offsets) & 3u) ||
      (reinterpret_cast<uintptr_t>(group_rows) & 3u) || !aligned16(w1) || !aligned16(w2) ||
      (w3 && !aligned16(w3)) || !aligned16(dw1) || !aligned16(dw2) || (dw3 && !aligned16(dw3)))
    return MOE_ERR_INVALID_ARG;
  if (max_rows > 0) {
    if (!x_rows || !dy_rows || !dx_rows) return MOE_ERR_INVALID_ARG;
    if (!aligned16(x_rows) || !aligned16(dy_rows) || !aligned16(dx_rows))
      return MOE_ERR_INVALID_ARG;
    const size_t need = moe::ffn_backward_workspace_bytes(num_experts, max_rows, hidden,
                                                          ffn_hidden, act);
    if (!ws || ws_bytes < need || (reinterpret_cast<uintptr_t>(ws) & 255u))
      return MOE_ERR_WORKSPACE;
  }
  moe::FfnBackwardArgs a{num_experts, max_rows, hidden, ffn_hidden, act, x_rows, group_offsets,
                         group_rows, w1, w3, w2, dy_rows, dx_rows, dw1, dw3, dw2, ws};
  return status_of(moe::launch_ffn_backward(a, static_cast<hipStream_t>(stream)));
}

// Backward on packed weights: the forward GEMM's shape limits (d, h multiples
// of 64, E <= 1024) besides the backward's own.
static int check_ffn_backward_packed(int32_t E, int32_t max_rows, int32_t d, int32_t h,
                                     int32_t act, int32_t dtype) {
  const int st = check_ffn_backward(E, max_rows, d, h, act, dtype);
  if (st != MOE_OK) return st;
  if (E > kMaxFfnExperts || d % 64 != 0 || h % 64 != 0) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

size_t moe_expert_ffn_backward_packed_workspace_size(int32_t num_experts, int32_t max_rows,
                                                     int32_t hidden, int32_t ffn_hidden,
                                                     int32_t act, int32_t dtype) {
  if (check_ffn_backward_packed(num_experts, max_rows, hidden, ffn_hidden, act, dtype) != MOE_OK)
    return 0;
  return moe::ffn_bwd_packed_workspace_bytes(num_experts, max_rows, hidden, ffn_hidden, act);
}

int moe_expert_ffn_backward_packed(int32_t num_experts, int32_t max_rows, int32_t hidden,
                                   int32_t ffn_hidden, int32_t act, int32_t dtype,
                                   const void* x_rows, const int32_t* group_offsets,
                                   const int32_t* group_rows, const void* w1_packed,
                                   const void* w3_packed, const void* w2t_packed,
                                   const void* w13t_packed, const void* dy_rows, void* dx_rows,
                                   float* dw1, float* dw3, float* dw2, void* ws, size_t ws_bytes,
                                   void* stream) {
  int st = check_ffn_backward_packed(num_experts, max_rows, hidden, ffn_hidden, act, dtype);
  if (st != MOE_OK) return st;
  const bool swiglu = act == MOE_SWIGLU;
  if (!group_offsets || !w1_packed || !w2t_packed || !w13t_packed || !dw1 || !dw2)
    return MOE_ERR_INVALID_ARG;
  if (swiglu != (w3_packed != nullptr) || swiglu != (dw3 != nullptr)) return MOE_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(group_offsets) & 3u) ||
      (reinterpret_cast<uintptr_t>(group_rows) & 3u) || !aligned16(w1_packed) ||
      (w3_packed && !aligned16(w3_packed)) || !aligned16(w2t_packed) ||
      !aligned16(w13t_packed) || !aligned16(dw1) || !aligned16(dw2) || (dw3 && !aligned16(dw3)))
    return MOE_ERR_INVALID_ARG;
  if (max_rows > 0) {
    if (!x_rows || !dy_rows || !dx_rows) return MOE_ERR_INVALID_ARG;
    if (!aligned16(x_rows) || !aligned16(dy_rows) || !aligned16(dx_rows))
      return MOE_ERR_INVALID_ARG;
    const size_t need = moe::ffn_bwd_packed_workspace_bytes(num_experts, max_rows, hidden,
                                                            ffn_hidden, act);
    if (!ws || ws_bytes < need || (reinterpret_cast<uintptr_t>(ws) & 255u))
      return MOE_ERR_WORKSPACE;
  }
  moe::FfnBwdPackedArgs a{num_experts, max_rows, hidden, ffn_hidden, act, x_rows,
                          group_offsets, group_rows, w1_packed, w3_packed, w2t_packed,
                          w13t_packed, dy_rows, dx_rows, ws};
  return status_of(
      moe::launch_ffn_backward_packed(a, dw1, dw3, dw2, static_cast<hipStream_t>(stream)));
}

int moe_expert_ffn_plan(int32_t num_experts, int32_t max_rows, int32_t hidden,
                        int32_t ffn_hidden, int32_t act, int32_t dtype,
                        const int32_t* group_offsets, void* ws, size_t ws_bytes, void* stream) {
  int st = check_ffn_call(1, num_experts, max_rows, hidden, ffn_hidden, act, dtype, nullptr,
                          group_offsets, nullptr, nullptr, nullptr, nullptr, ws, ws_bytes);
  if (st != MOE_OK || max_rows == 0) return st;
  moe::FfnArgs a{num_experts, max_rows, hidden, ffn_hidden, act, dtype, nullptr,
                 group_offsets, nullptr, nullptr, nullptr, nullptr, ws};
  return status_of(moe::launch_ffn_plan(a, static_cast<hipStream_t>(stream)));
}

int moe_expert_ffn_up(int32_t num_experts, int32_t max_rows, int32_t hidden, int32_t ffn_hidden,
                      int32_t act, int32_t dtype, const void* x_rows,
                      const int32_t* group_offsets, const void* w1, const void* w3,
                      void* ws, size_t ws_bytes, void* stream) {
  int st = check_ffn_call(2, num_experts, max_rows, hidden, ffn_hidden, act, dtype, x_rows,
                          group_offsets, w1, w3, nullptr, nullptr, ws, ws_bytes);
  if (st != MOE_OK || max_rows == 0) return st;
  moe::FfnArgs a{num_experts, max_rows, hidden, ffn_hidden, act, dtype, x_rows,
                 group_offsets, w1, w3, nullptr, nullptr, ws};
  return status_of(moe::launch_ffn_up(a, static_cast<hipStream_t>(stream)));
}

int moe_expert_ffn_down(int32_t num_experts, int32_t max_rows, int32_t hidden,
                        int32_t ffn_hidden, int32_t act, int32_t dtype,
                        const int32_t* group_offsets, const void* w2, void* y_rows,
                        const moe_fused_combine* fused, void* ws, size_t ws_bytes,
                        void* stream) {
  int st = check_ffn_call(3, num_experts, max_rows, hidden, ffn_hidden, act, dtype, nullptr,
                          group_offsets, nullptr, nullptr, w2, y_rows, ws, ws_bytes, fused);
  if (st != MOE_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  moe::FusedCombineArgs fc{};
  if (fused) fc = {fused->num_tokens, fused->top_k, fused->topk_w, fused->token_of_row,
                   fused->slot_of_row, fused->y_acc};
  moe::FfnArgs a{num_experts, max_rows, hidden, ffn_hidden, act, dtype, nullptr,
                 group_offsets, nullptr, nullptr, w2, y_rows, ws, fused ? &fc : nullptr};
  if (max_rows == 0) {
    if (!fused || fused->num_tokens == 0) return MOE_OK;
    return status_of(moe::launch_ffn_zero_acc(a, s));
  }
  return status_of(moe::launch_ffn_down(a, s));
}

int moe_expert_ffn_pack_weights(int32_t num_experts, int32_t rows, int32_t cols, int32_t dtype,
                                const void* w, void* w_packed, void* stream) {
  if (num_experts < 1 || rows < 1 || cols < 1) return MOE_ERR_INVALID_ARG;
  if (dtype != MOE_F32 && dtype != MOE_BF16) return MOE_ERR_INVALID_ARG;
  if (dtype != MOE_BF16 || rows % 64 != 0 || cols % 64 != 0) return MOE_ERR_UNSUPPORTED;
  if (!w || !w_packed || !aligned16(w) || !aligned16(w_packed)) return MOE_ERR_INVALID_ARG;
  const size_t bytes = (size_t)num_experts * rows * cols * 2;
  const char* a0 = static_cast<const char*>(w);
  const char* b0 = static_cast<const char*>(w_packed);
  if (a0 < b0 + bytes && b0 < a0 + bytes) return MOE_ERR_INVALID_ARG;  // must not overlap
  return status_of(moe::launch_pack_weights(num_experts, rows, cols, w, w_packed,
                                            static_cast<hipStream_t>(stream)));
}

int moe_expert_ffn_pack_weights_t(int32_t num_experts, int32_t rows, int32_t cols_a,
                                  int32_t cols, int32_t dtype, const void* wa, const void* wb,
                                  void* w_packed, void* stream) {
  if (num_experts < 1 || rows < 1 || cols < 1 || cols_a < 1 || cols_a > cols)
    return MOE_ERR_INVALID_ARG;
  if (dtype != MOE_F32 && dtype != MOE_BF16) return MOE_ERR_INVALID_ARG;
  if (dtype != MOE_BF16 || rows % 64 != 0 || cols % 64 != 0 || cols_a % 8 != 0)
    return MOE_ERR_UNSUPPORTED;
  if (!wa || !w_packed || !aligned16(wa) || !aligned16(w_packed)) return MOE_ERR_INVALID_ARG;
  if ((cols_a < cols) != (wb != nullptr) || (wb && !aligned16(wb))) return MOE_ERR_INVALID_ARG;
  const size_t bytes = (size_t)num_experts * rows * cols * 2;
  const char* b0 = static_cast<const char*>(w_packed);
  const char* a0 = static_cast<const char*>(wa);
  const size_t abytes = (size_t)num_experts * rows * cols_a * 2;
  if (a0 < b0 + bytes && b0 < a0 + abytes) return MOE_ERR_INVALID_ARG;  // must not overlap
  if (wb) {
    const char* c0 = static_cast<const char*>(wb);
    const size_t cbytes = (size_t)num_experts * rows * (cols - cols_a) * 2;
    if (c0 < b0 + bytes && b0 < c0 + cbytes) return MOE_ERR_INVALID_ARG;
  }
  return status_of(moe::launch_pack_weights_t(num_experts, rows, cols_a, cols, wa, wb, w_packed,
                                              static_cast<hipStream_t>(stream)));
}

int moe_combine(const moe_route_desc* desc, const void* y_perm, const int32_t* row_of_slot,
                const float* topk_w, const void* residual, const void* shared_out,
                const float* y_acc, void* y, void* stream) {
  int st = check_desc(desc);
  if (st != MOE_OK) return st;
  const int N = desc->num_tokens;
  if (N == 0) return MOE_OK;
  if (!y) return MOE_ERR_INVALID_ARG;
  if (y_acc) {
    if (!aligned16(y_acc)) return MOE_ERR_INVALID_ARG;
  } else {
    if (!y_perm || !row_of_slot || !topk_w || !aligned16(y_perm)) return MOE_ERR_INVALID_ARG;
  }
  if (!aligned16(y) || (residual && !aligned16(residual)) ||
      (shared_out && !aligned16(shared_out)))
    return MOE_ERR_INVALID_ARG;
  moe::CombineArgs a{N, desc->hidden, desc->top_k, desc->dtype, y_perm, row_of_slot, topk_w,
                     residual, shared_out, y, y_acc};
  return status_of(moe::launch_combine(a, static_cast<hipStream_t>(stream)));
}

int moe_combine_backward(const moe_route_desc* desc, const void* dy, const void* y_perm,
                         const int32_t* row_of_slot, const float* topk_w, void* dy_perm,
                         float* dtopk_w, void* stream) {
  int st = check_desc(desc);
  if (st != MOE_OK) return st;
  const int N = desc->num_tokens;
  if (N > 0) {
    if (!dy || !y_perm || !row_of_slot || !topk_w || !dy_perm || !dtopk_w)
      return MOE_ERR_INVALID_ARG;
    if (!aligned16(dy) || !aligned16(y_perm) || !aligned16(dy_perm) ||
        (reinterpret_cast<uintptr_t>(dtopk_w) & 3u))
      return MOE_ERR_INVALID_ARG;
  }
  moe::CombineBackwardArgs a{N, desc->hidden, desc->top_k, desc->dtype, dy, y_perm,
                             row_of_slot, topk_w, dy_perm, dtopk_w};
  return status_of(moe::launch_combine_backward(a, static_cast<hipStream_t>(stream)));
}

int moe_permute_backward(const moe_route_desc* desc, const void* dx_perm,
                         const int32_t* row_of_slot, void* dx, void* stream) {
  int st = check_desc(desc);
  if (st != MOE_OK) return st;
  const int N = desc->num_tokens;
  if (N > 0) {
    if (!dx_perm || !row_of_slot || !dx) return MOE_ERR_INVALID_ARG;
    if (!aligned16(dx_perm) || !aligned16(dx)) return MOE_ERR_INVALID_ARG;
  }
  return status_of(moe::launch_permute_backward(N, desc->hidden, desc->top_k, desc->dtype,
                                                dx_perm, row_of_slot, dx,
                                                static_cast<hipStream_t>(stream)));
}

size_t moe_router_backward_workspace_size(const moe_route_desc* desc) {
  if (check_desc(desc) != MOE_OK) return 0;
  return moe::router_backward_workspace_bytes(desc->num_tokens, desc->hidden, desc->num_experts);
}

int moe_router_backward(const moe_route_desc* desc, const void* x, const void* w_router,
                        const float* logits, const int32_t* topk_idx, const float* dtopk_w,
                        const int32_t* counts, float aux_coef, float* dlogits, float* dw_router,
                        float* drouter_bias, void* dx, int32_t accumulate_dx, float* aux_loss,
                        void* ws, size_t ws_bytes, void* stream) {
  int st = check_desc(desc);
  if (st != MOE_OK) return st;
  if (!isfinite(aux_coef)) return MOE_ERR_INVALID_ARG;
  if (!dw_router || (aux_coef != 0.f && !counts)) return MOE_ERR_INVALID_ARG;
  const int N = desc->num_tokens;
  const auto al4 = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; };
  if (!al4(dw_router) || !al4(drouter_bias) || !al4(aux_loss) || !al4(dlogits) || !al4(counts))
    return MOE_ERR_INVALID_ARG;
  if (N > 0) {
    if (!x || !w_router || !logits || !topk_idx || !dtopk_w) return MOE_ERR_INVALID_ARG;
    if (!al4(logits) || !al4(topk_idx) || !al4(dtopk_w) || (dx && !aligned16(dx)))
      return MOE_ERR_INVALID_ARG;
    const size_t need = moe::router_backward_workspace_bytes(N, desc->hidden, desc->num_experts);
    if (!ws || ws_bytes < need || (reinterpret_cast<uintptr_t>(ws) & 255u)) return MOE_ERR_WORKSPACE;
  }
  moe::RouterBackwardArgs a{N, desc->hidden, desc->num_experts, desc->top_k, desc->score_fn,
                            desc->dtype, x, w_router, logits, topk_idx, dtopk_w, counts,
                            aux_coef, dlogits, dw_router, drouter_bias, dx,
                            accumulate_dx ? 1 : 0, aux_loss, ws};
  return status_of(moe::launch_router_backward(a, static_cast<hipStream_t>(stream)));
}

int moe_bias_update(int32_t num_experts, int32_t num_tokens, int32_t top_k,
                    const int32_t* counts, float step, float* sel_bias, void* stream) {
  if (num_experts < 1 || num_tokens < 0 || top_k < 1 || !counts || !sel_bias)
    return MOE_ERR_INVALID_ARG;
  if (!isfinite(step)) return MOE_ERR_INVALID_ARG;
  return status_of(moe::launch_bias_update(num_experts, num_tokens, top_k, counts, step,
                                           sel_bias, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
