// combine.hip -- weighted combine back to token order, and the selection-bias
// update, for gfx950.
//
// Combine: glossary "Expert Parallelism", step 4 of "How tokens travel between
// GPUs" (expert outputs come back to the token, weighted by the router scores
// and summed) and "Load balancing and capacity" (a skipped token passes
// through the residual connection unchanged).  One wave per token gathers its
// k expert rows with 16-byte vector loads, accumulates residual + shared +
// sum_j w_j * row_j in fp32 in that order, and rounds once.
//
// Bias update: same page, bias-based balancing bullet (after each step, lower
// the bias of overloaded experts, raise it for idle ones).
#include "device.h"
#include "kernels.h"

namespace moe {

template <int DTYPE>  // 0 fp32 (4 per vector), 1 bf16 (8 per vector)
__global__ __launch_bounds__(256) void combine_rows(const u32x4* __restrict__ y_perm,
                                                    const int32_t* __restrict__ row_of_slot,
                                                    const float* __restrict__ topk_w,
                                                    const u32x4* __restrict__ residual,
                                                    const u32x4* __restrict__ shared_out,
                                                    u32x4* __restrict__ y, int N, int vec_per_row,
                                                    int k) {
  constexpr int VE = DTYPE == 0 ? 4 : 8;  // elements per 16-byte vector
  const int lane = threadIdx.x % 64;
  const int gw = blockIdx.x * 4 + threadIdx.x / 64;
  const int nw = gridDim.x * 4;
  for (int t = gw; t < N; t += nw) {
    const int my_row = lane < k ? row_of_slot[(size_t)t * k + lane] : -1;
    const float my_w = lane < k ? topk_w[(size_t)t * k + lane] : 0.f;
    int rows[8];
    float ws[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      rows[j] = __shfl(my_row, j, 64);
      ws[j] = __shfl(my_w, j, 64);
    }
    for (int v = lane; v < vec_per_row; v += 64) {
      float acc[VE];
      const size_t tv = (size_t)t * vec_per_row + v;
      auto add_vec = [&](const u32x4 q, float scale, bool first) {
        const uint32_t w4[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if constexpr (DTYPE == 0) {
            const float f = __uint_as_float(w4[i]);
            acc[i] = first ? f * scale : __fmaf_rn(f, scale, acc[i]);
          } else {
            const float lo = bf16_to_f32(w4[i] & 0xffffu), hi = bf16_to_f32(w4[i] >> 16);
            acc[2 * i] = first ? lo * scale : __fmaf_rn(lo, scale, acc[2 * i]);
            acc[2 * i + 1] = first ? hi * scale : __fmaf_rn(hi, scale, acc[2 * i + 1]);
          }
        }
      };
#pragma unroll
      for (int i = 0; i < VE; ++i) acc[i] = 0.f;
      if (residual) add_vec(residual[tv], 1.f, true);
      if (shared_out) add_vec(shared_out[tv], 1.f, false);
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (j < k && rows[j] >= 0) add_vec(y_perm[(size_t)rows[j] * vec_per_row + v], ws[j], false);
      u32x4 out;
      uint32_t o4[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if constexpr (DTYPE == 0) o4[i] = __float_as_uint(acc[i]);
        else o4[i] = pack_bf16x2(acc[2 * i], acc[2 * i + 1]);
      }
      out.x = o4[0];
      out.y = o4[1];
      out.z = o4[2];
      out.w = o4[3];
      y[tv] = out;
    }
  }
}

hipError_t launch_combine(const CombineArgs& a, hipStream_t st) {
  if (a.N == 0) return hipSuccess;
  const int elem = a.dtype == 0 ? 4 : 2;
  const int vec_per_row = a.d * elem / 16;
  const int blocks = std::max(1, std::min((a.N + 3) / 4, 8192));
  auto yp = static_cast<const u32x4*>(a.y_perm);
  auto res = static_cast<const u32x4*>(a.residual);
  auto sh = static_cast<const u32x4*>(a.shared_out);
  auto y = static_cast<u32x4*>(a.y);
  if (a.dtype == 0)
    combine_rows<0><<<blocks, 256, 0, st>>>(yp, a.row_of_slot, a.topk_w, res, sh, y, a.N,
                                            vec_per_row, a.k);
  else
    combine_rows<1><<<blocks, 256, 0, st>>>(yp, a.row_of_slot, a.topk_w, res, sh, y, a.N,
                                            vec_per_row, a.k);
  return hipGetLastError();
}

// Load is compared with the mean N*k/E in integers: counts[e]*E vs N*k.
__global__ void bias_update_kernel(int E, long long nk, const int32_t* __restrict__ counts,
                                   float step, float* __restrict__ sel_bias) {
  for (int e = blockIdx.x * blockDim.x + threadIdx.x; e < E; e += gridDim.x * blockDim.x) {
    const long long load = (long long)counts[e] * E;
    if (load > nk) sel_bias[e] = sel_bias[e] - step;
    else if (load < nk) sel_bias[e] = sel_bias[e] + step;
  }
}

hipError_t launch_bias_update(int E, int N, int k, const int32_t* counts, float step,
                              float* sel_bias, hipStream_t st) {
  bias_update_kernel<<<(E + 255) / 256, 256, 0, st>>>(E, (long long)N * k, counts, step,
                                                      sel_bias);
  return hipGetLastError();
}

}  // namespace moe
