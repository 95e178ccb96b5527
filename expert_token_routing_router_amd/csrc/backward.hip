// backward.hip -- backward of the layer's data path on gfx950: the combine's
// expert terms and the permute, read backwards (the four steps of the
// glossary "Expert Parallelism", "How tokens travel between GPUs", in reverse
// order for a training step).
//
// combine:  y[t] = residual[t] + shared[t] + sum_j w_tj y_perm[r_tj]
//   => dy_perm[r_tj] = w_tj dy[t]      (fp32 product, rounded once to the dtype)
//      dtopk_w[t, j] = <dy[t], y_perm[r_tj]>  (exact products summed in fp64
//                                              per lane, then over the wave)
//      (the residual and shared terms pass dy on unchanged: nothing to run)
// permute:  x_perm[r_tj] = x[t]
//   => dx[t] = sum_j dx_perm[r_tj]     (fp32, in slot order, rounded once)
//
// Both are row gathers / scatters, one wave per token with 16-byte vectors:
// HBM-bound, like the forward permute and combine.
#include "device.h"
#include "kernels.h"

namespace moe {

template <int DTYPE>  // 0 fp32 (4 per vector), 1 bf16 (8 per vector)
__global__ __launch_bounds__(256) void combine_backward_rows(
    const u32x4* __restrict__ dy, const u32x4* __restrict__ y_perm,
    const int32_t* __restrict__ row_of_slot, const float* __restrict__ topk_w,
    u32x4* __restrict__ dy_perm, float* __restrict__ dtopk_w, int N, int vec_per_row, int k) {
  const int lane = threadIdx.x % 64;
  const int gw = blockIdx.x * 4 + threadIdx.x / 64;
  const int nw = gridDim.x * 4;
  for (int t = gw; t < N; t += nw) {
    const int my_row = lane < k ? row_of_slot[(size_t)t * k + lane] : -1;
    const float my_w = lane < k ? topk_w[(size_t)t * k + lane] : 0.f;
    const u32x4* g = dy + (size_t)t * vec_per_row;
    double my_dot = 0.0;
    for (int j = 0; j < k; ++j) {
      const int r = __shfl(my_row, j, 64);  // uniform
      if (r < 0) continue;
      const float w = __shfl(my_w, j, 64);
      const u32x4* yp = y_perm + (size_t)r * vec_per_row;
      u32x4* out = dy_perm + (size_t)r * vec_per_row;
      double part = 0.0;
      for (int v = lane; v < vec_per_row; v += 64) {
        const u32x4 gv = g[v], yv = yp[v];
        u32x4 o;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          if constexpr (DTYPE == 0) {
            const float a = __uint_as_float(gv[c]), b = __uint_as_float(yv[c]);
            part += (double)a * (double)b;
            o[c] = __float_as_uint(w * a);
          } else {
            const float a0 = bf16_to_f32(gv[c] & 0xffffu), a1 = bf16_to_f32(gv[c] >> 16);
            const float b0 = bf16_to_f32(yv[c] & 0xffffu), b1 = bf16_to_f32(yv[c] >> 16);
            part += (double)(a0 * b0) + (double)(a1 * b1);  // bf16 x bf16 is exact in fp32
            o[c] = pack_bf16x2(w * a0, w * a1);
          }
        }
        out[v] = o;
      }
      const double dot = wave_sum(part);
      if (lane == j) my_dot = dot;
    }
    if (lane < k) dtopk_w[(size_t)t * k + lane] = my_row >= 0 ? (float)my_dot : 0.f;
  }
}

template <int DTYPE>
__global__ __launch_bounds__(256) void permute_backward_rows(
    const u32x4* __restrict__ dx_perm, const int32_t* __restrict__ row_of_slot,
    u32x4* __restrict__ dx, int N, int vec_per_row, int k) {
  constexpr int VE = DTYPE == 0 ? 4 : 8;
  const int lane = threadIdx.x % 64;
  const int gw = blockIdx.x * 4 + threadIdx.x / 64;
  const int nw = gridDim.x * 4;
  for (int t = gw; t < N; t += nw) {
    const int my_row = lane < k ? row_of_slot[(size_t)t * k + lane] : -1;
    int rows[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) rows[j] = __shfl(my_row, j, 64);
    for (int v = lane; v < vec_per_row; v += 64) {
      float acc[VE];
#pragma unroll
      for (int i = 0; i < VE; ++i) acc[i] = 0.f;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        if (j < k && rows[j] >= 0) {
          const u32x4 q = dx_perm[(size_t)rows[j] * vec_per_row + v];
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            if constexpr (DTYPE == 0) {
              acc[c] += __uint_as_float(q[c]);
            } else {
              acc[2 * c] += bf16_to_f32(q[c] & 0xffffu);
              acc[2 * c + 1] += bf16_to_f32(q[c] >> 16);
            }
          }
        }
      }
      u32x4 o;
      if constexpr (DTYPE == 0) {
        o = u32x4{__float_as_uint(acc[0]), __float_as_uint(acc[1]), __float_as_uint(acc[2]),
                  __float_as_uint(acc[3])};
      } else {
        o = u32x4{pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]),
                  pack_bf16x2(acc[4], acc[5]), pack_bf16x2(acc[6], acc[7])};
      }
      dx[(size_t)t * vec_per_row + v] = o;
    }
  }
}

static int row_blocks(int N) { return std::max(1, std::min((N + 3) / 4, 8192)); }

hipError_t launch_combine_backward(const CombineBackwardArgs& a, hipStream_t st) {
  if (a.N == 0) return hipSuccess;
  const int vec_per_row = a.d * (a.dtype == 0 ? 4 : 2) / 16;
  auto dy = static_cast<const u32x4*>(a.dy);
  auto yp = static_cast<const u32x4*>(a.y_perm);
  auto out = static_cast<u32x4*>(a.dy_perm);
  if (a.dtype == 0)
    combine_backward_rows<0><<<row_blocks(a.N), 256, 0, st>>>(dy, yp, a.row_of_slot, a.topk_w,
                                                              out, a.dtopk_w, a.N, vec_per_row, a.k);
  else
    combine_backward_rows<1><<<row_blocks(a.N), 256, 0, st>>>(dy, yp, a.row_of_slot, a.topk_w,
                                                              out, a.dtopk_w, a.N, vec_per_row, a.k);
  return hipGetLastError();
}

hipError_t launch_permute_backward(int N, int d, int k, int dtype, const void* dx_perm,
                                   const int32_t* row_of_slot, void* dx, hipStream_t st) {
  if (N == 0) return hipSuccess;
  const int vec_per_row = d * (dtype == 0 ? 4 : 2) / 16;
  auto in = static_cast<const u32x4*>(dx_perm);
  auto out = static_cast<u32x4*>(dx);
  if (dtype == 0)
    permute_backward_rows<0><<<row_blocks(N), 256, 0, st>>>(in, row_of_slot, out, N,
                                                           vec_per_row, k);
  else
    permute_backward_rows<1><<<row_blocks(N), 256, 0, st>>>(in, row_of_slot, out, N,
                                                           vec_per_row, k);
  return hipGetLastError();
}

}  // namespace moe
