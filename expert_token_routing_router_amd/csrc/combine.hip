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
#include <type_traits>

#include "device.h"
#include "kernels.h"

namespace moe {

// V 16-byte vectors per lane and stream are in flight per pass (V = 2 for
// rows longer than 128 vectors; measured on MI355X: 46 -> 41 us for
// d = 4096, 141 -> 134 us for d = 7168, while one vector keeps the
// occupancy d = 1024 needs), and the next token's row ids and weights are
// loaded while the current token's rows move.
// KM: slots per token the kernel holds rows for (k <= KM).
template <int DTYPE, int V, int KM>  // DTYPE 0 fp32 (4 per vector), 1 bf16 (8 per vector)
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
  auto add_vec = [&](float* acc, const u32x4 q, float scale) {
    const uint32_t w4[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if constexpr (DTYPE == 0) {
        acc[i] = __fmaf_rn(__uint_as_float(w4[i]), scale, acc[i]);
      } else {
        acc[2 * i] = __fmaf_rn(bf16_to_f32(w4[i] & 0xffffu), scale, acc[2 * i]);
        acc[2 * i + 1] = __fmaf_rn(bf16_to_f32(w4[i] >> 16), scale, acc[2 * i + 1]);
      }
    }
  };
  int next_row = gw < N && lane < k ? row_of_slot[(size_t)gw * k + lane] : -1;
  float next_w = gw < N && lane < k ? topk_w[(size_t)gw * k + lane] : 0.f;
  for (int t = gw; t < N; t += nw) {
    const int my_row = next_row;
    const float my_w = next_w;
    const int tn = t + nw;
    next_row = tn < N && lane < k ? row_of_slot[(size_t)tn * k + lane] : -1;
    next_w = tn < N && lane < k ? topk_w[(size_t)tn * k + lane] : 0.f;
    int rows[8];
    float ws[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      rows[j] = __shfl(my_row, j, 64);
      ws[j] = __shfl(my_w, j, 64);
    }
    for (int v0 = 0; v0 < vec_per_row; v0 += V * 64) {
      const size_t tv0 = (size_t)t * vec_per_row + v0 + lane;
      // Every load of this chunk first (residual, shared, the k expert rows),
      // then the adds in the fixed order: one memory round trip per chunk.
      u32x4 qr[V], qs[V], qy[KM][V];
#pragma unroll
      for (int u = 0; u < V; ++u) {
        const bool in = v0 + u * 64 + lane < vec_per_row;
        if (residual && in) qr[u] = residual[tv0 + u * 64];
        if (shared_out && in) qs[u] = shared_out[tv0 + u * 64];
      }
#pragma unroll
      for (int j = 0; j < KM; ++j) {
        if (j < k && rows[j] >= 0) {
          const u32x4* src = y_perm + (size_t)rows[j] * vec_per_row + v0 + lane;
#pragma unroll
          for (int u = 0; u < V; ++u)
            if (v0 + u * 64 + lane < vec_per_row) qy[j][u] = src[u * 64];
        }
      }
      float acc[V][VE];
#pragma unroll
      for (int u = 0; u < V; ++u) {
#pragma unroll
        for (int i = 0; i < VE; ++i) acc[u][i] = 0.f;
      }
      // residual + shared + sum_j w_j row_j, in that order (a skipped slot
      // adds nothing).
#pragma unroll
      for (int u = 0; u < V; ++u) {
        if (v0 + u * 64 + lane < vec_per_row) {
          if (residual) add_vec(acc[u], qr[u], 1.f);
          if (shared_out) add_vec(acc[u], qs[u], 1.f);
        }
      }
#pragma unroll
      for (int j = 0; j < KM; ++j) {
        if (j < k && rows[j] >= 0) {
#pragma unroll
          for (int u = 0; u < V; ++u)
            if (v0 + u * 64 + lane < vec_per_row) add_vec(acc[u], qy[j][u], ws[j]);
        }
      }
#pragma unroll
      for (int u = 0; u < V; ++u) {
        if (v0 + u * 64 + lane < vec_per_row) {
          u32x4 out;
          if constexpr (DTYPE == 0) {
            out = u32x4{__float_as_uint(acc[u][0]), __float_as_uint(acc[u][1]),
                        __float_as_uint(acc[u][2]), __float_as_uint(acc[u][3])};
          } else {
            out = u32x4{pack_bf16x2(acc[u][0], acc[u][1]), pack_bf16x2(acc[u][2], acc[u][3]),
                        pack_bf16x2(acc[u][4], acc[u][5]), pack_bf16x2(acc[u][6], acc[u][7])};
          }
          y[tv0 + u * 64] = out;
        }
      }
    }
  }
}

// Finish of the fused combine: the down GEMM has added sum_j w_j * row_j into
// the fp32 accumulator y_acc; y = residual + shared + y_acc in fp32 in that
// order, rounded once.  One thread per 16 bytes of y (4 fp32 / 8 bf16
// elements), grid-stride.
template <int DTYPE>
__global__ __launch_bounds__(256) void combine_finish(const float* __restrict__ y_acc,
                                                      const u32x4* __restrict__ residual,
                                                      const u32x4* __restrict__ shared_out,
                                                      u32x4* __restrict__ y, size_t nvec) {
  constexpr int VE = DTYPE == 0 ? 4 : 8;
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t v = (size_t)blockIdx.x * blockDim.x + threadIdx.x; v < nvec; v += stride) {
    float acc[VE];
#pragma unroll
    for (int i = 0; i < VE; ++i) acc[i] = 0.f;
    auto add = [&](const u32x4 q) {
      const uint32_t w4[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if constexpr (DTYPE == 0) {
          acc[i] += __uint_as_float(w4[i]);
        } else {
          acc[2 * i] += bf16_to_f32(w4[i] & 0xffffu);
          acc[2 * i + 1] += bf16_to_f32(w4[i] >> 16);
        }
      }
    };
    if (residual) add(residual[v]);
    if (shared_out) add(shared_out[v]);
    const u32x4* yv = reinterpret_cast<const u32x4*>(y_acc) + v * (VE / 4);
#pragma unroll
    for (int c = 0; c < VE / 4; ++c) {
      const u32x4 q = yv[c];
      acc[4 * c] += __uint_as_float(q.x);
      acc[4 * c + 1] += __uint_as_float(q.y);
      acc[4 * c + 2] += __uint_as_float(q.z);
      acc[4 * c + 3] += __uint_as_float(q.w);
    }
    u32x4 out;
    if constexpr (DTYPE == 0) {
      out = u32x4{__float_as_uint(acc[0]), __float_as_uint(acc[1]), __float_as_uint(acc[2]),
                  __float_as_uint(acc[3])};
    } else {
      out = u32x4{pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]),
                  pack_bf16x2(acc[4], acc[5]), pack_bf16x2(acc[6], acc[7])};
    }
    y[v] = out;
  }
}

hipError_t launch_combine(const CombineArgs& a, hipStream_t st) {
  if (a.N == 0) return hipSuccess;
  if (a.y_acc) {
    const int elem = a.dtype == 0 ? 4 : 2;
    const size_t nvec = (size_t)a.N * a.d * elem / 16;
    const int blocks = (int)std::min<size_t>((nvec + 255) / 256, 8192);
    auto res = static_cast<const u32x4*>(a.residual);
    auto sh = static_cast<const u32x4*>(a.shared_out);
    auto y = static_cast<u32x4*>(a.y);
    if (a.dtype == 0) combine_finish<0><<<blocks, 256, 0, st>>>(a.y_acc, res, sh, y, nvec);
    else combine_finish<1><<<blocks, 256, 0, st>>>(a.y_acc, res, sh, y, nvec);
    return hipGetLastError();
  }
  const int elem = a.dtype == 0 ? 4 : 2;
  const int vec_per_row = a.d * elem / 16;
  const int blocks = std::max(1, std::min((a.N + 3) / 4, 8192));
  auto yp = static_cast<const u32x4*>(a.y_perm);
  auto res = static_cast<const u32x4*>(a.residual);
  auto sh = static_cast<const u32x4*>(a.shared_out);
  auto y = static_cast<u32x4*>(a.y);
  const bool wide = vec_per_row > 128;
  auto go = [&](auto kernel) {
    kernel<<<blocks, 256, 0, st>>>(yp, a.row_of_slot, a.topk_w, res, sh, y, a.N, vec_per_row,
                                   a.k);
  };
  // One kernel copy per (dtype, vectors in flight, slots held): registers are
  // reserved only for the slots a workload has.
  auto pick = [&](auto dt, auto v) {
    constexpr int D = decltype(dt)::value, VV = decltype(v)::value;
    if (a.k <= 1) go(combine_rows<D, VV, 1>);
    else if (a.k <= 2) go(combine_rows<D, VV, 2>);
    else if (a.k <= 4) go(combine_rows<D, VV, 4>);
    else go(combine_rows<D, VV, 8>);
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  if (a.dtype == 0) {
    if (wide) pick(I0{}, I2{}); else pick(I0{}, I1{});
  } else {
    if (wide) pick(I1{}, I2{}); else pick(I1{}, I1{});
  }
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
