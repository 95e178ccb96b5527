// router_backward.hip -- backward of the router and of an auxiliary
// load-balancing loss, for gfx950.
//
// The training step reads step 1 of the glossary's "How tokens travel between
// GPUs" (the router scores each token against each expert, keeps the k best,
// and weights their outputs) backwards: from the gradient at the combine
// weights to the gradient at the logits, then through the router's linear
// layer z = x W_r^T + b.  The auxiliary loss is the one the glossary's "Load
// balancing and capacity" section and MLSys ch.10 section 10.5 name without a
// formula; read here as the Switch Transformer's: coef * E * sum_e f_e P_e,
// f_e the fraction of assignments routed to e (a constant), P_e the mean over
// tokens of the token's router distribution (softmax over all E, or the
// sigmoid affinities normalised over all E).
//
// Kernels:
//  router_dz      one wave per token: the token's distribution over all E
//                 (wave max and sums), the gradient through the score
//                 function at the k selected experts, the auxiliary term at
//                 every expert; writes dz[t, :] (fp32) and the token's
//                 sum_e f_e P_e.
//  router_wgrad   dW_r = dz^T x and db = column sums of dz: 64 x 64 output
//                 tiles, the token dimension split over grid.z into partial
//                 sums in the workspace (so small E x d still fills the GPU).
//  router_reduce  sums the partials in split order (deterministic).
//  router_dgrad   dx = dz W_r (+ the caller's dx), 64 x 64 tiles, K = E.
//  router_loss    one block: the auxiliary loss from the per-token terms,
//                 summed in a fixed order.
// All fp32 arithmetic (fp64 for the loss sum); operands staged through LDS.
#include "device.h"
#include "kernels.h"

namespace moe {

namespace {

constexpr int kRbTile = 64, kRbK = 32;

template <int NJ>
__global__ __launch_bounds__(256) void router_dz(const float* __restrict__ z,
                                                 const int32_t* __restrict__ topk_idx,
                                                 const float* __restrict__ dtopk_w,
                                                 const int32_t* __restrict__ counts, int N, int E,
                                                 int k, int score_fn, float coef,
                                                 float* __restrict__ dz,
                                                 float* __restrict__ loss_terms) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= N) return;  // whole waves leave together; no block barrier below
  const float* zt = z + (size_t)t * E;
  const bool sig = score_fn == 2;
  float zl[NJ], P[NJ], a[NJ], dzl[NJ];
  float m = -INFINITY;
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int e = lane + 64 * j;
    zl[j] = e < E ? zt[e] : -INFINITY;
    m = fmaxf(m, zl[j]);
    dzl[j] = 0.f;
  }
  // The token's distribution over all E: softmax, or sigmoid / sum of sigmoids.
  float A = 0.f;
  if (sig) {
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      a[j] = lane + 64 * j < E ? 1.f / (1.f + expf(-zl[j])) : 0.f;
      A += a[j];
    }
  } else {
    m = wave_max(m);
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      a[j] = lane + 64 * j < E ? expf(zl[j] - m) : 0.f;
      A += a[j];
    }
  }
  A = wave_sum(A);
#pragma unroll
  for (int j = 0; j < NJ; ++j) P[j] = a[j] / A;

  // The k selected experts: ids, gradients at their weights and logits.
  int my_e = 0;
  float my_g = 0.f, my_z = 0.f;
  if (lane < k) {
    my_e = topk_idx[(size_t)t * k + lane];
    my_g = dtopk_w[(size_t)t * k + lane];
    my_z = zt[my_e];
  }
  // c_j: the gradient at the logit of selected expert j through the weights.
  float zmax_s = -INFINITY;
  for (int j = 0; j < k; ++j) zmax_s = fmaxf(zmax_s, __shfl(my_z, j, 64));
  float norm = 0.f, wg = 0.f;
  for (int j = 0; j < k; ++j) {
    const float zj = __shfl(my_z, j, 64), gj = __shfl(my_g, j, 64);
    float vj;
    if (score_fn == 0) vj = expf(zj - zmax_s);                // unnormalised softmax
    else if (score_fn == 1) vj = expf(zj - m) / A;            // p at the expert
    else vj = 1.f / (1.f + expf(-zj));                        // affinity
    norm += vj;
    wg += vj * gj;
  }
  // softmax over the k: w = v / norm, wg /= norm; all-E softmax: sum_j p_j g_j
  // as is; sigmoid: w = a / S with S = norm.
  if (score_fn != 1) wg /= norm;
  if (score_fn == 1) {
#pragma unroll
    for (int j = 0; j < NJ; ++j) dzl[j] -= P[j] * wg;
  }
  for (int j = 0; j < k; ++j) {
    const int ej = __shfl(my_e, j, 64);
    const float zj = __shfl(my_z, j, 64), gj = __shfl(my_g, j, 64);
    float c;
    if (score_fn == 0) {
      c = expf(zj - zmax_s) / norm * (gj - wg);
    } else if (score_fn == 1) {
      c = expf(zj - m) / A * gj;
    } else {
      const float aj = 1.f / (1.f + expf(-zj));
      c = aj * (1.f - aj) * (gj - wg) / norm;
    }
#pragma unroll
    for (int j2 = 0; j2 < NJ; ++j2)
      if (ej == lane + 64 * j2) dzl[j2] += c;
  }

  // Auxiliary loss: f_e = counts_e / (N k); fp = sum_e f_e P_e.
  if (coef != 0.f) {
    const float inv_nk = 1.f / ((float)N * (float)k);
    float f[NJ], fp = 0.f;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int e = lane + 64 * j;
      f[j] = e < E ? (float)counts[e] * inv_nk : 0.f;
      fp += f[j] * P[j];
    }
    fp = wave_sum(fp);
    const float scale = coef * (float)E / (float)N;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      if (sig) dzl[j] += scale * a[j] * (1.f - a[j]) * (f[j] - fp) / A;
      else dzl[j] += scale * P[j] * (f[j] - fp);
    }
    if (lane == 0) loss_terms[t] = fp;
  }
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int e = lane + 64 * j;
    if (e < E) dz[(size_t)t * E + e] = dzl[j];
  }
}

__device__ __forceinline__ float ld_elem(const void* p, int dtype, size_t i) {
  return dtype == 0 ? static_cast<const float*>(p)[i]
                    : bf16_to_f32(static_cast<const bf16_t*>(p)[i]);
}

// Partial dW_r[m0.., n0..] and db over tokens [t0, t1): out(m, n) = sum_t
// dz[t, m] x[t, n].  Thread (ty, tx) of 16 x 16 owns rows 4 ty.. and columns
// 4 tx.. of the 64 x 64 tile.
__global__ __launch_bounds__(256) void router_wgrad(const float* __restrict__ dz,
                                                    const void* __restrict__ x, int dtype, int N,
                                                    int E, int d, int kchunk,
                                                    float* __restrict__ part,
                                                    float* __restrict__ dbpart) {
  __shared__ float As[kRbK][kRbTile + 4];
  __shared__ float Bs[kRbK][kRbTile + 4];
  const int m0 = blockIdx.x * kRbTile, n0 = blockIdx.y * kRbTile, ks = blockIdx.z;
  const int t0 = ks * kchunk, t1 = min(N, t0 + kchunk);
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  float acc[4][4] = {};
  float dbacc = 0.f;
  for (int tb = t0; tb < t1; tb += kRbK) {
    for (int q = tid; q < kRbK * kRbTile; q += 256) {
      const int kk = q / kRbTile, c = q % kRbTile, t = tb + kk;
      As[kk][c] = (t < t1 && m0 + c < E) ? dz[(size_t)t * E + m0 + c] : 0.f;
      Bs[kk][c] = (t < t1 && n0 + c < d) ? ld_elem(x, dtype, (size_t)t * d + n0 + c) : 0.f;
    }
    __syncthreads();
#pragma unroll 8
    for (int kk = 0; kk < kRbK; ++kk) {
      float av[4], bv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        av[i] = As[kk][4 * ty + i];
        bv[i] = Bs[kk][4 * tx + i];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(av[i], bv[j], acc[i][j]);
    }
    if (blockIdx.y == 0 && tid < kRbTile)
      for (int kk = 0; kk < kRbK; ++kk) dbacc += As[kk][tid];
    __syncthreads();
  }
  float* out = part + (size_t)ks * E * d;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int mrow = m0 + 4 * ty + i;
    if (mrow >= E) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = n0 + 4 * tx + j;
      if (n < d) out[(size_t)mrow * d + n] = acc[i][j];
    }
  }
  if (blockIdx.y == 0 && tid < kRbTile && m0 + tid < E) dbpart[(size_t)ks * E + m0 + tid] = dbacc;
}

// Sum of the split partials, in split order: dW_r (E*d values), then db.
__global__ __launch_bounds__(256) void router_reduce(const float* __restrict__ part,
                                                     const float* __restrict__ dbpart, int E,
                                                     int d, int ksplit, float* __restrict__ dw,
                                                     float* __restrict__ db) {
  const size_t n = (size_t)E * d;
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n + E; i += stride) {
    float s = 0.f;
    if (i < n) {
      for (int ks = 0; ks < ksplit; ++ks) s += part[(size_t)ks * n + i];
      dw[i] = s;
    } else if (db) {
      const size_t e = i - n;
      for (int ks = 0; ks < ksplit; ++ks) s += dbpart[(size_t)ks * E + e];
      db[e] = s;
    }
  }
}

// dx[t0.., n0..] = (dx) + sum_e dz[t, e] W_r[e, n], K = E in steps of 32;
// rounded once to the dtype.
__global__ __launch_bounds__(256) void router_dgrad(const float* __restrict__ dz,
                                                    const void* __restrict__ w, int dtype, int N,
                                                    int E, int d, int accumulate,
                                                    void* __restrict__ dx) {
  __shared__ float As[kRbK][kRbTile + 4];  // As[e][t]
  __shared__ float Bs[kRbK][kRbTile + 4];  // Bs[e][n]
  const int t0 = blockIdx.x * kRbTile, n0 = blockIdx.y * kRbTile;
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  float acc[4][4] = {};
  for (int e0 = 0; e0 < E; e0 += kRbK) {
    for (int q = tid; q < kRbK * kRbTile; q += 256) {
      const int kk = q % kRbK, c = q / kRbK;  // dz rows: e contiguous
      As[kk][c] = (t0 + c < N && e0 + kk < E) ? dz[(size_t)(t0 + c) * E + e0 + kk] : 0.f;
      const int kb = q / kRbTile, cb = q % kRbTile;
      Bs[kb][cb] = (e0 + kb < E && n0 + cb < d) ? ld_elem(w, dtype, (size_t)(e0 + kb) * d + n0 + cb)
                                                : 0.f;
    }
    __syncthreads();
#pragma unroll 8
    for (int kk = 0; kk < kRbK; ++kk) {
      float av[4], bv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        av[i] = As[kk][4 * ty + i];
        bv[i] = Bs[kk][4 * tx + i];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(av[i], bv[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int t = t0 + 4 * ty + i;
    if (t >= N) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = n0 + 4 * tx + j;
      if (n >= d) continue;
      const size_t o = (size_t)t * d + n;
      const float v = accumulate ? acc[i][j] + ld_elem(dx, dtype, o) : acc[i][j];
      if (dtype == 0) static_cast<float*>(dx)[o] = v;
      else static_cast<bf16_t*>(dx)[o] = static_cast<bf16_t>(pack_bf16x2(v, 0.f) & 0xffffu);
    }
  }
}

// aux_loss = scale * sum_t terms[t], each thread summing a strided range in
// order in fp64, then a tree over the block in a fixed order.
__global__ __launch_bounds__(256) void router_loss(const float* __restrict__ terms, int N,
                                                   float scale, float* __restrict__ out) {
  __shared__ double s[256];
  double acc = 0.0;
  for (int t = threadIdx.x; t < N; t += 256) acc += (double)terms[t];
  s[threadIdx.x] = acc;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if (threadIdx.x < o) s[threadIdx.x] += s[threadIdx.x + o];
    __syncthreads();
  }
  if (threadIdx.x == 0) *out = (float)((double)scale * s[0]);
}

__global__ void router_zero_loss(float* out) { *out = 0.f; }

int ceil_div(int a, int b) { return (a + b - 1) / b; }

// Token splits of the weight gradient: enough blocks to fill the GPU, at
// least 256 tokens per split, at most 64 splits.
int wgrad_splits(int N, int E, int d) {
  const int tiles = ceil_div(E, kRbTile) * ceil_div(d, kRbTile);
  int ks = ceil_div(1024, tiles);
  ks = std::min(ks, std::max(1, N / 256));
  return std::max(1, std::min(ks, 64));
}

size_t a256(size_t x) { return (x + 255) / 256 * 256; }

}  // namespace

size_t router_backward_workspace_bytes(int N, int d, int E) {
  if (N <= 0) return 0;
  const int ks = wgrad_splits(N, E, d);
  return a256((size_t)N * E * 4) + a256((size_t)N * 4) +
         a256((size_t)ks * E * d * 4) + a256((size_t)ks * E * 4);
}

hipError_t launch_router_backward(const RouterBackwardArgs& a, hipStream_t st) {
  if (a.N == 0) {
    // No tokens: zero gradients (one reduce over no partials) and a zero loss.
    router_reduce<<<std::max(1, std::min(ceil_div(a.E * a.d + a.E, 256), 4096)), 256, 0, st>>>(
        nullptr, nullptr, a.E, a.d, 0, a.dw_router, a.db);
    if (a.aux_loss) router_zero_loss<<<1, 1, 0, st>>>(a.aux_loss);
    return hipGetLastError();
  }
  char* ws = static_cast<char*>(a.ws);
  float* dz = a.dlogits ? a.dlogits : reinterpret_cast<float*>(ws);
  ws += a256((size_t)a.N * a.E * 4);
  float* terms = reinterpret_cast<float*>(ws);
  ws += a256((size_t)a.N * 4);
  const int ks = wgrad_splits(a.N, a.E, a.d);
  float* part = reinterpret_cast<float*>(ws);
  ws += a256((size_t)ks * a.E * a.d * 4);
  float* dbpart = reinterpret_cast<float*>(ws);

  const int zb = ceil_div(a.N, 4);
  const int nj = ceil_div(a.E, 64);
  auto go = [&](auto kern) {
    kern<<<zb, 256, 0, st>>>(a.logits, a.topk_idx, a.dtopk_w, a.counts, a.N, a.E, a.k,
                             a.score_fn, a.aux_coef, dz, terms);
  };
  if (nj <= 1) go(router_dz<1>);
  else if (nj <= 2) go(router_dz<2>);
  else go(router_dz<4>);

  const dim3 gw(ceil_div(a.E, kRbTile), ceil_div(a.d, kRbTile), ks);
  router_wgrad<<<gw, 256, 0, st>>>(dz, a.x, a.dtype, a.N, a.E, a.d, ceil_div(a.N, ks), part,
                                    dbpart);
  router_reduce<<<std::max(1, std::min(ceil_div(a.E * a.d + a.E, 256), 4096)), 256, 0, st>>>(
      part, dbpart, a.E, a.d, ks, a.dw_router, a.db);
  if (a.dx) {
    const dim3 gd(ceil_div(a.N, kRbTile), ceil_div(a.d, kRbTile));
    router_dgrad<<<gd, 256, 0, st>>>(dz, a.w_router, a.dtype, a.N, a.E, a.d, a.accumulate_dx,
                                     a.dx);
  }
  if (a.aux_loss) {
    if (a.aux_coef != 0.f)
      router_loss<<<1, 256, 0, st>>>(terms, a.N, a.aux_coef * (float)a.E / (float)a.N,
                                     a.aux_loss);
    else
      router_zero_loss<<<1, 1, 0, st>>>(a.aux_loss);
  }
  return hipGetLastError();
}

}  // namespace moe
