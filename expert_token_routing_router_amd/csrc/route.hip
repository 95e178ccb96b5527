// route.hip -- router scoring and top-k selection for gfx950.
//
// Router scores (glossary "Expert Parallelism", "How tokens travel between
// GPUs", step 1 and its routing snippet: the router is a Linear(d, E) over the
// hidden state).  The logit of (t, e) is defined as the fp64 sum, left to
// right over the hidden index, of x[t,i]*w[e,i] (exact products), then + the
// router bias in fp64, rounded once to fp32.  Selection is then bit-exact and
// independent of how the work is split, because every output keeps that one
// sequential chain.
//
// Kernels:
//  router_weight_to_f64  w[E,d] (bf16/fp32) -> wt[d][Ep] fp64, transposed and
//                        zero-padded to Ep experts, so that one hidden index
//                        of a chunk of experts is a contiguous, wave-uniform run
//                        the scalar unit can load.
//  logits_f64            one wave = 64 tokens (one per lane) x EC experts; the
//                        x tile sits in LDS as fp32 (exact for bf16/fp32), the
//                        weights arrive as scalar operands, so each hidden
//                        index costs one LDS read and EC fp64 FMAs per lane.
//  select_topk           one wave per token: sigmoid/bias, group limit, top-k
//                        by (score desc, index asc) with wave arg-max, combine
//                        weights, and a per-block histogram of the choices.
#include "device.h"
#include "kernels.h"

namespace moe {

__global__ void router_weight_to_f64(const void* __restrict__ w, int dtype, int E, int d,
                                     int Ep, double* __restrict__ wt) {
  // Coalesced read over i (the contiguous index of w), strided write.
  const size_t total = (size_t)Ep * d;
  for (size_t q = (size_t)blockIdx.x * blockDim.x + threadIdx.x; q < total;
       q += (size_t)gridDim.x * blockDim.x) {
    const int e = (int)(q / d), i = (int)(q % d);
    const double v = e < E ? (double)load_elem(w, dtype, (size_t)e * d + i) : 0.0;
    wt[(size_t)i * Ep + e] = v;
  }
}

__global__ void zero_i32(int32_t* __restrict__ p, int n) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) p[i] = 0;
}

void launch_zero_i32(int32_t* p, int n, hipStream_t st) { zero_i32<<<1, 256, 0, st>>>(p, n); }

// Block: 256 threads = 4 waves.  The block covers TT token tiles of 64 and
// EG = 4 / TT expert chunks of EC.  Grid: (ceil(N / (64*TT)), ceil(Ep / (EC*EG))).
template <int EC, int TT>
__global__ __launch_bounds__(256) void logits_f64(const void* __restrict__ x, int dtype, int N,
                                                  int d, int E, int Ep,
                                                  const double* __restrict__ wt,
                                                  const float* __restrict__ router_bias,
                                                  float* __restrict__ logits,
                                                  int32_t* __restrict__ counts_to_zero) {
  constexpr int EG = 4 / TT;
  constexpr int BK = 64;
  __shared__ float xs[BK][TT * 64 + 1];  // [hidden index][token], fp32 (exact); +1: no bank conflicts on the transposed store
  __shared__ double wsm[BK][EG * EC];    // the block's weight columns of this K block

  if (counts_to_zero && blockIdx.x == 0 && blockIdx.y == 0) {
    for (int e = threadIdx.x; e < E; e += blockDim.x) counts_to_zero[e] = 0;
  }

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / 64);
  const int lane = threadIdx.x % 64;
  const int tt = wave / EG;                 // token tile of this wave inside the block
  const int eg = wave % EG;                 // expert chunk of this wave inside the block
  const int t0 = blockIdx.x * (TT * 64);
  const int e0 = (blockIdx.y * EG + eg) * EC;  // wave-uniform
  const int t = t0 + tt * 64 + lane;
  const bool active_chunk = e0 < Ep;

  double acc[EC];
#pragma unroll
  for (int c = 0; c < EC; ++c) acc[c] = 0.0;

  // K blocks of BK hidden indices; the next block's x and w values are
  // loaded into registers while the current one is multiplied.
  constexpr int XPT = TT * 64 * BK / 256;  // x values per thread per K block
  constexpr int WPT = (BK * EG * EC + 255) / 256;
  const int eb = blockIdx.y * EG * EC;
  float xr[XPT];
  double wr[WPT];
  auto fetch = [&](int k0) {
    const int kw = min(BK, d - k0);
#pragma unroll
    for (int u = 0; u < XPT; ++u) {
      const int q = threadIdx.x + 256 * u;
      const int r = q / BK, kk = q % BK, tr = t0 + r;
      xr[u] = (tr < N && kk < kw) ? load_elem(x, dtype, (size_t)tr * d + k0 + kk) : 0.f;
    }
#pragma unroll
    for (int u = 0; u < WPT; ++u) {
      const int q = threadIdx.x + 256 * u;
      const int kk = q / (EG * EC), j = q % (EG * EC);
      wr[u] = (q < BK * EG * EC && kk < kw && eb + j < Ep) ? wt[(size_t)(k0 + kk) * Ep + eb + j] : 0.0;
    }
  };
  fetch(0);
  for (int k0 = 0; k0 < d; k0 += BK) {
    const int kw = min(BK, d - k0);
    __syncthreads();  // every wave is done with the previous block
#pragma unroll
    for (int u = 0; u < XPT; ++u) {
      const int q = threadIdx.x + 256 * u;
      xs[q % BK][q / BK] = xr[u];  // transposed: [hidden index][token]
    }
#pragma unroll
    for (int u = 0; u < WPT; ++u) {
      const int q = threadIdx.x + 256 * u;
      if (q < BK * EG * EC) wsm[q / (EG * EC)][q % (EG * EC)] = wr[u];
    }
    __syncthreads();
    if (k0 + BK < d) fetch(k0 + BK);
    if (active_chunk) {
      // Unrolled so that the LDS reads run ahead of the fp64 chains; the
      // chains themselves keep their order (k ascending).
      if (kw == BK) {
#pragma unroll 16
        for (int kk = 0; kk < BK; ++kk) {
          const double xv = (double)xs[kk][tt * 64 + lane];
#pragma unroll
          for (int c = 0; c < EC; ++c) acc[c] = __fma_rn(xv, wsm[kk][eg * EC + c], acc[c]);
        }
      } else {
        for (int kk = 0; kk < kw; ++kk) {
          const double xv = (double)xs[kk][tt * 64 + lane];
#pragma unroll
          for (int c = 0; c < EC; ++c) acc[c] = __fma_rn(xv, wsm[kk][eg * EC + c], acc[c]);
        }
      }
    }
  }
  if (!active_chunk || t >= N) return;
#pragma unroll
  for (int c = 0; c < EC; ++c) {
    const int e = e0 + c;
    if (e < E) {
      double a = acc[c];
      if (router_bias) a = a + (double)router_bias[e];
      logits[(size_t)t * E + e] = __double2float_rn(a);
    }
  }
}

// Affinity of the sigmoid score: logistic function in fp64, rounded once.
__device__ __forceinline__ float sigmoid_affinity(float z) {
  return __double2float_rn(1.0 / (1.0 + exp(-(double)z)));
}

// One wave per token; a block of 4 waves walks TPB tokens.  Lane l holds
// experts l, l+64, l+128, l+192.
constexpr int kSelectTokensPerBlock = 64;
constexpr int kSelectWaves = 16;  // 4 tokens per wave

template <int NJ>  // ceil(E / 64) experts per lane
__global__ __launch_bounds__(kSelectWaves * 64) void select_topk(const float* __restrict__ logits,
                                                   const float* __restrict__ sel_bias, int N,
                                                   int E, int k, int G, int kg, int score_fn,
                                                   int32_t* __restrict__ topk_idx,
                                                   float* __restrict__ topk_w,
                                                   int32_t* __restrict__ counts) {
  __shared__ int32_t hist[256];
  __shared__ float sbuf[kSelectWaves][256];
  for (int e = threadIdx.x; e < E; e += blockDim.x) hist[e] = 0;
  __syncthreads();

  const int wave = threadIdx.x / 64, lane = threadIdx.x % 64;
  const int per = E / G;
  const int t_begin = blockIdx.x * kSelectTokensPerBlock;
  const int t_end = min(N, t_begin + kSelectTokensPerBlock);

  // The wave's tokens' logits are loaded up front, so their latency is paid
  // once per wave rather than once per token.
  constexpr int kTPW = kSelectTokensPerBlock / kSelectWaves;
  float zpre[kTPW][NJ];
#pragma unroll
  for (int i = 0; i < kTPW; ++i) {
    const int t = t_begin + wave + i * kSelectWaves;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int e = lane + 64 * j;
      zpre[i][j] = (t < t_end && e < E) ? logits[(size_t)t * E + e] : 0.f;
    }
  }
#pragma unroll
  for (int i = 0; i < kTPW; ++i) {
    const int t = t_begin + wave + i * kSelectWaves;
    if (t >= t_end) break;
    float z[NJ], s[NJ];
    bool ok[NJ];
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int e = lane + 64 * j;
      ok[j] = e < E;
      z[j] = zpre[i][j];
      const float a = score_fn == 2 ? sigmoid_affinity(z[j]) : z[j];
      s[j] = (ok[j] && sel_bias) ? a + sel_bias[e] : a;
    }

    // Group limit: only experts of the kg best groups stay eligible.
    if (G > 1) {
#pragma unroll
      for (int j = 0; j < NJ; ++j)
        if (ok[j]) sbuf[wave][lane + 64 * j] = s[j];
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
      float gs = 0.f;
      int gi = -1;
      if (lane < G) {
        gs = sbuf[wave][lane * per];
        for (int e = lane * per + 1; e < (lane + 1) * per; ++e) gs = fmaxf(gs, sbuf[wave][e]);
        gi = lane;
      }
      uint64_t keep = 0;
      for (int r = 0; r < kg; ++r) {
        float bs = gs;
        int bi = gi;
        wave_argmax(bs, bi);
        keep |= 1ull << bi;
        if (lane == bi) gi = -1;  // taken
      }
#pragma unroll
      for (int j = 0; j < NJ; ++j)
        if (ok[j]) ok[j] = (keep >> ((lane + 64 * j) / per)) & 1ull;
      __builtin_amdgcn_wave_barrier();
    }

    // Top-k by repeated wave arg-max (k <= 8; fully unrolled so the per-token
    // arrays stay in registers).
    int sel[8];
    float zsel[8];
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      sel[r] = 0;
      zsel[r] = 0.f;
      if (r < k) {
        float bs = 0.f;
        int bi = -1;
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
          const int e = lane + 64 * j;
          if (ok[j] && (bi < 0 || s[j] > bs)) {  // increasing e: ties keep the lower index
            bs = s[j];
            bi = e;
          }
        }
        wave_argmax(bs, bi);
        sel[r] = bi;
        const int owner = bi % 64, jj = bi / 64;
        float zv = z[0];
#pragma unroll
        for (int j = 1; j < NJ; ++j)
          if (jj == j) zv = z[j];
        zsel[r] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(zv), owner));
        if (lane == owner) {
#pragma unroll
          for (int j = 0; j < NJ; ++j)
            if (jj == j) ok[j] = false;
        }
      }
    }

    // Combine weights from the unbiased scores.
    double wsum = 0.0, w[8];
    if (score_fn == 0) {
      double zmax = (double)zsel[0];
#pragma unroll
      for (int r = 1; r < 8; ++r)
        if (r < k) zmax = fmax(zmax, (double)zsel[r]);
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        w[r] = r < k ? exp((double)zsel[r] - zmax) : 0.0;
        wsum += w[r];
      }
    } else if (score_fn == 1) {
      float m = -INFINITY;
#pragma unroll
      for (int j = 0; j < NJ; ++j)
        if (lane + 64 * j < E) m = fmaxf(m, z[j]);
      const double zmax = (double)wave_max(m);
      double part = 0.0;
#pragma unroll
      for (int j = 0; j < NJ; ++j)
        if (lane + 64 * j < E) part += exp((double)z[j] - zmax);
      wsum = wave_sum(part);
#pragma unroll
      for (int r = 0; r < 8; ++r) w[r] = r < k ? exp((double)zsel[r] - zmax) : 0.0;
    } else {
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        w[r] = r < k ? (double)sigmoid_affinity(zsel[r]) : 0.0;
        wsum += w[r];
      }
    }
    // Lane r < k writes slot r.
    int my_e = sel[0];
    double my_w = w[0];
#pragma unroll
    for (int r = 1; r < 8; ++r)
      if (lane == r) {
        my_e = sel[r];
        my_w = w[r];
      }
    if (lane < k) {
      topk_idx[(size_t)t * k + lane] = my_e;
      topk_w[(size_t)t * k + lane] = (float)(my_w / wsum);
      atomicAdd(&hist[my_e], 1);
    }
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += blockDim.x)
    if (hist[e]) atomicAdd(&counts[e], hist[e]);
}

// ---------------------------------------------------------------- launch ---

// Experts per wave chunk and the padded expert count of the fp64 weight copy.
static int route_chunk(int E) { return E <= 8 ? 8 : 16; }
static int route_padded_experts(int E) {
  const int ec = route_chunk(E);
  return (E + ec - 1) / ec * ec;
}

static size_t exact_logits_bytes(int N, int d, int E) {
  if (N <= 0) return 0;
  return (size_t)route_padded_experts(E) * d * sizeof(double);
}

// The certified path (bf16 inputs) streams rows in 32-element chunks.
static bool use_certified(const RouteArgs& a) {
  return a.dtype == 1 && a.d % 32 == 0 && a.E <= 256;
}

size_t route_workspace_bytes(int N, int d, int E, int dtype) {
  const size_t exact = exact_logits_bytes(N, d, E);
  const size_t cert = dtype == 1 ? route_certified_workspace_bytes(N, d, E) : 0;
  return exact > cert ? exact : cert;
}

// Exact fp64 logits of every pair; zeroes `counts` on the way (may be null).
static hipError_t launch_exact_logits(const RouteArgs& a, hipStream_t st) {
  const int EC = route_chunk(a.E);
  const int Ep = route_padded_experts(a.E);
  double* wt = static_cast<double*>(a.ws);
  {
    const size_t total = (size_t)Ep * a.d;
    const int blocks = (int)std::min<size_t>((total + 255) / 256, 4096);
    router_weight_to_f64<<<blocks, 256, 0, st>>>(a.w_router, a.dtype, a.E, a.d, Ep, wt);
  }
  const int chunks = (Ep + EC - 1) / EC;
  if (EC == 8) {
    // At most 8 experts: four waves of 2 experts each per 64-token tile, so
    // the grid has one block per 64 tokens.
    dim3 grid((a.N + 63) / 64, 1);
    logits_f64<2, 1><<<grid, 256, 0, st>>>(a.x, a.dtype, a.N, a.d, a.E, Ep, wt, a.router_bias,
                                            a.logits, a.counts);
  } else if (chunks >= 4) {
    dim3 grid((a.N + 63) / 64, (chunks + 3) / 4);
    logits_f64<16, 1><<<grid, 256, 0, st>>>(a.x, a.dtype, a.N, a.d, a.E, Ep, wt, a.router_bias,
                                             a.logits, a.counts);
  } else if (chunks >= 2) {
    dim3 grid((a.N + 127) / 128, (chunks + 1) / 2);
    logits_f64<16, 2><<<grid, 256, 0, st>>>(a.x, a.dtype, a.N, a.d, a.E, Ep, wt, a.router_bias,
                                             a.logits, a.counts);
  } else {
    dim3 grid((a.N + 255) / 256, 1);
    logits_f64<16, 4><<<grid, 256, 0, st>>>(a.x, a.dtype, a.N, a.d, a.E, Ep, wt, a.router_bias,
                                             a.logits, a.counts);
  }
  return hipGetLastError();
}

hipError_t launch_router_logits(const RouteArgs& a, hipStream_t st) {
  if (a.N == 0) return hipSuccess;
  return launch_exact_logits(a, st);
}

hipError_t launch_route(const RouteArgs& a, hipStream_t st) {
  if (a.N == 0) {
    zero_i32<<<1, 256, 0, st>>>(a.counts, a.E);
    return hipGetLastError();
  }
  if (use_certified(a)) return launch_route_certified(a, st);
  hipError_t err = launch_exact_logits(a, st);
  if (err != hipSuccess) return err;
  const int blocks = (a.N + kSelectTokensPerBlock - 1) / kSelectTokensPerBlock;
  auto select = [&](auto kernel) {
    kernel<<<blocks, kSelectWaves * 64, 0, st>>>(a.logits, a.sel_bias, a.N, a.E, a.k, a.G, a.kg,
                                                 a.score_fn, a.topk_idx, a.topk_w, a.counts);
  };
  switch ((a.E + 63) / 64) {
    case 1: select(select_topk<1>); break;
    case 2: select(select_topk<2>); break;
    case 3: select(select_topk<3>); break;
    default: select(select_topk<4>); break;
  }
  return hipGetLastError();
}

}  // namespace moe
