// backward_ffn.hip -- backward of the expert FFN on gfx950: the gradients of
// the layer's expert networks for a training step (each expert is an ordinary
// feed-forward block: glossary "Expert Parallelism", introduction; notes
// "为何不用 TP 切专家").
//
// Forward (ffn.hip): u = x W1^T, v = x W3^T, H = act(u) [* v], y = H W2^T.
// Backward over each expert's rows, by the chain rule:
//   g   = dy W2                  gradient at H
//   du  = g act'(u) [* v]        gradient at u            (rounded to bf16)
//   dv  = g silu(u)              gradient at v (SwiGLU)   (rounded to bf16)
//   dx  = du W1 [+ dv W3]                                 (rounded to bf16)
//   dW1 = du^T x, dW3 = dv^T x, dW2 = dy^T H              (fp32, summed over rows)
// u and v are recomputed, not kept from the forward.
//
// Three kernels, all on v_mfma_f32_32x32x16_bf16 with fp32 accumulators:
//   bwd_act    per 128-row tile of an expert, K = d: the three products x W1^T,
//              x W3^T and dy W2 share the tile; the epilogue writes H and
//              G = [du | dv] (bf16) to the workspace;
//   bwd_dgrad  dx = G [W1 ; W3], K = h (2h for SwiGLU);
//   bwd_wgrad  weight gradients, K = the expert's rows: G^T x into dW1 / dW3,
//              dy^T H into dW2.  An expert with no rows gets zeros.
// Block tile: 128 output columns x 128 output rows; 4 waves of 64 x 64 (2 x 2
// fragments of 32 x 32).  A staged operand tile holds 32 k per row in LDS,
// rows padded to 40 elements; operands whose memory runs along the row
// index instead (W2 in bwd_act, the weights in bwd_dgrad, every operand of
// bwd_wgrad) are transposed on their way into LDS, each thread loading the
// same 8 rows at two consecutive k and writing them as 8 packed k pairs.
// The next K step's global loads are in flight while the current step is
// multiplied.
#include "device.h"
#include "kernels.h"

namespace moe {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kBK = 32, kLdk = kBK + 8;  // staged row: 32 k + 8 pad elements (80 bytes)
constexpr int kTM = 128, kTN = 128;      // block tile: output columns x output rows
constexpr int kThreads = 256;
constexpr int kRelu = 0, kGelu = 1, kSwiglu = 2;

size_t align256(size_t x) { return (x + 255) / 256 * 256; }

// The 16-byte vectors one thread stages per K step for an R-row tile.
template <int R>
struct Stage {
  static_assert(R == 128, "staged tiles are 128 rows: two vectors per thread");
  u32x4 v[R * (kBK / 8) / kThreads];
};

// Rows whose k run is contiguous: element (row, k) at src[(row0 + row) * ld +
// k0 + k]; rows at or past nrow read as zero.
template <int R>
__device__ __forceinline__ void fetch_k(Stage<R>& s, const bf16_t* __restrict__ src, size_t ld,
                                        int row0, int nrow, int k0) {
#pragma unroll
  for (int p = 0; p < R * 4 / kThreads; ++p) {
    const int idx = p * kThreads + threadIdx.x, row = idx >> 2, c = idx & 3;
    s.v[p] = row < nrow ? *reinterpret_cast<const u32x4*>(src + (size_t)(row0 + row) * ld +
                                                          k0 + 8 * c)
                        : u32x4{0u, 0u, 0u, 0u};
  }
}

template <int R>
__device__ __forceinline__ void put_k(bf16_t* T, const Stage<R>& s) {
#pragma unroll
  for (int p = 0; p < R * 4 / kThreads; ++p) {
    const int idx = p * kThreads + threadIdx.x, row = idx >> 2, c = idx & 3;
    *reinterpret_cast<u32x4*>(T + row * kLdk + 8 * c) = s.v[p];
  }
}

// Rows whose memory runs along the row index: element (row, k) at
// src[(k0 + k) * ld + row0 + row]; k at or past nk, and rows at or past nrow
// (a multiple of 8), read as zero.  Thread i stages rows [8c, 8c + 8) at
// k = 2kp and 2kp + 1 (kp = i / 16, c = i % 16).
template <int R>
__device__ __forceinline__ void fetch_t(Stage<R>& s, const bf16_t* __restrict__ src, size_t ld,
                                        int row0, int nrow, int k0, int nk) {
  const int kp = threadIdx.x >> 4, c = threadIdx.x & 15;
  const bool row_ok = 8 * c < nrow;
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const int k = 2 * kp + p;
    s.v[p] = (row_ok && k < nk)
                 ? *reinterpret_cast<const u32x4*>(src + (size_t)(k0 + k) * ld + row0 + 8 * c)
                 : u32x4{0u, 0u, 0u, 0u};
  }
}

template <int R>
__device__ __forceinline__ void put_t(bf16_t* T, const Stage<R>& s) {
  const int kp = threadIdx.x >> 4, c = threadIdx.x & 15;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint32_t a = s.v[0][q], b = s.v[1][q];  // rows 8c + 2q, 8c + 2q + 1 at k = 2kp, 2kp + 1
    *reinterpret_cast<uint32_t*>(T + (8 * c + 2 * q) * kLdk + 2 * kp) = (a & 0xffffu) | (b << 16);
    *reinterpret_cast<uint32_t*>(T + (8 * c + 2 * q + 1) * kLdk + 2 * kp) =
        (a >> 16) | (b & 0xffff0000u);
  }
}

// acc[f][j] += P rows [wm*64 + 32f, +32) x Q rows [wn*64 + 32j, +32) over
// the 32 staged k.  Afterwards lane l holds, in acc[f][j][4g + i], output
// column wm*64 + 32f + 8g + 4(l/32) + i of output row wn*64 + 32j + l%32.
typedef f32x16 Acc[2][2];

__device__ __forceinline__ void mma(Acc& acc, const bf16_t* P, const bf16_t* Q, int wm, int wn,
                                    int lane) {
  const int lr = lane & 31, lk = (lane >> 5) * 8;
#pragma unroll
  for (int kk = 0; kk < kBK; kk += 16) {
    bf16x8 q[2], p[2];
#pragma unroll
    for (int j = 0; j < 2; ++j)
      q[j] = *reinterpret_cast<const bf16x8*>(Q + (wn * 64 + j * 32 + lr) * kLdk + kk + lk);
#pragma unroll
    for (int f = 0; f < 2; ++f)
      p[f] = *reinterpret_cast<const bf16x8*>(P + (wm * 64 + f * 32 + lr) * kLdk + kk + lk);
#pragma unroll
    for (int f = 0; f < 2; ++f)
#pragma unroll
      for (int j = 0; j < 2; ++j)
        acc[f][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(p[f], q[j], acc[f][j], 0, 0, 0);
  }
}

__device__ __forceinline__ void zero(Acc& acc) {
#pragma unroll
  for (int f = 0; f < 2; ++f)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[f][j][i] = 0.f;
}

__device__ __forceinline__ void store4_bf16(bf16_t* p, float a, float b, float c, float d) {
  *reinterpret_cast<uint2*>(p) = make_uint2(pack_bf16x2(a, b), pack_bf16x2(c, d));
}

// Expert e's segment: rows [offsets[e], offsets[e+1]) clamped to max_rows and,
// when group_rows is given, to its first group_rows[e] rows (the rows that hold
// data in a padded layout).
__device__ __forceinline__ int2 segment(const int32_t* __restrict__ offsets,
                                        const int32_t* __restrict__ group_rows, int e,
                                        int max_rows) {
  const int lo = min(offsets[e], max_rows);
  int hi = min(offsets[e + 1], max_rows);
  if (group_rows) hi = min(hi, lo + max(group_rows[e], 0));
  return make_int2(lo, hi);
}

// 128-row tiles of every expert's segment, in expert order: tiles[q] = (expert,
// first row, end row).  At most cap tiles are written (segments that overlap
// could ask for more); count = the number written.
__global__ __launch_bounds__(1024) void bwd_plan(const int32_t* __restrict__ offsets,
                                                 const int32_t* __restrict__ group_rows, int E,
                                                 int max_rows, int cap, int4* __restrict__ tiles,
                                                 int32_t* __restrict__ count) {
  __shared__ int32_t s[1024];
  const int e = threadIdx.x;
  int lo = 0, hi = 0, n = 0;
  if (e < E) {
    const int2 sg = segment(offsets, group_rows, e, max_rows);
    lo = sg.x;
    hi = sg.y;
    n = hi > lo ? (hi - lo + kTN - 1) / kTN : 0;
  }
  s[e] = n;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    const int add = e >= off ? s[e - off] : 0;
    __syncthreads();
    s[e] += add;
    __syncthreads();
  }
  const int start = s[e] - n;
  for (int q = 0; q < n && start + q < cap; ++q)
    tiles[start + q] = make_int4(e, lo + q * kTN, min(hi, lo + (q + 1) * kTN), 0);
  if (e == 1023) *count = min(s[1023], cap);
}

// H and G = [du | dv] for one 128-row tile and 128 columns of h.
template <int ACT>
__global__ __launch_bounds__(kThreads) void bwd_act(
    const bf16_t* __restrict__ x, const bf16_t* __restrict__ dy, const bf16_t* __restrict__ w1,
    const bf16_t* __restrict__ w3, const bf16_t* __restrict__ w2, const int4* __restrict__ tiles,
    const int32_t* __restrict__ tile_count, int d, int h, bf16_t* __restrict__ Hbuf,
    bf16_t* __restrict__ G) {
  constexpr bool DUAL = ACT == kSwiglu;
  if ((int)blockIdx.y >= *tile_count) return;
  const int4 t = tiles[blockIdx.y];
  const int e = t.x, r0 = t.y, nr = t.z - t.y;
  const int m0 = blockIdx.x * kTM, nm = min(kTM, h - m0);
  const size_t wsz = (size_t)h * d;
  const bf16_t* W1 = w1 + e * wsz;
  const bf16_t* W3 = DUAL ? w3 + e * wsz : nullptr;
  const bf16_t* W2 = w2 + e * wsz;
  __shared__ __align__(16) bf16_t P1[kTM * kLdk];
  __shared__ __align__(16) bf16_t P3[DUAL ? kTM * kLdk : 8];
  __shared__ __align__(16) bf16_t P2[kTM * kLdk];
  __shared__ __align__(16) bf16_t QX[kTN * kLdk];
  __shared__ __align__(16) bf16_t QD[kTN * kLdk];
  Stage<kTM> s1, s3, s2;
  Stage<kTN> sx, sd;
  auto fetch = [&](int k0) {
    fetch_k<kTM>(s1, W1, d, m0, nm, k0);
    if constexpr (DUAL) fetch_k<kTM>(s3, W3, d, m0, nm, k0);
    fetch_t<kTM>(s2, W2, h, m0, nm, k0, kBK);  // (m = j, k = i) = W2[i][j]
    fetch_k<kTN>(sx, x, d, r0, nr, k0);
    fetch_k<kTN>(sd, dy, d, r0, nr, k0);
  };
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, wm = w & 1, wn = w >> 1;
  Acc au, av, ag;
  zero(au);
  zero(av);
  zero(ag);
  fetch(0);
  for (int k0 = 0; k0 < d; k0 += kBK) {
    __syncthreads();
    put_k<kTM>(P1, s1);
    if constexpr (DUAL) put_k<kTM>(P3, s3);
    put_t<kTM>(P2, s2);
    put_k<kTN>(QX, sx);
    put_k<kTN>(QD, sd);
    __syncthreads();
    if (k0 + kBK < d) fetch(k0 + kBK);
    mma(au, P1, QX, wm, wn, lane);
    if constexpr (DUAL) mma(av, P3, QX, wm, wn, lane);
    mma(ag, P2, QD, wm, wn, lane);
  }
  const size_t ldg = DUAL ? 2 * (size_t)h : (size_t)h;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int n = wn * 64 + j * 32 + (lane & 31);
    if (n >= nr) continue;
    const size_t row = (size_t)(r0 + n);
#pragma unroll
    for (int f = 0; f < 2; ++f) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int m = wm * 64 + f * 32 + g * 8 + 4 * (lane >> 5);
        if (m >= nm) continue;
        float hv[4], gu[4], gv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float u = au[f][j][4 * g + i], gg = ag[f][j][4 * g + i];
          if constexpr (ACT == kRelu) {
            hv[i] = fmaxf(u, 0.f);
            gu[i] = u > 0.f ? gg : 0.f;
          } else if constexpr (ACT == kGelu) {
            const float Phi = 0.5f * (1.f + erff(u * 0.70710678118654752f));
            const float phi = 0.39894228040143268f * expf(-0.5f * u * u);
            hv[i] = u * Phi;
            gu[i] = gg * (Phi + u * phi);
          } else {
            const float v = av[f][j][4 * g + i];
            const float s = 1.f / (1.f + expf(-u)), si = u * s;
            hv[i] = si * v;
            gu[i] = gg * v * (s * (1.f + u * (1.f - s)));
            gv[i] = gg * si;
          }
        }
        const int col = m0 + m;
        store4_bf16(Hbuf + row * h + col, hv[0], hv[1], hv[2], hv[3]);
        store4_bf16(G + row * ldg + col, gu[0], gu[1], gu[2], gu[3]);
        if constexpr (DUAL) store4_bf16(G + row * ldg + h + col, gv[0], gv[1], gv[2], gv[3]);
      }
    }
  }
}

// dx for one 128-row tile and 128 columns of d: K runs over [du | dv].
template <bool DUAL>
__global__ __launch_bounds__(kThreads) void bwd_dgrad(
    const bf16_t* __restrict__ G, const bf16_t* __restrict__ w1, const bf16_t* __restrict__ w3,
    const int4* __restrict__ tiles, const int32_t* __restrict__ tile_count, int d, int h,
    bf16_t* __restrict__ dx) {
  if ((int)blockIdx.y >= *tile_count) return;
  const int4 t = tiles[blockIdx.y];
  const int e = t.x, r0 = t.y, nr = t.z - t.y;
  const int m0 = blockIdx.x * kTM, nm = min(kTM, d - m0);
  const int K = DUAL ? 2 * h : h;
  const size_t wsz = (size_t)h * d;
  const bf16_t* W1 = w1 + e * wsz;
  const bf16_t* W3 = DUAL ? w3 + e * wsz : nullptr;
  __shared__ __align__(16) bf16_t P[kTM * kLdk];
  __shared__ __align__(16) bf16_t Q[kTN * kLdk];
  Stage<kTM> sp;
  Stage<kTN> sq;
  auto fetch = [&](int k0) {
    const bool second = DUAL && k0 >= h;  // h % 32 == 0: a K step lies in one half
    fetch_t<kTM>(sp, second ? W3 : W1, d, m0, nm, second ? k0 - h : k0, kBK);  // (i, j) = W[j][i]
    fetch_k<kTN>(sq, G, K, r0, nr, k0);
  };
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, wm = w & 1, wn = w >> 1;
  Acc acc;
  zero(acc);
  fetch(0);
  for (int k0 = 0; k0 < K; k0 += kBK) {
    __syncthreads();
    put_t<kTM>(P, sp);
    put_k<kTN>(Q, sq);
    __syncthreads();
    if (k0 + kBK < K) fetch(k0 + kBK);
    mma(acc, P, Q, wm, wn, lane);
  }
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int n = wn * 64 + j * 32 + (lane & 31);
    if (n >= nr) continue;
    bf16_t* out = dx + (size_t)(r0 + n) * d + m0;
#pragma unroll
    for (int f = 0; f < 2; ++f) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int m = wm * 64 + f * 32 + g * 8 + 4 * (lane >> 5);
        if (m < nm)
          store4_bf16(out + m, acc[f][j][4 * g], acc[f][j][4 * g + 1], acc[f][j][4 * g + 2],
                      acc[f][j][4 * g + 3]);
      }
    }
  }
}

// Weight gradient of expert blockIdx.y: out(n, m) = sum over the expert's rows
// r of Q[r][n] P[r][m] (P, Q row-major with leading dimensions ldp, ldq).
// Output row n < split goes to outA[e][n], row n >= split to outB[e][n - split]
// (fp32, M columns).
__global__ __launch_bounds__(kThreads) void bwd_wgrad(
    const bf16_t* __restrict__ Psrc, int ldp, const bf16_t* __restrict__ Qsrc, int ldq,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ group_rows, int max_rows,
    int M, int Nn, int split, float* __restrict__ outA, float* __restrict__ outB) {
  const int e = blockIdx.y;
  const int mt = (M + kTM - 1) / kTM;
  const int m0 = (blockIdx.x % mt) * kTM, n0 = (blockIdx.x / mt) * kTN;
  const int nm = min(kTM, M - m0), nn = min(kTN, Nn - n0);
  const int2 sg = segment(offsets, group_rows, e, max_rows);
  const int lo = sg.x, K = max(sg.y - sg.x, 0);
  __shared__ __align__(16) bf16_t P[kTM * kLdk];
  __shared__ __align__(16) bf16_t Q[kTN * kLdk];
  Stage<kTM> sp;
  Stage<kTN> sq;
  auto fetch = [&](int k0) {
    const int nk = min(kBK, K - k0);
    fetch_t<kTM>(sp, Psrc, ldp, m0, nm, lo + k0, nk);
    fetch_t<kTN>(sq, Qsrc, ldq, n0, nn, lo + k0, nk);
  };
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, wm = w & 1, wn = w >> 1;
  Acc acc;
  zero(acc);
  if (K > 0) fetch(0);
  for (int k0 = 0; k0 < K; k0 += kBK) {
    __syncthreads();
    put_t<kTM>(P, sp);
    put_t<kTN>(Q, sq);
    __syncthreads();
    if (k0 + kBK < K) fetch(k0 + kBK);
    mma(acc, P, Q, wm, wn, lane);
  }
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int nl = wn * 64 + j * 32 + (lane & 31);
    if (nl >= nn) continue;
    const int n = n0 + nl;
    float* orow = n < split ? outA + ((size_t)e * split + n) * M
                            : outB + ((size_t)e * (Nn - split) + (n - split)) * M;
#pragma unroll
    for (int f = 0; f < 2; ++f) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int m = wm * 64 + f * 32 + g * 8 + 4 * (lane >> 5);
        if (m < nm)
          *reinterpret_cast<float4*>(orow + m0 + m) = make_float4(
              acc[f][j][4 * g], acc[f][j][4 * g + 1], acc[f][j][4 * g + 2], acc[f][j][4 * g + 3]);
      }
    }
  }
}

int tile_cap(int E, int max_rows) { return (max_rows + kTN - 1) / kTN + E; }

}  // namespace

size_t ffn_backward_workspace_bytes(int E, int max_rows, int d, int h, int act) {
  (void)d;
  const size_t kg = act == kSwiglu ? 2 * (size_t)h : (size_t)h;
  return align256(sizeof(int32_t)) + align256((size_t)tile_cap(E, max_rows) * sizeof(int4)) +
         align256((size_t)max_rows * h * 2) + align256((size_t)max_rows * kg * 2);
}

int ffn_backward_max_tiles(int E, int max_rows) { return tile_cap(E, max_rows); }

hipError_t launch_ffn_backward(const FfnBackwardArgs& a, hipStream_t st) {
  const bool dual = a.act == kSwiglu;
  const int kg = dual ? 2 * a.h : a.h;
  const bf16_t* x = static_cast<const bf16_t*>(a.x_rows);
  const bf16_t* dy = static_cast<const bf16_t*>(a.dy_rows);
  const bf16_t* w1 = static_cast<const bf16_t*>(a.w1);
  const bf16_t* w3 = static_cast<const bf16_t*>(a.w3);
  const bf16_t* w2 = static_cast<const bf16_t*>(a.w2);
  bf16_t* Hbuf = nullptr;
  bf16_t* G = nullptr;
  if (a.max_rows > 0) {
    const int cap = tile_cap(a.E, a.max_rows);
    char* ws = static_cast<char*>(a.ws);
    int32_t* count = reinterpret_cast<int32_t*>(ws);
    int4* tiles = reinterpret_cast<int4*>(ws + align256(sizeof(int32_t)));
    Hbuf = reinterpret_cast<bf16_t*>(ws + align256(sizeof(int32_t)) +
                                     align256((size_t)cap * sizeof(int4)));
    G = reinterpret_cast<bf16_t*>(reinterpret_cast<char*>(Hbuf) +
                                  align256((size_t)a.max_rows * a.h * 2));
    bwd_plan<<<1, 1024, 0, st>>>(a.offsets, a.group_rows, a.E, a.max_rows, cap, tiles, count);
    const dim3 ga((a.h + kTM - 1) / kTM, cap);
    switch (a.act) {
      case kRelu:
        bwd_act<kRelu><<<ga, kThreads, 0, st>>>(x, dy, w1, w3, w2, tiles, count, a.d, a.h, Hbuf, G);
        break;
      case kGelu:
        bwd_act<kGelu><<<ga, kThreads, 0, st>>>(x, dy, w1, w3, w2, tiles, count, a.d, a.h, Hbuf, G);
        break;
      default:
        bwd_act<kSwiglu><<<ga, kThreads, 0, st>>>(x, dy, w1, w3, w2, tiles, count, a.d, a.h, Hbuf,
                                                  G);
        break;
    }
    const dim3 gd((a.d + kTM - 1) / kTM, cap);
    bf16_t* dx = static_cast<bf16_t*>(a.dx_rows);
    if (dual)
      bwd_dgrad<true><<<gd, kThreads, 0, st>>>(G, w1, w3, tiles, count, a.d, a.h, dx);
    else
      bwd_dgrad<false><<<gd, kThreads, 0, st>>>(G, w1, w3, tiles, count, a.d, a.h, dx);
  }
  // Weight gradients (zeros for experts without rows, so they run even for
  // an empty batch: no operand is read then).
  const dim3 g13(((a.d + kTM - 1) / kTM) * ((kg + kTN - 1) / kTN), a.E);
  bwd_wgrad<<<g13, kThreads, 0, st>>>(x, a.d, G, kg, a.offsets, a.group_rows, a.max_rows, a.d,
                                      kg, a.h, a.dw1, a.dw3);
  const dim3 g2(((a.h + kTM - 1) / kTM) * ((a.d + kTN - 1) / kTN), a.E);
  bwd_wgrad<<<g2, kThreads, 0, st>>>(Hbuf, a.h, dy, a.d, a.offsets, a.group_rows, a.max_rows,
                                     a.h, a.d, a.d, a.dw2, nullptr);
  return hipGetLastError();
}

// The backward on packed weights: u (v), g and dx on the forward's grouped
// GEMM (LDS-DMA ring, packed weights), then the weight gradients on the same
// GEMM from G, H, x and dy transposed per expert (ffn.hip).  An empty batch
// only zeroes the weight gradients.
hipError_t launch_ffn_backward_packed(const FfnBwdPackedArgs& a, float* dw1, float* dw3,
                                      float* dw2, hipStream_t st) {
  if (a.max_rows == 0) {
    const size_t hd = (size_t)a.E * a.h * a.d;
    hipError_t err = launch_zero_f32(dw1, hd, st);
    if (err == hipSuccess && dw3) err = launch_zero_f32(dw3, hd, st);
    if (err == hipSuccess) err = launch_zero_f32(dw2, hd, st);
    return err;
  }
  void* gv = nullptr;
  void* hv = nullptr;
  const hipError_t err = launch_ffn_bwd_packed_gemms(a, &gv, &hv, st);
  if (err != hipSuccess) return err;
  char* wg = static_cast<char*>(a.ws) +
             ffn_bwd_gemms_workspace_bytes(a.E, a.max_rows, a.d, a.h, a.act);
  return launch_ffn_bwd_wgrad(a, gv, hv, wg, dw1, dw3, dw2, st);
}

}  // namespace moe
