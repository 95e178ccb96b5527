// ffn.hip -- the expert FFN as grouped GEMMs on gfx950 MFMA.
//
// Glossary "Expert Parallelism", step 3 of "How tokens travel between GPUs":
// each GPU runs its local experts over the rows it received.  Rows are grouped
// by expert (offsets from the dispatch step, on the device), so every expert
// is one GEMM over a contiguous row range, and all experts run in one launch:
//
//   GEMM1:  H[rows, h] = act(X[rows, d] W1_e^T)     (SwiGLU: two B operands,
//           gate W1_e and up W3_e, combined as silu(gate) * up in registers)
//   GEMM2:  Y[rows, d] = H[rows, h] W2_e^T
//
// Both are "A row-major [M,K], B row-major [N,K]" products, K contiguous in
// both operands, which is the natural operand order of the MFMA units.
//
// Scheduling: a prologue kernel turns the per-expert row counts into a prefix
// of M tiles.  The GEMM grid is sized for the worst case (max_rows/BM + E
// tiles); block b is remapped so that consecutive logical tiles run on the
// same XCD (the hardware deals blocks round-robin over the 8 XCDs), logical
// tiles walk the N tiles of one M tile first (A tile reused from that XCD's
// L2), and blocks past the real tile count exit at once.
//
// bf16 kernel: 256 threads (2x2 waves), tile BM x BN x 64, each wave owns
// (BM/2) x (BN/2) as 32x32 MFMA blocks (v_mfma_f32_32x32x16_bf16).  Tiles go
// global -> registers -> LDS (double buffered), the next K tile's global loads
// in flight while the current one is multiplied.  LDS rows are 64 bf16 = eight
// 16-byte chunks; chunk c of row r is stored at c ^ (r & 7) so the 16-byte
// fragment reads of 8 consecutive rows hit 8 different bank groups.
//
// fp32 kernel (fp32 workloads): same schedule, v_mfma_f32_16x16x4_f32, 64x64
// tiles, K step 16; plain padded LDS rows.
#include "device.h"
#include "kernels.h"

namespace moe {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

enum { ACT_RELU = 0, ACT_GELU = 1, ACT_SWIGLU = 2, ACT_NONE = 3 };

__device__ __forceinline__ float apply_act(float u, int act) {
  if (act == ACT_RELU) return fmaxf(u, 0.f);
  if (act == ACT_GELU) return 0.5f * u * (1.f + erff(u * 0.70710678118654752440f));
  return u;
}

__device__ __forceinline__ float silu(float g) { return g / (1.f + __expf(-g)); }

// ----------------------------------------------------------- tile prefix ---

// One block of 1024 threads: tile_start[e] = sum over e' < e of
// ceil(rows_e' / BM); tile_start[E] = total.  E <= 1024.
__global__ __launch_bounds__(1024) void ffn_tile_prefix(const int32_t* __restrict__ offsets,
                                                        int E, int BM,
                                                        int32_t* __restrict__ tile_start) {
  __shared__ int32_t s[1024];
  const int e = threadIdx.x;
  int32_t n = 0;
  if (e < E) {
    const int32_t rows = offsets[e + 1] - offsets[e];
    n = rows > 0 ? (rows + BM - 1) / BM : 0;
  }
  s[e] = n;
  __syncthreads();
  for (int o = 1; o < 1024; o <<= 1) {
    const int32_t v = e >= o ? s[e - o] : 0;
    __syncthreads();
    s[e] += v;
    __syncthreads();
  }
  if (e < E) tile_start[e] = s[e] - n;
  if (e == E - 1) tile_start[E] = s[e];
}

// Map a block to (expert, first row, row end, n tile); false if past the end.
__device__ __forceinline__ bool locate_tile(int b, int grid8, int n_tiles,
                                            const int32_t* __restrict__ tile_start,
                                            const int32_t* __restrict__ offsets, int E, int BM,
                                            int max_rows, int& e, int& r0, int& r1, int& nt) {
  // XCD-aware remap: hardware XCD = b % 8; give each XCD a contiguous range.
  const int per_xcd = grid8 / 8;
  const int logical = (b % 8) * per_xcd + b / 8;
  const int mt = logical / n_tiles;
  nt = logical % n_tiles;
  const int total = tile_start[E];
  if (mt >= total) return false;
  int lo = 0, hi = E - 1;  // largest e with tile_start[e] <= mt
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (tile_start[mid] <= mt) lo = mid;
    else hi = mid - 1;
  }
  e = lo;
  r0 = offsets[e] + (mt - tile_start[e]) * BM;
  r1 = min(min(offsets[e + 1], r0 + BM), max_rows);
  return r0 < r1;
}

// ------------------------------------------------------------- bf16 MFMA ---

template <int BM, int BN, bool DUAL>
struct Bf16Smem {
  u32x4 a[2][BM * 8];
  u32x4 b[2][BN * 8];
  u32x4 b2[2][DUAL ? BN * 8 : 1];
};

// ACT: ACT_RELU / ACT_GELU / ACT_SWIGLU (then DUAL) / ACT_NONE.
template <int BM, int BN, int ACT>
__global__ __launch_bounds__(256) void grouped_gemm_bf16(
    const bf16_t* __restrict__ A, const bf16_t* __restrict__ B, const bf16_t* __restrict__ B2,
    bf16_t* __restrict__ C, int K, int N, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ tile_start, int E, int n_tiles, int max_rows) {
  constexpr bool DUAL = ACT == ACT_SWIGLU;
  constexpr int BK = 64;
  constexpr int FM = BM / 64, FN = BN / 64;       // 32x32 blocks per wave
  constexpr int LA = BM * 8 / 256, LB = BN * 8 / 256;  // 16-byte loads per thread
  __shared__ Bf16Smem<BM, BN, DUAL> sm;

  int e, r0, r1, nt;
  if (!locate_tile(blockIdx.x, gridDim.x, n_tiles, tile_start, offsets, E, BM, max_rows, e, r0,
                   r1, nt))
    return;
  const int n0 = nt * BN;
  const int tid = threadIdx.x, lane = tid % 64, wave = tid / 64;
  const int wm = wave / 2, wn = wave % 2;

  const size_t bexp = (size_t)e * N * K;
  const u32x4* Ag = reinterpret_cast<const u32x4*>(A);
  const u32x4* Bg = reinterpret_cast<const u32x4*>(B + bexp);
  const u32x4* B2g = DUAL ? reinterpret_cast<const u32x4*>(B2 + bexp) : nullptr;
  const int kchunks = K / 8;  // 16-byte chunks per row

  // Per-thread global chunk coordinates (row in tile, chunk in row).
  int a_row[LA], b_row[LB];
  const int cpos = tid % 8;
#pragma unroll
  for (int i = 0; i < LA; ++i) {
    const int r = (tid + i * 256) / 8;
    a_row[i] = min(r0 + r, r1 - 1);  // clamp: rows past the group are computed, not stored
  }
#pragma unroll
  for (int i = 0; i < LB; ++i) {
    const int r = (tid + i * 256) / 8;
    b_row[i] = min(n0 + r, N - 1);
  }

  u32x4 ra[LA], rb[LB], rb2[DUAL ? LB : 1];
  auto swz = [](int r, int c) { return r * 8 + (c ^ (r & 7)); };
#define MOE_GLOAD(kt_)                                                             \
  do {                                                                             \
    const int kc_ = (kt_) * 8 + cpos;                                              \
    _Pragma("unroll") for (int i = 0; i < LA; ++i) ra[i] =                         \
        Ag[(size_t)a_row[i] * kchunks + kc_];                                      \
    _Pragma("unroll") for (int i = 0; i < LB; ++i) rb[i] =                         \
        Bg[(size_t)b_row[i] * kchunks + kc_];                                      \
    if constexpr (DUAL) {                                                          \
      _Pragma("unroll") for (int i = 0; i < LB; ++i) rb2[i] =                      \
          B2g[(size_t)b_row[i] * kchunks + kc_];                                   \
    }                                                                              \
  } while (0)
#define MOE_SSTORE(buf_)                                                           \
  do {                                                                             \
    _Pragma("unroll") for (int i = 0; i < LA; ++i)                                 \
        sm.a[buf_][swz((tid + i * 256) / 8, cpos)] = ra[i];                        \
    _Pragma("unroll") for (int i = 0; i < LB; ++i)                                 \
        sm.b[buf_][swz((tid + i * 256) / 8, cpos)] = rb[i];                        \
    if constexpr (DUAL) {                                                          \
      _Pragma("unroll") for (int i = 0; i < LB; ++i)                               \
          sm.b2[buf_][swz((tid + i * 256) / 8, cpos)] = rb2[i];                    \
    }                                                                              \
  } while (0)

  floatx16 acc[FM][FN];
  floatx16 acc2[DUAL ? FM : 1][DUAL ? FN : 1];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      acc[i][j] = floatx16{};
      if constexpr (DUAL) acc2[i][j] = floatx16{};
    }

  const int ktiles = K / BK;
  MOE_GLOAD(0);
  MOE_SSTORE(0);
  __syncthreads();
  for (int kt = 0; kt < ktiles; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < ktiles) MOE_GLOAD(kt + 1);
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      const int c = kk * 2 + lane / 32;
      bf16x8_t af[FM], bfr[FN], bfr2[DUAL ? FN : 1];
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        const int r = wm * (BM / 2) + i * 32 + lane % 32;
        af[i] = __builtin_bit_cast(bf16x8_t, sm.a[buf][swz(r, c)]);
      }
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int r = wn * (BN / 2) + j * 32 + lane % 32;
        bfr[j] = __builtin_bit_cast(bf16x8_t, sm.b[buf][swz(r, c)]);
        if constexpr (DUAL) bfr2[j] = __builtin_bit_cast(bf16x8_t, sm.b2[buf][swz(r, c)]);
      }
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
          if constexpr (DUAL)
            acc2[i][j] =
                __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr2[j], acc2[i][j], 0, 0, 0);
        }
    }
    if (kt + 1 < ktiles) MOE_SSTORE(buf ^ 1);
    __syncthreads();
  }
#undef MOE_GLOAD
#undef MOE_SSTORE

  // Epilogue: activation, round to bf16, store rows inside [r0, r1).
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int col = n0 + wn * (BN / 2) + j * 32 + lane % 32;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int row = r0 + wm * (BM / 2) + i * 32 + 8 * (v / 4) + 4 * (lane / 32) + (v % 4);
        float o;
        if constexpr (DUAL) o = silu(acc[i][j][v]) * acc2[i][j][v];
        else o = apply_act(acc[i][j][v], ACT);
        if (row < r1 && col < N) C[(size_t)row * N + col] = (bf16_t)f32_to_bf16(o);
      }
    }
}

// ------------------------------------------------------------- fp32 MFMA ---

template <int ACT>
__global__ __launch_bounds__(256) void grouped_gemm_f32(
    const float* __restrict__ A, const float* __restrict__ B, const float* __restrict__ B2,
    float* __restrict__ C, int K, int N, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ tile_start, int E, int n_tiles, int max_rows) {
  constexpr bool DUAL = ACT == ACT_SWIGLU;
  constexpr int BM = 64, BN = 64, BK = 16, LDK = BK + 1;
  __shared__ float As[BM][LDK], Bs[BN][LDK], B2s[DUAL ? BN : 1][LDK];

  int e, r0, r1, nt;
  if (!locate_tile(blockIdx.x, gridDim.x, n_tiles, tile_start, offsets, E, BM, max_rows, e, r0,
                   r1, nt))
    return;
  const int n0 = nt * BN;
  const int tid = threadIdx.x, lane = tid % 64, wave = tid / 64;
  const int wm = wave / 2, wn = wave % 2;  // each wave: 32 x 32 = 2 x 2 blocks of 16x16
  const size_t bexp = (size_t)e * N * K;

  floatx4 acc[2][2], acc2[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      acc[i][j] = floatx4{};
      acc2[i][j] = floatx4{};
    }

  for (int k0 = 0; k0 < K; k0 += BK) {
    __syncthreads();
    for (int q = tid; q < BM * BK; q += 256) {
      const int r = q / BK, kk = q % BK;
      As[r][kk] = A[(size_t)min(r0 + r, r1 - 1) * K + k0 + kk];
      const int n = min(n0 + r, N - 1);
      Bs[r][kk] = B[bexp + (size_t)n * K + k0 + kk];
      if constexpr (DUAL) B2s[r][kk] = B2[bexp + (size_t)n * K + k0 + kk];
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < BK; kk += 4) {
      const int kq = kk + lane / 16;
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const float a = As[wm * 32 + i * 16 + lane % 16][kq];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int n = wn * 32 + j * 16 + lane % 16;
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, Bs[n][kq], acc[i][j], 0, 0, 0);
          if constexpr (DUAL)
            acc2[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, B2s[n][kq], acc2[i][j], 0, 0, 0);
        }
      }
    }
  }
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int col = n0 + wn * 32 + j * 16 + lane % 16;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int row = r0 + wm * 32 + i * 16 + 4 * (lane / 16) + v;
        float o;
        if constexpr (DUAL) o = silu(acc[i][j][v]) * acc2[i][j][v];
        else o = apply_act(acc[i][j][v], ACT);
        if (row < r1 && col < N) C[(size_t)row * N + col] = o;
      }
    }
}

// ---------------------------------------------------------------- launch ---

constexpr int kBf16BM = 128, kBf16BN = 128, kF32BM = 64, kF32BN = 64;

static size_t align256(size_t x) { return (x + 255) / 256 * 256; }

size_t ffn_workspace_bytes(int E, int max_rows, int d, int h, int act, int dtype) {
  (void)d;
  (void)act;
  const size_t elem = dtype == 0 ? 4 : 2;
  return align256((size_t)(E + 1) * sizeof(int32_t)) + align256((size_t)max_rows * h * elem);
}

static int grid_for(int max_rows, int BM, int E, int n_tiles) {
  const long long m_tiles = (long long)(max_rows + BM - 1) / BM + E;
  long long g = m_tiles * n_tiles;
  g = (g + 7) / 8 * 8;  // multiple of 8 for the XCD remap
  return (int)g;
}

static int32_t* ffn_tile_start(const FfnArgs& a) { return static_cast<int32_t*>(a.ws); }
static void* ffn_hidden_buf(const FfnArgs& a) {
  return static_cast<char*>(a.ws) + align256((size_t)(a.E + 1) * sizeof(int32_t));
}
static int ffn_bm(int dtype) { return dtype == 0 ? kF32BM : kBf16BM; }
static int ffn_bn(int dtype) { return dtype == 0 ? kF32BN : kBf16BN; }

hipError_t launch_ffn_plan(const FfnArgs& a, hipStream_t st) {
  ffn_tile_prefix<<<1, 1024, 0, st>>>(a.offsets, a.E, ffn_bm(a.dtype), ffn_tile_start(a));
  return hipGetLastError();
}

hipError_t launch_ffn_up(const FfnArgs& a, hipStream_t st) {
  const int BM = ffn_bm(a.dtype), BN = ffn_bn(a.dtype);
  const int nt = (a.h + BN - 1) / BN;
  const int g = grid_for(a.max_rows, BM, a.E, nt);
  int32_t* ts = ffn_tile_start(a);
  if (a.dtype == 0) {
    const float* X = static_cast<const float*>(a.x_rows);
    const float* W1 = static_cast<const float*>(a.w1);
    const float* W3 = static_cast<const float*>(a.w3);
    float* Hf = static_cast<float*>(ffn_hidden_buf(a));
    if (a.act == ACT_RELU)
      grouped_gemm_f32<ACT_RELU><<<g, 256, 0, st>>>(X, W1, nullptr, Hf, a.d, a.h, a.offsets, ts,
                                                    a.E, nt, a.max_rows);
    else if (a.act == ACT_GELU)
      grouped_gemm_f32<ACT_GELU><<<g, 256, 0, st>>>(X, W1, nullptr, Hf, a.d, a.h, a.offsets, ts,
                                                    a.E, nt, a.max_rows);
    else
      grouped_gemm_f32<ACT_SWIGLU><<<g, 256, 0, st>>>(X, W1, W3, Hf, a.d, a.h, a.offsets, ts,
                                                      a.E, nt, a.max_rows);
  } else {
    const bf16_t* X = static_cast<const bf16_t*>(a.x_rows);
    const bf16_t* W1 = static_cast<const bf16_t*>(a.w1);
    const bf16_t* W3 = static_cast<const bf16_t*>(a.w3);
    bf16_t* Hb = static_cast<bf16_t*>(ffn_hidden_buf(a));
    if (a.act == ACT_RELU)
      grouped_gemm_bf16<kBf16BM, kBf16BN, ACT_RELU><<<g, 256, 0, st>>>(
          X, W1, nullptr, Hb, a.d, a.h, a.offsets, ts, a.E, nt, a.max_rows);
    else if (a.act == ACT_GELU)
      grouped_gemm_bf16<kBf16BM, kBf16BN, ACT_GELU><<<g, 256, 0, st>>>(
          X, W1, nullptr, Hb, a.d, a.h, a.offsets, ts, a.E, nt, a.max_rows);
    else
      grouped_gemm_bf16<kBf16BM, kBf16BN, ACT_SWIGLU><<<g, 256, 0, st>>>(
          X, W1, W3, Hb, a.d, a.h, a.offsets, ts, a.E, nt, a.max_rows);
  }
  return hipGetLastError();
}

hipError_t launch_ffn_down(const FfnArgs& a, hipStream_t st) {
  const int BM = ffn_bm(a.dtype), BN = ffn_bn(a.dtype);
  const int nt = (a.d + BN - 1) / BN;
  const int g = grid_for(a.max_rows, BM, a.E, nt);
  int32_t* ts = ffn_tile_start(a);
  if (a.dtype == 0) {
    grouped_gemm_f32<ACT_NONE><<<g, 256, 0, st>>>(
        static_cast<const float*>(ffn_hidden_buf(a)), static_cast<const float*>(a.w2), nullptr,
        static_cast<float*>(a.y_rows), a.h, a.d, a.offsets, ts, a.E, nt, a.max_rows);
  } else {
    grouped_gemm_bf16<kBf16BM, kBf16BN, ACT_NONE><<<g, 256, 0, st>>>(
        static_cast<const bf16_t*>(ffn_hidden_buf(a)), static_cast<const bf16_t*>(a.w2),
        nullptr, static_cast<bf16_t*>(a.y_rows), a.h, a.d, a.offsets, ts, a.E, nt, a.max_rows);
  }
  return hipGetLastError();
}

}  // namespace moe
