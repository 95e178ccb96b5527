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

// erf(x) by Abramowitz & Stegun, Handbook of Mathematical Functions, formula
// 7.1.26: for x >= 0, erf(x) = 1 - (a1 t + a2 t^2 + a3 t^3 + a4 t^4 + a5 t^5)
// exp(-x^2) with t = 1 / (1 + p x); absolute error <= 1.5e-7 (the fp32
// evaluation adds a few ulp), far below the bf16 rounding H goes through.
// erf is odd, so the sign is restored at the end.
__device__ __forceinline__ float erf_as7126(float x) {
  const float ax = fabsf(x);
  const float t = __frcp_rn(fmaf(0.3275911f, ax, 1.0f));
  float poly = fmaf(1.061405429f, t, -1.453152027f);
  poly = fmaf(poly, t, 1.421413741f);
  poly = fmaf(poly, t, -0.284496736f);
  poly = fmaf(poly, t, 0.254829592f);
  poly *= t;
  const float r = 1.0f - poly * __expf(-ax * ax);
  return copysignf(r, x);
}

__device__ __forceinline__ float apply_act(float u, int act) {
  if (act == ACT_RELU) return fmaxf(u, 0.f);
  if (act == ACT_GELU) return 0.5f * u * (1.f + erf_as7126(u * 0.70710678118654752440f));
  return u;
}

__device__ __forceinline__ float silu(float g) { return g / (1.f + __expf(-g)); }

// ------------------------------------------------------------- tile plan ---

// One block of 1024 threads (E <= 1024): expert e owns ceil(rows_e / BM) row
// tiles; tile q of the batch is tiles[q] = {e, first row, row end, 0}, and
// *count = number of tiles.  Rows are clamped to max_rows.
__global__ __launch_bounds__(1024) void ffn_plan_tiles(const int32_t* __restrict__ offsets,
                                                       int E, int BM, int max_rows,
                                                       int4* __restrict__ tiles,
                                                       int32_t* __restrict__ count) {
  __shared__ int32_t s[1024];
  const int e = threadIdx.x;
  int32_t lo = 0, hi = 0, n = 0;
  if (e < E) {
    lo = min(offsets[e], max_rows);
    hi = min(offsets[e + 1], max_rows);
    n = hi > lo ? (hi - lo + BM - 1) / BM : 0;
  }
  s[e] = n;
  __syncthreads();
  for (int o = 1; o < 1024; o <<= 1) {
    const int32_t v = e >= o ? s[e - o] : 0;
    __syncthreads();
    s[e] += v;
    __syncthreads();
  }
  const int32_t start = s[e] - n;
  for (int q = 0; q < n; ++q) {
    const int32_t r0 = lo + q * BM;
    tiles[start + q] = make_int4(e, r0, min(hi, r0 + BM), 0);
  }
  if (e == E - 1) *count = s[e];
}

// XCD-aware block order.  The hardware deals blocks round-robin over the 8
// XCDs (block b runs on XCD b % 8).  The grid is sized for the worst case, so
// only the first `total` logical tiles (known on the device) are real; XCD x
// takes the contiguous range [x*per, (x+1)*per) of them, per = ceil(total/8),
// so the N tiles of one M tile (same A rows) share that XCD's L2 and every XCD
// gets an equal share.  Returns -1 for blocks with nothing to do.
__device__ __forceinline__ int xcd_logical(int b, int total) {
  const int per = (total + 7) / 8;
  const int slot = b / 8;
  if (slot >= per) return -1;
  const int logical = (b % 8) * per + slot;
  return logical < total ? logical : -1;
}

// ------------------------------------------------------------- bf16 MFMA ---

// LDS rows hold BK bf16 (BK = 32: 64 bytes = four 16-byte chunks).  Chunk c of row r
// lives at c ^ swz(r): consecutive rows reading the same logical chunk then hit
// distinct bank groups for 8- and for 16-lane LDS phases.
__device__ __forceinline__ int swz4(int r) { return ((r >> 1) ^ (r >> 2)) & 3; }
// Same for 128-byte rows (64 bf16, eight chunks).  Both depend on the low four
// row bits only, so rows 16 or 32 apart share the pattern.
__device__ __forceinline__ int swz8(int r) { return (r ^ ((r >> 3) & 1)) & 7; }
template <int BK>
__device__ __forceinline__ int swz(int r) { return BK == 32 ? swz4(r) : swz8(r); }

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// s_waitcnt vmcnt(N), other counters untouched (gfx9 encoding: vmcnt[3:0] in
// bits 3:0 and vmcnt[5:4] in bits 15:14; expcnt 7 and lgkmcnt 15 mean "no wait").
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | (((N >> 4) & 3) << 14));
}

constexpr int kLdsBytes = 160 * 1024;  // LDS per CU (and per workgroup) on gfx950

// Workgroup barrier for the LDS ring.  Before it, each wave has waited for
// its own global->LDS loads of the stage about to be read (explicit
// s_waitcnt vmcnt) and has consumed every LDS read of the stage about to be
// overwritten; the barrier then makes both true for the whole block.  A
// __syncthreads() would also drain the loads of the stages still in flight,
// which is exactly the latency the ring is there to hide, so only compiler
// reordering is fenced here.
__device__ __forceinline__ void ring_barrier() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Grouped GEMM C[rows, N] = act(A[rows, K] B_e[N, K]^T) for bf16.
// Block tile 256 (rows) x BN (columns), K step 32, 4 waves as 2 x 2, wave tile
// 128 x BN/2.  DUAL (SwiGLU): the B stage holds BN rows of W1 (gate) and BN
// rows of W3 (up); the wave keeps both accumulators and combines them in the
// epilogue.  MFMA v_mfma_f32_32x32x16_bf16 with the weight fragment as the
// first operand, so a lane's accumulator holds 4 consecutive output columns of
// one row.  Stages arrive by global_load_lds_dwordx4 (16 bytes per lane,
// straight into LDS) into a 4-deep ring; the XOR swizzle is applied by the
// choice of source address.
template <int BM, int BN, int BK, int WAVES, int ACT>
__global__ __launch_bounds__(WAVES * 64, 1) __attribute__((amdgpu_waves_per_eu(WAVES / 4, WAVES / 4)))
void grouped_gemm_bf16(
    const bf16_t* __restrict__ A, const bf16_t* __restrict__ B, const bf16_t* __restrict__ B2,
    bf16_t* __restrict__ C, int K, int N, const int4* __restrict__ tiles,
    const int32_t* __restrict__ tile_count, int n_tiles) {
  constexpr bool DUAL = ACT == ACT_SWIGLU;
  constexpr int RB = BK * 2;                          // bytes per staged row
  constexpr int CH = BK / 8;                          // 16-byte chunks per row
  constexpr int RPL = 1024 / RB;                      // rows per 1-KB load
  constexpr int KK = BK / 16;                         // MFMA K steps per stage
  constexpr int BROWS = DUAL ? 2 * BN : BN;           // weight rows per stage
  constexpr int ROWS = BM + BROWS;                    // rows per stage
  constexpr int STAGE = ROWS * RB;                    // bytes per stage
  constexpr int NS = kLdsBytes / STAGE < 6 ? kLdsBytes / STAGE : 6;  // ring depth
  constexpr int LOADS = ROWS / RPL / WAVES;           // 1 KB loads per wave per stage
  static_assert(NS >= 3, "the ring needs three stages");
  static_assert(KK % 2 == 0, "register sets alternate per K step");
  constexpr int WGN = WAVES / 2;                      // waves along N (2 along M)
  constexpr int WM = BM / 2, WN = BN / WGN;           // wave tile (rows x output cols)
  constexpr int FM = WM / 32, FN = WN / 32;
  constexpr int FN2 = DUAL ? FN : 1;
  constexpr int EPI_ROW = WN * 2 + 16;                // epilogue LDS row bytes (padded)
  constexpr int EPI = WAVES * WM * EPI_ROW;
  constexpr int SMEM = NS * STAGE > EPI ? NS * STAGE : EPI;
  static_assert(ROWS % (WAVES * RPL) == 0, "stage rows must split evenly over the waves");
  static_assert(WN % 32 == 0, "wave tile must be whole 32-column MFMA blocks");
  __shared__ __attribute__((aligned(1024))) char smem[SMEM];

  const int logical = xcd_logical(blockIdx.x, *tile_count * n_tiles);
  if (logical < 0) return;
  const int mt = logical / n_tiles, nt = logical % n_tiles;
  const int4 tile = tiles[mt];
  const int e = tile.x, r0 = tile.y, r1 = tile.z;
  const int n0 = nt * BN;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WGN, wn = wave % WGN;

  // Per-lane source pointers of this wave's LOADS 1-KB loads (16 rows each).
  const bf16_t* src[LOADS];
#pragma unroll
  for (int i = 0; i < LOADS; ++i) {
    const int q = wave * LOADS + i;           // load index within the stage
    const int sr = q * RPL + lane / CH;       // stage row
    const int c = (lane % CH) ^ swz<BK>(sr);  // logical chunk this lane fetches
    if (sr < BM) {
      const int row = min(r0 + sr, r1 - 1);   // rows past the tile: computed, never stored
      src[i] = A + (size_t)row * K + c * 8;
    } else {
      const int br = sr - BM;
      const bf16_t* W = (DUAL && br >= BN) ? B2 : B;
      const int n = min(n0 + (DUAL ? br % BN : br), N - 1);
      src[i] = W + ((size_t)e * N + n) * K + c * 8;
    }
  }
  // LDS byte offsets (within a stage) of this lane's MFMA fragments; the
  // chunk index of K step kk is (kk * 2 + lane / 32) ^ swizzle(row).
  int xoff[FM], woff[FN], woff2[FN2];
#pragma unroll
  for (int i = 0; i < FM; ++i) xoff[i] = (wm * WM + i * 32 + (lane & 31)) * RB;
#pragma unroll
  for (int j = 0; j < FN; ++j) {
    woff[j] = (BM + wn * WN + j * 32 + (lane & 31)) * RB;
    if constexpr (DUAL) woff2[j] = (BM + BN + wn * WN + j * 32 + (lane & 31)) * RB;
  }
  // Fragment rows differ from lane&31 by multiples of 32 (BM and BN are), and
  // the swizzle only looks at the low four row bits.
  const int sw = swz<BK>(lane & 31);

  // Issue the global->LDS loads of K tile kt_ into ring slot slot_.
#define MOE_RING_ISSUE(kt_, slot_)                                                         \
  do {                                                                                     \
    char* base_ = smem + (slot_) * STAGE + wave * LOADS * 1024;                            \
    _Pragma("unroll") for (int i = 0; i < LOADS; ++i)                                      \
        __builtin_amdgcn_global_load_lds((void*)(src[i] + (kt_) * BK),                     \
                                         (lds_ptr_t)(base_ + i * 1024), 16, 0, 0);         \
  } while (0)
  // Read the fragments of K step kk_ of ring slot slot_ into set S.
#define MOE_LOAD_KK(slot_, kk_, S)                                                         \
  do {                                                                                     \
    const char* st_ = smem + (slot_) * STAGE + ((((kk_) * 2 + (lane >> 5)) ^ sw) << 4);     \
    _Pragma("unroll") for (int i = 0; i < FM; ++i)                                         \
        xf##S[i] = *reinterpret_cast<const bf16x8_t*>(st_ + xoff[i]);                      \
    _Pragma("unroll") for (int j = 0; j < FN; ++j) {                                       \
      wf##S[j] = *reinterpret_cast<const bf16x8_t*>(st_ + woff[j]);                        \
      if constexpr (DUAL) vf##S[j] = *reinterpret_cast<const bf16x8_t*>(st_ + woff2[j]);   \
    }                                                                                      \
  } while (0)
#define MOE_MFMA_KK(S)                                                                     \
  do {                                                                                     \
    _Pragma("unroll") for (int i = 0; i < FM; ++i)                                         \
    _Pragma("unroll") for (int j = 0; j < FN; ++j) {                                       \
      acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf##S[j], xf##S[i], acc[i][j],   \
                                                          0, 0, 0);                        \
      if constexpr (DUAL)                                                                  \
        acc2[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf##S[j], xf##S[i],           \
                                                             acc2[i][j], 0, 0, 0);         \
    }                                                                                      \
  } while (0)
  // Wait until the next stage's loads have landed in every wave: at most
  // `later` younger stages may still be in flight (vmcnt counts 1-KB loads).
#define MOE_WAIT_STAGE(later_)                                                             \
  do {                                                                                     \
    switch (later_) {                                                                      \
      case 0: wait_vmcnt<0>(); break;                                                      \
      case 1: wait_vmcnt<LOADS>(); break;                                                  \
      case 2: wait_vmcnt<2 * LOADS>(); break;                                              \
      case 3: wait_vmcnt<3 * LOADS>(); break;                                              \
      default: wait_vmcnt<4 * LOADS>(); break;                                             \
    }                                                                                      \
    ring_barrier();                                                                        \
  } while (0)

  floatx16 acc[FM][FN];
  floatx16 acc2[DUAL ? FM : 1][FN2];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      acc[i][j] = floatx16{};
      if constexpr (DUAL) acc2[i][j] = floatx16{};
    }
  // Two register sets, one K step (16) each: set 0 holds step 0 of a tile,
  // set 1 step 1.  Each set is refilled while the other one feeds the MFMAs.
  bf16x8_t xf0[FM], wf0[FN], vf0[FN2];
  bf16x8_t xf1[FM], wf1[FN], vf1[FN2];

  const int ktiles = K / BK;
#pragma unroll
  for (int s = 0; s < NS - 1; ++s)
    if (s < ktiles) MOE_RING_ISSUE(s, s);
  MOE_WAIT_STAGE(min(NS - 2, ktiles - 1));
  MOE_LOAD_KK(0, 0, 0);
  for (int kt = 0; kt < ktiles; ++kt) {
    const int slot = kt % NS;
#pragma unroll
    for (int kk = 0; kk < KK; kk += 2) {
      MOE_LOAD_KK(slot, kk + 1, 1);
      MOE_MFMA_KK(0);
      if (kk + 2 < KK) {
        MOE_LOAD_KK(slot, kk + 2, 0);
      } else if (kt + 1 < ktiles) {
        // Tile kt+1 visible to all waves; every wave is past its reads of
        // tile kt-1, so that slot can be refilled.
        MOE_WAIT_STAGE(min(NS - 3, ktiles - kt - 2));
        if (kt + NS - 1 < ktiles) MOE_RING_ISSUE(kt + NS - 1, (kt + NS - 1) % NS);
        MOE_LOAD_KK((kt + 1) % NS, 0, 0);
      }
      MOE_MFMA_KK(1);
    }
  }
#undef MOE_LOAD_KK
#undef MOE_MFMA_KK
#undef MOE_WAIT_STAGE
#undef MOE_RING_ISSUE

  // Epilogue: activation, bf16, through LDS to 16-byte row stores.
  ring_barrier();
  char* ep = smem + wave * WM * EPI_ROW;
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        float o[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const float a = acc[i][j][4 * g + u];
          if constexpr (DUAL) o[u] = silu(a) * acc2[i][j][4 * g + u];
          else o[u] = apply_act(a, ACT);
        }
        const int m = i * 32 + (lane & 31);
        const int n = j * 32 + 8 * g + 4 * (lane >> 5);
        uint2 packed = make_uint2(pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]));
        *reinterpret_cast<uint2*>(ep + m * EPI_ROW + n * 2) = packed;
      }
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's LDS writes are done
  __builtin_amdgcn_wave_barrier();
  constexpr int CPR = WN / 8;          // 16-byte chunks per output row
  constexpr int RPI = 64 / CPR;        // rows per wave instruction
  const int row_base = r0 + wm * WM;
  const int col_base = n0 + wn * WN;
#pragma unroll 4
  for (int it = 0; it < WM / RPI; ++it) {
    const int m = it * RPI + lane / CPR;
    const int ch = lane % CPR;
    const int row = row_base + m, col = col_base + ch * 8;
    if (row < r1 && col < N) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(ep + m * EPI_ROW + ch * 16);
      *reinterpret_cast<u32x4*>(C + (size_t)row * N + col) = v;
    }
  }
}

// ------------------------------------------------------------- fp32 MFMA ---

template <int ACT>
__global__ __launch_bounds__(256) void grouped_gemm_f32(
    const float* __restrict__ A, const float* __restrict__ B, const float* __restrict__ B2,
    float* __restrict__ C, int K, int N, const int4* __restrict__ tiles,
    const int32_t* __restrict__ tile_count, int n_tiles) {
  constexpr bool DUAL = ACT == ACT_SWIGLU;
  constexpr int BM = 64, BN = 64, BK = 16, LDK = BK + 1;
  __shared__ float As[BM][LDK], Bs[BN][LDK], B2s[DUAL ? BN : 1][LDK];

  const int logical = xcd_logical(blockIdx.x, *tile_count * n_tiles);
  if (logical < 0) return;
  const int mt = logical / n_tiles, nt = logical % n_tiles;
  const int4 tile = tiles[mt];
  const int e = tile.x, r0 = tile.y, r1 = tile.z;
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

constexpr int kBf16BM = 256, kBf16Waves = 8, kF32BM = 64, kF32BN = 64;

static size_t align256(size_t x) { return (x + 255) / 256 * 256; }

static int ffn_bm(int dtype) { return dtype == 0 ? kF32BM : kBf16BM; }

// Upper bound of row tiles: every expert may end in a partial tile.
static int max_m_tiles(int max_rows, int BM, int E) { return (max_rows + BM - 1) / BM + E; }

static size_t ffn_plan_bytes(int E, int max_rows, int dtype) {
  return align256(sizeof(int32_t)) +
         align256((size_t)max_m_tiles(max_rows, ffn_bm(dtype), E) * sizeof(int4));
}

size_t ffn_workspace_bytes(int E, int max_rows, int d, int h, int act, int dtype) {
  (void)d;
  (void)act;
  const size_t elem = dtype == 0 ? 4 : 2;
  return ffn_plan_bytes(E, max_rows, dtype) + align256((size_t)max_rows * h * elem);
}

static int32_t* ffn_count(const FfnArgs& a) { return static_cast<int32_t*>(a.ws); }
static int4* ffn_tiles(const FfnArgs& a) {
  return reinterpret_cast<int4*>(static_cast<char*>(a.ws) + align256(sizeof(int32_t)));
}
static void* ffn_hidden_buf(const FfnArgs& a) {
  return static_cast<char*>(a.ws) + ffn_plan_bytes(a.E, a.max_rows, a.dtype);
}

static int grid_of(int m_tiles, int n_tiles) {
  const long long g = (long long)m_tiles * n_tiles;
  return (int)((g + 7) / 8 * 8);  // 8 * per >= any real tile count
}

hipError_t launch_ffn_plan(const FfnArgs& a, hipStream_t st) {
  ffn_plan_tiles<<<1, 1024, 0, st>>>(a.offsets, a.E, ffn_bm(a.dtype), a.max_rows, ffn_tiles(a),
                                     ffn_count(a));
  return hipGetLastError();
}

template <int BN, int BK, int ACT>
static void launch_bf16(const bf16_t* A, const bf16_t* B, const bf16_t* B2, bf16_t* C, int K,
                        int N, const FfnArgs& a, hipStream_t st) {
  const int nt = (N + BN - 1) / BN;
  const int g = grid_of(max_m_tiles(a.max_rows, kBf16BM, a.E), nt);
  grouped_gemm_bf16<kBf16BM, BN, BK, kBf16Waves, ACT><<<g, kBf16Waves * 64, 0, st>>>(A, B, B2, C, K, N, ffn_tiles(a), ffn_count(a), nt);
}

template <int ACT>
static void launch_f32(const float* A, const float* B, const float* B2, float* C, int K, int N,
                       const FfnArgs& a, hipStream_t st) {
  const int nt = (N + kF32BN - 1) / kF32BN;
  const int g = grid_of(max_m_tiles(a.max_rows, kF32BM, a.E), nt);
  grouped_gemm_f32<ACT><<<g, 256, 0, st>>>(A, B, B2, C, K, N, ffn_tiles(a), ffn_count(a), nt);
}

hipError_t launch_ffn_up(const FfnArgs& a, hipStream_t st) {
  if (a.dtype == 0) {
    auto X = static_cast<const float*>(a.x_rows);
    auto W1 = static_cast<const float*>(a.w1);
    auto W3 = static_cast<const float*>(a.w3);
    auto H = static_cast<float*>(ffn_hidden_buf(a));
    if (a.act == ACT_RELU) launch_f32<ACT_RELU>(X, W1, nullptr, H, a.d, a.h, a, st);
    else if (a.act == ACT_GELU) launch_f32<ACT_GELU>(X, W1, nullptr, H, a.d, a.h, a, st);
    else launch_f32<ACT_SWIGLU>(X, W1, W3, H, a.d, a.h, a, st);
  } else {
    auto X = static_cast<const bf16_t*>(a.x_rows);
    auto W1 = static_cast<const bf16_t*>(a.w1);
    auto W3 = static_cast<const bf16_t*>(a.w3);
    auto H = static_cast<bf16_t*>(ffn_hidden_buf(a));
    if (a.act == ACT_SWIGLU) launch_bf16<128, 32, ACT_SWIGLU>(X, W1, W3, H, a.d, a.h, a, st);
    else if (a.h >= 2048) {
      if (a.act == ACT_RELU) launch_bf16<256, 32, ACT_RELU>(X, W1, nullptr, H, a.d, a.h, a, st);
      else launch_bf16<256, 32, ACT_GELU>(X, W1, nullptr, H, a.d, a.h, a, st);
    } else {
      if (a.act == ACT_RELU) launch_bf16<128, 32, ACT_RELU>(X, W1, nullptr, H, a.d, a.h, a, st);
      else launch_bf16<128, 32, ACT_GELU>(X, W1, nullptr, H, a.d, a.h, a, st);
    }
  }
  return hipGetLastError();
}

hipError_t launch_ffn_down(const FfnArgs& a, hipStream_t st) {
  if (a.dtype == 0) {
    launch_f32<ACT_NONE>(static_cast<const float*>(ffn_hidden_buf(a)),
                         static_cast<const float*>(a.w2), nullptr, static_cast<float*>(a.y_rows),
                         a.h, a.d, a, st);
  } else {
    auto H = static_cast<const bf16_t*>(ffn_hidden_buf(a));
    auto W2 = static_cast<const bf16_t*>(a.w2);
    auto Y = static_cast<bf16_t*>(a.y_rows);
    if (a.d >= 1024) launch_bf16<256, 32, ACT_NONE>(H, W2, nullptr, Y, a.h, a.d, a, st);
    else launch_bf16<128, 32, ACT_NONE>(H, W2, nullptr, Y, a.h, a.d, a, st);
  }
  return hipGetLastError();
}

}  // namespace moe
