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
// Scheduling: a prologue kernel turns the per-expert row counts into a list
// of row tiles (each expert split into equal tiles of at most BM rows).  The
// GEMM grid is sized for the worst case (max_rows/BM + E tiles); block b is
// remapped so that consecutive logical tiles run on the same XCD (the
// hardware deals blocks round-robin over the 8 XCDs), logical tiles walk the N
// tiles of one row tile first (A rows reused from that XCD's L2), and blocks
// past the real tile count exit at once.
//
// bf16 kernel (grouped_gemm_bf16): 8 waves, tiles of up to 320 rows, operands
// streamed global -> LDS by direct DMA into a multi-stage ring, MFMA
// v_mfma_f32_32x32x16_bf16, epilogue straight from registers.  Details at the
// kernel.
//
// fp32 kernel (fp32 workloads): v_mfma_f32_16x16x4_f32, 64x64 tiles, K step
// 16, plain padded LDS rows.
#include <algorithm>

#include "device.h"
#include "kernels.h"

namespace moe {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

enum { ACT_RELU = 0, ACT_GELU = 1, ACT_SWIGLU = 2, ACT_NONE = 3 };

// GELU(u) = 0.5 u (1 + erf(u / sqrt 2)) with erf from Abramowitz & Stegun,
// Handbook of Mathematical Functions, formula 7.1.26: for x >= 0,
// erf(x) = 1 - P(t) exp(-x^2), P(t) = a1 t + a2 t^2 + a3 t^3 + a4 t^4 + a5 t^5,
// t = 1 / (1 + p x), absolute error <= 1.5e-7.  erf is odd, so with x = |u|/sqrt 2
// the factor 1 + erf is 2 - P e for u >= 0 and P e for u < 0 (e = exp(-u^2/2)),
// and both cases are GELU(u) = max(u, 0) - 0.5 |u| P e.  The code folds 1/sqrt 2
// into p and the 0.5 into the a_i, and takes e as 2^(-u^2 log2(e) / 2) on
// v_exp_f32.  t comes from v_rcp_f32 (within 2 ulp on gfx950); the fp32
// evaluation adds a few ulp, all far below the bf16 rounding H goes through.
// The same evaluation with its parts kept for the backward: h = GELU(u), and
// tqe = t q e = P(t) e / 2, so that Phi(u) = 1 - tqe (u >= 0) or tqe (u < 0).
__device__ __forceinline__ void gelu_as7126_parts(float u, float& h, float& tqe, float& e) {
  const float a = fabsf(u);
  const float t = __builtin_amdgcn_rcpf(fmaf(0.3275911f * 0.70710678118654752440f, a, 1.0f));
  float q = fmaf(0.5f * 1.061405429f, t, 0.5f * -1.453152027f);
  q = fmaf(q, t, 0.5f * 1.421413741f);
  q = fmaf(q, t, 0.5f * -0.284496736f);
  q = fmaf(q, t, 0.5f * 0.254829592f);
  e = __builtin_amdgcn_exp2f(u * u * -0.72134752044448170368f);
  h = fmaf(-(a * t), q * e, fmaxf(u, 0.f));
  tqe = t * (q * e);
}

__device__ __forceinline__ float gelu_as7126(float u) {
  float h, tqe, e;
  gelu_as7126_parts(u, h, tqe, e);
  return h;
}

__device__ __forceinline__ float apply_act(float u, int act) {
  if (act == ACT_RELU) return fmaxf(u, 0.f);
  if (act == ACT_GELU) return gelu_as7126(u);
  return u;
}

// g sigmoid(g); v_rcp_f32 (within 2 ulp) in place of an IEEE divide.
__device__ __forceinline__ float silu(float g) { return g * __builtin_amdgcn_rcpf(1.f + __expf(-g)); }

// H = act(u) [* v], du = g act'(u) [* v], dv = g silu(u) (SwiGLU), all in
// fp32, for the backward.  H comes from the forward's own expressions
// (gelu_as7126, silu).  GELU: gelu(u) = u Phi(u) and gelu'(u) = Phi(u) +
// u phi(u), with Phi from the same formula 7.1.26 evaluation (its absolute
// error 1.5e-7 / 2) and phi(u) = e / sqrt(2 pi) from the same e = exp(-u^2/2).
template <int ACT>
__device__ __forceinline__ void bwd_act_grad(float u, float v, float g, float& hv, float& du,
                                             float& dv) {
  if constexpr (ACT == ACT_RELU) {
    hv = fmaxf(u, 0.f);
    du = u > 0.f ? g : 0.f;
    dv = 0.f;
  } else if constexpr (ACT == ACT_GELU) {
    float tqe, e;
    gelu_as7126_parts(u, hv, tqe, e);
    const float Phi = u >= 0.f ? 1.f - tqe : tqe;
    du = g * fmaf(u * 0.39894228040143268f, e, Phi);
    dv = 0.f;
  } else {
    const float s = __builtin_amdgcn_rcpf(1.f + __expf(-u)), si = u * s;
    hv = si * v;
    du = g * v * (s * (1.f + u * (1.f - s)));
    dv = g * si;
  }
}

// ------------------------------------------------------------- tile plan ---

// One block of 1024 threads (E <= 1024): expert e owns n_e = ceil(rows_e / BM)
// row tiles of equal height, rounded up to whole 32-row MFMA fragments
// (chunk_e = 32 ceil(ceil(rows_e / n_e) / 32) <= BM; since (n_e - 1) BM <
// rows_e, no tile is empty).  The tiles are {e, first row, row end, first
// 16-row group}, numbered in expert order, and *count = number of tiles; the
// list may then be reordered (longest first, below).  The group
// numbering gives every tile ceil(rows / 16) groups of its own, in expert order:
// the packed hidden buffer of the bf16 FFN stores a tile's rows there.  Rows
// are clamped to max_rows and, when group_rows is given, each segment to its
// first group_rows[e] rows.  Nondecreasing offsets need at most cap_tiles
// tiles and cap_groups groups (the workspace's sizes); a tile past either is
// not written, and count[0] stops before the first such tile.  count[1] is
// the row-tile group size of the GEMMs' block order (see tile_of), count[2]
// the row tile height BM.
// Inclusive scan over the 1024 threads of a block: shuffles inside each wave,
// then the 16 wave totals (two barriers instead of a Hillis-Steele loop).
__device__ __forceinline__ int32_t block_scan_1024(int32_t v, int32_t* wsum) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int32_t u = __shfl_up(v, o, 64);
    if (lane >= o) v += u;
  }
  __syncthreads();  // wsum is free (a previous scan may still be reading it)
  if (lane == 63) wsum[wv] = v;
  __syncthreads();
  for (int w = 0; w < wv; ++w) v += wsum[w];
  return v;
}

// Experts averaging at most this many rows take the 192-row tiles.
constexpr int kMidRowsPerExpert = 128;

// BMalt > 0: the plan picks its row tile height itself, BMalt when the
// segments hold at most kMidRowsPerExpert rows per expert on average, else BM,
// and stores it in count[2] (the GEMMs that serve both read it there).
__global__ __launch_bounds__(1024) void ffn_plan_tiles(const int32_t* __restrict__ offsets,
                                                       const int32_t* __restrict__ group_rows,
                                                       int E, int BM, int BMalt, int max_rows,
                                                       int cap_tiles, int cap_groups,
                                                       int4* __restrict__ tiles,
                                                       int32_t* __restrict__ count) {
  __shared__ int32_t wsum[16];
  __shared__ int32_t total_s, first_bad_s, multi_s, rows_s;
  __shared__ __align__(16) int32_t keys_l[1024];
  __shared__ int32_t rank_l[1024];
  const int e = threadIdx.x;
  if (e == 0) {
    first_bad_s = 0x7fffffff;
    multi_s = 0;
    rows_s = 0;
  }
  int32_t lo = 0, hi = 0, n = 0;
  if (e < E) {
    lo = min(offsets[e], max_rows);
    hi = min(offsets[e + 1], max_rows);
    if (group_rows) hi = min(hi, lo + max(group_rows[e], 0));
  }
  __syncthreads();
  if (hi > lo) atomicAdd(&rows_s, hi - lo);
  __syncthreads();
  const int bm = BMalt > 0 && (long long)rows_s <= (long long)kMidRowsPerExpert * E ? BMalt : BM;
  int32_t chunk = bm;
  if (e < E) {
    n = hi > lo ? (hi - lo + bm - 1) / bm : 0;
    if (n > 0) chunk = ((hi - lo + n - 1) / n + 31) / 32 * 32;
  }
  const int32_t n_incl = block_scan_1024(n, wsum);  // its first barrier orders multi_s = 0
  if (n >= 2) atomicAdd(&multi_s, n);
  const int32_t start = n_incl - n;
  if (e == E - 1) total_s = n_incl;
  // 16-row groups of this expert's tiles, then their exclusive prefix.
  int32_t ng = 0;
  for (int q = 0; q < n; ++q) ng += (min(hi, lo + (q + 1) * chunk) - (lo + q * chunk) + 15) / 16;
  int32_t g0 = block_scan_1024(ng, wsum) - ng;
  for (int q = 0; q < n; ++q) {
    const int32_t r0 = lo + q * chunk, r1 = min(hi, r0 + chunk);
    const int32_t g1 = g0 + (r1 - r0 + 15) / 16;
    if (start + q < cap_tiles && g1 <= cap_groups) {
      tiles[start + q] = make_int4(e, r0, r1, g0);
    } else {
      atomicMin(&first_bad_s, start + q);
      break;
    }
    g0 = g1;
  }
  __syncthreads();
  const int T = total_s;
  const bool grouped = T > 0 && 4 * multi_s >= T;
  if (e == 0) {
    count[0] = min(T, first_bad_s);
    // Block order of the GEMMs (tile_of): groups of 4 row tiles once a quarter
    // of the row tiles belong to experts of two or more.
    count[1] = grouped ? 4 : 1;
    count[2] = bm;
  }
  // Longest tiles first.  With one row tile per group the GEMMs hand XCD x
  // the x-th eighth of the logical tiles, and an XCD's blocks start in order
  // as its CUs free up: the row tiles are stored by decreasing row count
  // (ties by position), dealt round-robin to the eight XCD ranges, so every
  // XCD gets an equal mix and runs its shortest tiles last (a greedy
  // longest-first schedule; experts of 50 to 232 rows give tiles whose time
  // differs by their A rows and live fragments).  Batches of short tiles
  // (under 64 rows on average: decode-sized) keep expert order, which
  // measured faster there.  Only a tile's place in the list changes, never
  // its contents, so no output depends on the order.
  if (!grouped && T > 8 && T <= 1024 && first_bad_s >= T && rows_s >= 64 * T) {
    // Unique keys (row count, then earlier position first); a tile's rank is
    // the number of larger keys.  sub threads share a tile, each counting
    // over a quarter (or third, half) of the keys, four per LDS read.
    const int T4 = (T + 3) / 4;
    const int sub = min(4, 1024 / T);
    int4 mine = make_int4(0, 0, 0, 0);
    if (e < T) {
      mine = tiles[e];
      rank_l[e] = 0;
    }
    if (e < 4 * T4) keys_l[e] = e < T ? (mine.z - mine.y) * 1024 + (1023 - e) : -1;
    __syncthreads();
    const int t = e / sub, part = e % sub;
    if (t < T) {
      const int key = keys_l[t];
      const int4* keys4 = reinterpret_cast<const int4*>(keys_l);
      const int b0 = part * T4 / sub, b1 = (part + 1) * T4 / sub;
      int rank = 0;
#pragma unroll 4
      for (int q4 = b0; q4 < b1; ++q4) {
        const int4 o = keys4[q4];
        rank += (o.x > key) + (o.y > key) + (o.z > key) + (o.w > key);
      }
      atomicAdd(&rank_l[t], rank);
    }
    __syncthreads();
    if (e < T) {
      const int rank = rank_l[e];
      const int x = rank & 7;
      int pos = rank >> 3;
      for (int y = 0; y < x; ++y) pos += (T - y + 7) >> 3;
      tiles[pos] = mine;
    }
  }
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

// Logical tile -> (row tile, column tile).  gm == 1: row-major (the column
// tiles of one row tile are consecutive).  gm > 1: groups of gm consecutive row
// tiles walk their column tiles together, so the blocks an XCD runs at once
// (32 consecutive logical tiles) cover gm row tiles x 32/gm column tiles and
// share both the A rows and the weight slabs in that XCD's L2.  The last group
// may hold fewer row tiles.
__device__ __forceinline__ void tile_of(int logical, int n_tiles, int m_tiles, int gm, int& mt,
                                        int& nt) {
  if (gm <= 1) {
    mt = logical / n_tiles;
    nt = logical % n_tiles;
    return;
  }
  const int g = logical / (gm * n_tiles), idx = logical % (gm * n_tiles);
  const int rows = min(gm, m_tiles - g * gm);
  mt = g * gm + idx % rows;
  nt = idx / rows;
}

// ------------------------------------------------------------- bf16 MFMA ---

// Rows per slab of packed weights (rows = N of the GEMM, a multiple of 64): a
// slab's K stage is one contiguous run of SR * 64 bytes.
__host__ __device__ __forceinline__ int packed_slab_rows(int N) { return N % 256 == 0 ? 256 : 64; }

// Grouped GEMM C[rows, N] = act(A[rows, K] B_e[N, K]^T) for bf16.
//
// Block: 8 waves, tile of up to BM = 320 rows x BN columns, K step 32.  The
// waves form 2 (along M) x 4 (along N); wave (wm, wn) owns the 32-row
// fragments f = 2i + wm (i < 5) of the tile -- alternate fragments, so a
// short tile leaves the two M waves (which share a SIMD) equally loaded -- and
// the output columns [wn*BN/4, (wn+1)*BN/4).  Fragments holding no row of the
// tile are skipped: each number of live fragments has its own copy of the
// accumulators, K loop and epilogue, and the wave runs the copy that matches
// its share.  320-row tiles take a whole expert of up to 320 rows (one tile
// per expert at capacity factor 1.25 of 256 rows per expert); 160 x 64 wave
// tiles (160 accumulators) leave room for two waves per SIMD.  192-row tiles
// go up to 512 weight rows per stage (SwiGLU 256 columns of W1 and of W3, the
// down GEMM 512 columns): 96 x 128 wave tiles, 192 accumulators, one register
// set of fragments.  Every column tile re-reads the tile's A rows (from L2),
// and those reads share each CU's load path with the weight stream, so the
// wider tile (half the A reads) streams weights faster.
//
// MFMA v_mfma_f32_32x32x16_bf16 with the weight fragment as the first operand,
// so a lane's accumulator holds 4 consecutive output columns of one row.
// DUAL (SwiGLU): the B stage holds BN rows of W1 (gate) and BN rows of W3
// (up); the wave keeps both accumulators and combines them in the epilogue.
//
// Operands reach LDS by buffer_load_dwordx4 ... lds (16 bytes per lane, 1 KB
// = 16 rows of 64 bytes per instruction) into a ring of NS stages; waves 0-3
// fetch the A rows (XOR swizzle applied through the choice of source address),
// waves 4-7 the weight rows.  A stage's slot is refilled right after the
// barrier that follows its last LDS reads, so NS - 1 stages are in flight
// while one is consumed.  Weights come packed (moe_expert_ffn_pack_weights)
// so that one stage of a slab of 64 or 256 weight rows is one contiguous run
// already in LDS order: the weight stream reads long sequential runs of HBM.
// The epilogue converts to bf16 in registers (v_cvt_pk_bf16_f32), swaps
// half-rows between lanes l and l+32 (v_permlane32_swap) so each lane owns 8
// consecutive columns, and stores 16 bytes per lane straight to global memory.
constexpr int kGemmBM = 320, kGemmBMMid = 192, kGemmBMSmall = 128, kGemmWaves = 8;
// Cache-policy bits of the weight loads (nt | sc1 on gfx950): each weight
// byte is read once per launch, so it is fetched as streaming data.  Measured
// with the operand stream alone (no MFMA): 0.98 against 1.04 us per K stage.
constexpr int kWeightCpol = 2 | 16;

// MODE kUpGemm: A = the permuted rows (row-major [rows, K]), C = the packed
// hidden buffer.  MODE kDownGemm: A = the packed hidden buffer, C = row-major
// [rows, N].  The packed hidden buffer holds, for K stage t (32 columns) and
// 16-row group g (tiles[q].w numbers a tile's groups), one 1-KB block at
// element offset (t * ldg + g) * 512, laid out as the A stage rows sit in LDS
// (16-byte position L: row L/4 of the group, logical chunk (L % 4) ^ swz4(L/4)),
// so a down tile's K stage is one contiguous run.  MODE kDownFused: the down
// GEMM with the combine folded in: no C; each output row, rounded to bf16, is
// scaled by its routing weight and added into the token's fp32 accumulator
// row with hardware float atomics.  For that epilogue the MFMA operands are
// swapped (A fragment first), so a lane holds one output column of 16 rows and
// the 32 lanes of a half-wave cover 32 consecutive columns of one row: each
// atomic instruction touches two 128-byte runs instead of 64 scattered words.
//
// Two modes serve the backward of the expert FFN (u = x W1^T, v = x W3^T; the
// gradient at H is g = dy W2):
// MODE kUpRawF32: the up GEMM with no activation; u (and for SwiGLU v) go out
//   as fp32, row-major [rows, N], to be.U and be.V.
// MODE kBwdG: A = dy rows (row-major [rows, K = d]), B = W2^T packed (N = h):
//   the product is g; the epilogue reads u (and v) at the same positions and
//   forms H = act(u) [* v], du = g act'(u) [* v] and, for SwiGLU, dv =
//   g silu(u) (the activation named by ACT, with a single B operand), each
//   rounded to bf16: H row-major to be.H ([rows, N]); G = [du | dv] row-major
//   to be.G ([rows, kg], kg = N or 2N) and in the packed layout to C (K = kg:
//   dv's columns follow du's), where the dx GEMM reads it as its A.
// MODE kWgrad: the weight gradients, C[m, n] = sum over an expert's rows r of
//   A[r][m] B[r][n] (dW1 | dW3 from G and x, dW2 from dy and H): per expert a
//   GEMM whose reduction runs over its rows, padded to kst[e+1] - kst[e]
//   stages of 32 rows (zero rows past the segment).  A comes transposed in the
//   packed-A layout (block (kst[e] + t) * M/16 + m/16, as the down GEMM's A with
//   groups over m), B transposed in the weights' slab layout from element
//   kst[e] * 32 * N on (slab s of the expert at s * kt_e * SR * 32).  Output
//   rows m < split go to U ([E, split, N] fp32), the others to V ([E, M -
//   split, N]); an expert without rows gets zeros.
enum { kUpGemm = 0, kDownGemm = 1, kDownFused = 2, kUpRawF32 = 3, kBwdG = 4, kWgrad = 5 };

struct BwdEpiArgs {
  float* U;       // kUpRawF32: written; kBwdG: read; kWgrad: the first output
  float* V;       // SwiGLU only; kWgrad: the second output
  bf16_t* G;      // kBwdG: [du | dv] row-major, kg columns
  bf16_t* H;      // kBwdG: H row-major, N columns
  int kg;         // kBwdG: columns of G; kWgrad: rows of the first output
  int M;          // kWgrad: rows of C
  const int32_t* kst;  // kWgrad: stage offset of each expert, [E + 1]
};

// LDS bytes of one tile configuration (the ring the body below lays out).
template <int BM, int BN, int ACT, int MODE>
struct GemmLds {
  static constexpr bool DUAL = ACT == ACT_SWIGLU && MODE != kBwdG;
  static constexpr int RB = 64, BROWS = DUAL ? 2 * BN : BN, STAGE = (BM + BROWS) * RB;
  static constexpr int NS = kLdsBytes / STAGE < 6 ? kLdsBytes / STAGE : 6;
  static constexpr bool AP = MODE == kUpGemm || MODE == kUpRawF32 || MODE == kBwdG;
  static constexpr int ASLOT = BM * 2 * RB, WST = BROWS * RB;
  static constexpr int NW_ = (kLdsBytes - 2 * ASLOT) / WST;
  static constexpr int NW = AP ? (NW_ < 8 ? NW_ : 8) : NS;
  static constexpr int bytes = AP ? 2 * ASLOT + NW * WST : NS * STAGE;
};

// The kernel body, inlined into the kernels below; smem is the block's LDS
// array (GemmLds<...>::bytes at least, 1-KB aligned), m_tiles the plan's row
// tile count and gm its block-order group size.
template <int BM, int BN, int ACT, int MODE>
__device__ __forceinline__ void gemm_bf16_body(
    char* smem, const bf16_t* __restrict__ A, const bf16_t* __restrict__ B,
    const bf16_t* __restrict__ B2, bf16_t* __restrict__ C, int K, int N,
    const int4* __restrict__ tiles, int m_tiles, int n_tiles, int ldg, int gm, FusedCombineArgs fc,
    BwdEpiArgs be) {
  constexpr bool DUAL = ACT == ACT_SWIGLU && MODE != kBwdG;  // two B operands
  constexpr int BK = 32, RB = BK * 2;  // RB: bytes per staged row
  constexpr int RPL = 1024 / RB;                     // rows per 1-KB load
  constexpr int KK = BK / 16;                        // MFMA K steps per stage
  constexpr int BROWS = DUAL ? 2 * BN : BN;          // weight rows per stage
  constexpr int STAGE = (BM + BROWS) * RB;           // bytes per stage
  constexpr int NS = kLdsBytes / STAGE < 6 ? kLdsBytes / STAGE : 6;  // ring depth
  constexpr int LA = BM / RPL / 4;                   // loads per stage, A waves (0-3)
  constexpr int LB = BROWS / RPL / 4;                // loads per stage, B waves (4-7)
  constexpr int LMAX = LA > LB ? LA : LB;
  constexpr int WN = BN / 4;                         // output columns per wave
  constexpr int FM = BM / 64, FN = WN / 32;          // fragments per wave
  constexpr int FN2 = DUAL ? FN : 1;
  // Up GEMM (AP): the A rows are fetched as 128-byte pieces covering two K
  // stages (full cache lines, half the requests of 64-byte pieces) into two
  // pair slots; the weights keep their own ring of NW single stages.
  constexpr bool AP = MODE == kUpGemm || MODE == kUpRawF32 || MODE == kBwdG;
  constexpr bool FUSED = MODE == kDownFused;
  constexpr int ASLOT = BM * 2 * RB;                   // bytes of one A pair slot
  constexpr int WST = BROWS * RB;                      // bytes of one weight stage
  constexpr int NW_ = (kLdsBytes - 2 * ASLOT) / WST;
  constexpr int NW = AP ? (NW_ < 8 ? NW_ : 8) : NS;    // weight ring depth
  constexpr int LA2 = BM / 8 / 4;                      // A loads per pair, A waves (0-3)
  constexpr int LDSB = AP ? 2 * ASLOT + NW * WST : NS * STAGE;
  // Accumulator blocks (16 registers each) of a wave with all FM fragments
  // live.  Up to 10 (160 registers) the fragments of the two K steps of a
  // stage sit in two register sets, one refilled while the other feeds the
  // MFMAs; wider wave tiles (192 accumulators) keep one set, refilled between
  // the K steps, so the wave fits its 256 registers (two waves per SIMD: the
  // other wave's MFMAs run while this one waits on its LDS reads).
  constexpr int ACCB = FM * FN * (DUAL ? 2 : 1);
  constexpr bool ONESET = ACCB > 10;
  static_assert(ACCB <= 12, "at most 192 accumulators per wave");
  static_assert(!AP || (NW >= 3 && NW - 2 <= 6 && (NW - 1) * LB < 64 && 2 * LA2 < 64),
                "pair ring: A pairs two stages ahead, weight waits covered below");
  static_assert(NS >= 3 && NS - 1 <= 7, "the ring needs three stages; waits cover up to 7");
  static_assert(KK == 2, "register sets alternate per K step");
  static_assert(BM % (4 * RPL) == 0 && BROWS % (4 * RPL) == 0, "loads split over 4 waves");
  static_assert(WN % 32 == 0, "wave tile must be whole 32-column MFMA blocks");
  static_assert((NS - 1) * LMAX < 64, "loads in flight must fit the 6-bit vmcnt");
  static_assert(LDSB == GemmLds<BM, BN, ACT, MODE>::bytes, "LDS size of the configuration");

  const int logical = xcd_logical(blockIdx.x, m_tiles * n_tiles);
  if (logical < 0) return;
  int mt, nt;
  tile_of(logical, n_tiles, m_tiles, gm, mt, nt);
  const int4 tile = tiles[mt];
  const int e = tile.x, r0 = tile.y, r1 = tile.z, g0 = tile.w;
  const int n0 = nt * BN;
  // K stages of this tile: fixed, or (kWgrad) the expert's own.
  const int ktiles = MODE == kWgrad ? be.kst[e + 1] - be.kst[e] : K / BK;
  // wave is uniform: readfirstlane lets every per-wave index live in SGPRs.
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / 4, wn = wave % 4;
  const bool a_wave = wave < 4;
  const int grp = wave % 4;

  // Operands are fetched by buffer loads into LDS: a wave-uniform resource
  // (base address in scalar registers), a per-lane byte offset in one VGPR,
  // and wave-uniform offsets per load and per stage, so no per-lane 64-bit
  // pointer stays live across the K loop.  sbase is this wave's stream base
  // and kstep the elements from one K stage to the next (BK along an A row of
  // the up GEMM, which is addressed per pair instead; one ldg-group stage of
  // the packed hidden buffer; one slab stage, SR * BK elements, of the packed
  // weights); soff[i] is load i's byte offset within a stage.
  int ldst;  // LDS byte offset (within a stage) of this wave's first load
  const bf16_t* sbase;
  size_t kstep = 0;
  uint32_t soff[LMAX];
  uint32_t voff;
  // Up GEMM A waves: the lane's row relative to the tile (first load) and the
  // tile's last relative row; rows past it are clamped to it.
  int arel = 0, alast = 0;
  // A rows are spread over the four A waves in interleaved units (16-row
  // groups for the down GEMM, 8-row pieces of a pair for the up GEMM): load i
  // of wave grp fetches unit 4 i + grp.  A copy of the K loop for FA_ live
  // fragments issues only the loads of units below 64 FA_ rows (all a tile of
  // at most 64 FA_ rows holds), so a short tile fetches only its own rows.
  if (a_wave && !AP) {
    ldst = grp * 1024;
    sbase = A + (size_t)g0 * 512;
    kstep = (size_t)ldg * 512;
    voff = lane * 16;
    const int last = (r1 - r0 - 1) / RPL;  // the tile's last 16-row group
#pragma unroll
    for (int i = 0; i < LMAX; ++i)  // past the tile: fetched, never used
      soff[i] = (uint32_t)min(4 * (i < LA ? i : 0) + grp, last) * 1024u;
  } else if (a_wave) {
    // Load i of a pair: tile rows 8 (4 i + grp) + lane / 8, physical 16-byte
    // chunk lane % 8 of the row's 128 bytes, which holds logical chunk
    // (lane % 8) ^ swz8(row % 16); row % 16 = 8 (grp % 2) + lane / 8.
    ldst = 0;
    sbase = A + (size_t)r0 * K;
    arel = grp * 8 + lane / 8;
    alast = r1 - 1 - r0;
    voff = ((lane & 7) ^ swz8(8 * (grp & 1) + (lane >> 3))) * 16;
#pragma unroll
    for (int i = 0; i < LMAX; ++i) soff[i] = 0;
  } else {
    ldst = (AP ? 0 : BM * RB) + grp * LB * 1024;
    const int SR = packed_slab_rows(N);
    kstep = (size_t)SR * BK;
    voff = lane * 16;
    // A wave's LB loads are LB consecutive 16-row groups of one matrix
    // (BROWS / 4 rows; for SwiGLU BN is a multiple of that).
    const int br0 = grp * LB * RPL;
    sbase = ((DUAL && br0 >= BN) ? B2 : B) +
            (MODE == kWgrad ? (size_t)be.kst[e] * BK * N : (size_t)e * N * K);
#pragma unroll
    for (int i = 0; i < LMAX; ++i) {
      const int br = (grp * LB + (i < LB ? i : 0)) * RPL;  // first weight row in the stage
      const int n = min(n0 + (DUAL ? br % BN : br), N - RPL);  // 16-row group, clamped
      soff[i] = (uint32_t)(((size_t)(n / SR) * ktiles * SR * BK + (n % SR) / RPL * 512) * 2);
    }
  }

  // LDS byte offsets (within a stage) of this lane's MFMA fragments; the
  // chunk index of K step kk is (kk * 2 + lane / 32) ^ swizzle(row).
  // (AP: A rows are 128 bytes in their pair slot, weight rows are offsets
  // within their own stage.)
  int xoff[FM], woff[FN], woff2[FN2];
  constexpr int WBASE = AP ? 0 : BM;
#pragma unroll
  for (int i = 0; i < FM; ++i) xoff[i] = ((2 * i + wm) * 32 + (lane & 31)) * (AP ? 2 * RB : RB);
#pragma unroll
  for (int j = 0; j < FN; ++j) {
    woff[j] = (WBASE + wn * WN + j * 32 + (lane & 31)) * RB;
    if constexpr (DUAL) woff2[j] = (WBASE + BN + wn * WN + j * 32 + (lane & 31)) * RB;
  }
  // Fragment rows differ from lane&31 by multiples of 32 (BM is one too), and
  // the swizzles only look at the low four row bits.
  const int sw = swz4(lane & 31);
  const int sw8 = swz8(lane & 15);

  // Live fragments of this wave: the tile has ceil(rows / 32) fragments,
  // numbered so that this wave owns wm, wm + 2, ...
  const int nf = (r1 - r0 + 31) / 32;
  const int fa = min(FM, max(0, (nf - wm + 1) / 2));

  // Two register sets, one K step (16) each: set 0 holds step 0 of a stage,
  // set 1 step 1.  Each set is refilled while the other one feeds the MFMAs.
  bf16x8_t xf0[FM], wf0[FN], vf0[FN2];
  bf16x8_t xf1[FM], wf1[FN], vf1[FN2];

  // Issue the loads of K tile kt_ into ring slot slot_; the A waves issue
  // NA_ loads (units 4 i + grp), the weight waves LB.  The stream's resource
  // is rebased per stage, so the scalar offsets stay within one stage.
#define MOE_RING_ISSUE(kt_, slot_, NA_)                                                    \
  do {                                                                                     \
    char* base_ = smem + (slot_) * STAGE + ldst;                                           \
    const auto rs_ = buffer_rsrc(sbase + (size_t)(kt_) * kstep, 0xFFFFFFFFu);              \
    if (a_wave) {                                                                          \
      _Pragma("unroll") for (int i = 0; i < LA; ++i) if (i < (NA_))                        \
          buffer_load_lds16<0>(rs_, base_ + i * 4096, voff, soff[i]);                      \
    } else { /* weights are read once per launch: non-temporal, system scope */            \
      _Pragma("unroll") for (int i = 0; i < LB; ++i)                                       \
          buffer_load_lds16<kWeightCpol>(rs_, base_ + i * 1024, voff, soff[i]);            \
    }                                                                                      \
  } while (0)
  // AP: weight stage kt_ into its ring slot (weight waves), A pair p_ into
  // pair slot p_ & 1 (A waves).
#define MOE_ISSUE_W(kt_)                                                                   \
  do {                                                                                     \
    char* base_ = smem + 2 * ASLOT + ((kt_) % NW) * WST + ldst;                            \
    const auto rs_ = buffer_rsrc(sbase + (size_t)(kt_) * kstep, 0xFFFFFFFFu);              \
    _Pragma("unroll") for (int i = 0; i < LB; ++i)                                         \
        buffer_load_lds16<kWeightCpol>(rs_, base_ + i * 1024, voff, soff[i]);              \
  } while (0)
  // The A resource spans the tile's rows, every load stays inside it (rows
  // past the tile are clamped to its last row: fetched, never used).  The
  // empty asm makes the row offsets be recomputed at each issue (three VALU
  // operations per load) rather than held in registers across the loop.
#define MOE_ISSUE_A(p_, NA_)                                                               \
  do {                                                                                     \
    char* base_ = smem + ((p_) & 1) * ASLOT + grp * 1024;                                  \
    const auto rs_ = buffer_rsrc(sbase, (uint32_t)(alast + 1) * (uint32_t)K * 2u);         \
    int ar_ = arel;                                                                        \
    asm volatile("" : "+v"(ar_));                                                          \
    _Pragma("unroll") for (int i = 0; i < LA2; ++i) if (i < (NA_)) {                       \
      const uint32_t v_ = (uint32_t)min(ar_ + 32 * i, alast) * (uint32_t)K * 2u + voff;    \
      buffer_load_lds16<0>(rs_, base_ + i * 4096, v_, (uint32_t)(p_) * (2 * BK * 2));      \
    }                                                                                      \
  } while (0)
  // Read the fragments of K step kk_ of stage kt_ into set S (FA_ live row
  // fragments).
#define MOE_LOAD_KK(FA_, kt_, kk_, S)                                                      \
  do {                                                                                     \
    const char* xs_;                                                                       \
    const char* ws_;                                                                       \
    if constexpr (AP) {                                                                    \
      xs_ = smem + (((kt_) >> 1) & 1) * ASLOT +                                            \
            (((((kt_) & 1) * 4 + (kk_) * 2 + (lane >> 5)) ^ sw8) << 4);                    \
      ws_ = smem + 2 * ASLOT + ((kt_) % NW) * WST + ((((kk_) * 2 + (lane >> 5)) ^ sw) << 4); \
    } else {                                                                               \
      xs_ = smem + ((kt_) % NS) * STAGE + ((((kk_) * 2 + (lane >> 5)) ^ sw) << 4);          \
      ws_ = xs_;                                                                           \
    }                                                                                      \
    _Pragma("unroll") for (int i = 0; i < (FA_); ++i)                                      \
        xf##S[i] = *reinterpret_cast<const bf16x8_t*>(xs_ + xoff[i]);                      \
    _Pragma("unroll") for (int j = 0; j < FN; ++j) {                                       \
      wf##S[j] = *reinterpret_cast<const bf16x8_t*>(ws_ + woff[j]);                        \
      if constexpr (DUAL) vf##S[j] = *reinterpret_cast<const bf16x8_t*>(ws_ + woff2[j]);   \
    }                                                                                      \
  } while (0)
#define MOE_MFMA_KK(FA_, S)                                                                \
  do {                                                                                     \
    _Pragma("unroll") for (int i = 0; i < (FA_); ++i)                                      \
    _Pragma("unroll") for (int j = 0; j < FN; ++j) {                                       \
      if constexpr (FUSED)                                                                 \
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xf##S[i], wf##S[j], acc[i][j], \
                                                            0, 0, 0);                      \
      else                                                                                 \
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf##S[j], xf##S[i], acc[i][j], \
                                                            0, 0, 0);                      \
      if constexpr (DUAL)                                                                  \
        acc2[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf##S[j], xf##S[i],           \
                                                             acc2[i][j], 0, 0, 0);         \
    }                                                                                      \
  } while (0)
  // Wait until stage kt_ + 1 has landed in every wave, and let the slot of
  // stage kt_ be refilled: each wave waits for its own loads of stage kt_ + 1
  // (vmcnt counts this wave's 1-KB loads, `later_` younger stages may stay in
  // flight) and for its LDS reads of stage kt_ (lgkmcnt 0), then the barrier
  // makes both true for the whole block.  The slot a stage was read from is
  // thus free right after that stage's barrier: a ring of NS slots keeps
  // NS - 1 stages in flight while one is consumed.
#define MOE_SYNC_STAGE(later_, NA_)                                                        \
  do {                                                                                     \
    if (a_wave) wait_stages<(NA_)>(later_);                                                \
    else wait_stages<LB>(later_);                                                          \
    wait_lgkmcnt0();                                                                       \
    ring_barrier();                                                                        \
  } while (0)
  // Fragments and MFMAs of stage kt_: with two register sets, step 1's reads
  // were issued before step 0's MFMAs (set 0 holds step 0); with one set the
  // steps run one after the other.  MOE_STAGE_HEAD runs before the stage's
  // barrier, MOE_STAGE_TAIL after it (and after the refill): the two-set loop
  // reads step 0 of stage kt_ + 1 there, while set 1 still feeds the MFMAs.
#define MOE_STAGE_HEAD(FA_, kt_)                                                           \
  do {                                                                                     \
    if constexpr (ONESET) {                                                                \
      MOE_LOAD_KK(FA_, kt_, 0, 0);                                                         \
      MOE_MFMA_KK(FA_, 0);                                                                 \
      MOE_LOAD_KK(FA_, kt_, 1, 0);                                                         \
      MOE_MFMA_KK(FA_, 0);                                                                 \
    } else {                                                                               \
      MOE_LOAD_KK(FA_, kt_, 1, 1);                                                         \
      MOE_MFMA_KK(FA_, 0);                                                                 \
    }                                                                                      \
  } while (0)
#define MOE_STAGE_NEXT(FA_, kt_)                                                           \
  do {                                                                                     \
    if constexpr (!ONESET) MOE_LOAD_KK(FA_, (kt_) + 1, 0, 0);                              \
  } while (0)
#define MOE_STAGE_TAIL(FA_)                                                                \
  do {                                                                                     \
    if constexpr (!ONESET) MOE_MFMA_KK(FA_, 1);                                            \
  } while (0)
  // The whole K loop for FA_ live row fragments.  Every copy issues the same
  // loads and barriers; only the LDS reads and MFMAs differ.
#define MOE_K_LOOP(FA_)                                                                    \
  do {                                                                                     \
    _Pragma("unroll") for (int i = 0; i < (FA_); ++i)                                      \
    _Pragma("unroll") for (int j = 0; j < FN; ++j) {                                       \
      acc[i][j] = floatx16{};                                                              \
      if constexpr (DUAL) acc2[i][j] = floatx16{};                                         \
    }                                                                                      \
    int kt = 0;                                                                            \
    if constexpr (AP) {                                                                    \
      /* A pairs 0 and 1, weight stages 0 .. NW-1; stage 0 landed.          */             \
      if (a_wave) {                                                                        \
        MOE_ISSUE_A(0, 2 * (FA_));                                                         \
        if (ktiles > 2) {                                                                  \
          MOE_ISSUE_A(1, 2 * (FA_));                                                       \
          wait_vmcnt<2 * (FA_)>();                                                         \
        } else {                                                                           \
          wait_vmcnt<0>();                                                                 \
        }                                                                                  \
      } else {                                                                             \
        _Pragma("unroll") for (int s = 0; s < NW; ++s) if (s < ktiles) MOE_ISSUE_W(s);     \
        wait_stages<LB>(min(NW - 1, ktiles - 1));                                          \
      }                                                                                    \
      ring_barrier();                                                                      \
      if constexpr (!ONESET) MOE_LOAD_KK(FA_, 0, 0, 0);                                    \
      /* Steady state: the weight refill (stage kt + NW, into the slot of    */            \
      /* stage kt) and the next A pair are in range.  For the A waves the    */            \
      /* wait at stage kt is for a new pair when kt is odd (issued two       */            \
      /* stages ago, the only A loads in flight), after which pair (kt+3)/2 */             \
      /* goes into the slot of stages kt-1 and kt.                          */             \
      for (; kt + NW < ktiles; ++kt) {                                                     \
        MOE_STAGE_HEAD(FA_, kt);                                                           \
        if (a_wave) {                                                                      \
          if (kt & 1) wait_vmcnt<0>();                                                     \
        } else {                                                                           \
          wait_vmcnt<(NW - 2) * LB>();                                                     \
        }                                                                                  \
        wait_lgkmcnt0();                                                                   \
        ring_barrier();                                                                    \
        if (a_wave) {                                                                      \
          if (kt & 1) MOE_ISSUE_A((kt + 3) >> 1, 2 * (FA_));                               \
        } else {                                                                           \
          MOE_ISSUE_W(kt + NW);                                                            \
        }                                                                                  \
        MOE_STAGE_NEXT(FA_, kt);                                                           \
        MOE_STAGE_TAIL(FA_);                                                               \
      }                                                                                    \
      for (; kt < ktiles; ++kt) {                                                          \
        MOE_STAGE_HEAD(FA_, kt);                                                           \
        if (kt + 1 < ktiles) {                                                             \
          if (a_wave) {                                                                    \
            if (kt & 1) wait_vmcnt<0>();                                                   \
          } else {                                                                         \
            wait_stages<LB>(ktiles - kt - 2);                                              \
          }                                                                                \
          wait_lgkmcnt0();                                                                 \
          ring_barrier();                                                                  \
          if (a_wave && (kt & 1) && kt + 3 < ktiles) MOE_ISSUE_A((kt + 3) >> 1, 2 * (FA_)); \
          MOE_STAGE_NEXT(FA_, kt);                                                         \
        }                                                                                  \
        MOE_STAGE_TAIL(FA_);                                                               \
      }                                                                                    \
    } else {                                                                               \
      _Pragma("unroll") for (int s = 0; s < NS; ++s) if (s < ktiles) MOE_RING_ISSUE(s, s, FA_); \
      MOE_SYNC_STAGE(min(NS - 1, ktiles - 1), FA_);                                        \
      if constexpr (!ONESET) MOE_LOAD_KK(FA_, 0, 0, 0);                                    \
      /* Steady state: the refill (stage kt + NS, into the slot of stage kt) */            \
      /* is always in range and the wait count is fixed.                    */             \
      for (; kt + NS < ktiles; ++kt) {                                                     \
        MOE_STAGE_HEAD(FA_, kt);                                                           \
        if (a_wave) wait_vmcnt<(NS - 2) * (FA_)>(); else wait_vmcnt<(NS - 2) * LB>();      \
        wait_lgkmcnt0();                                                                   \
        ring_barrier();                                                                    \
        MOE_RING_ISSUE(kt + NS, kt % NS, FA_);                                             \
        MOE_STAGE_NEXT(FA_, kt);                                                           \
        MOE_STAGE_TAIL(FA_);                                                               \
      }                                                                                    \
      /* The last NS stages: nothing left to issue.                         */             \
      for (; kt < ktiles; ++kt) {                                                          \
        MOE_STAGE_HEAD(FA_, kt);                                                           \
        if (kt + 1 < ktiles) {                                                             \
          MOE_SYNC_STAGE(ktiles - kt - 2, FA_);                                            \
          MOE_STAGE_NEXT(FA_, kt);                                                         \
        }                                                                                  \
        MOE_STAGE_TAIL(FA_);                                                               \
      }                                                                                    \
    }                                                                                      \
  } while (0)

  // Epilogue: activation, bf16 pairs, then a half-row swap between lanes l
  // and l+32.  Before it, lane l (row l&31) holds columns 8g + 4(l>>5) + 0..3
  // for g = 0..3; after swapping g = 2p+1 of lane l with g = 2p of lane l+32,
  // lane l holds columns 16p + 0..7 and lane l+32 columns 16p + 8..15.
#define MOE_EPILOGUE(FA_)                                                                  \
  do {                                                                                     \
    _Pragma("unroll") for (int i = 0; i < (FA_); ++i) {                                    \
      const int lr = (2 * i + wm) * 32 + (lane & 31); /* row within the tile */            \
      const int row = r0 + lr;                                                             \
      _Pragma("unroll") for (int j = 0; j < FN; ++j)                                       \
      _Pragma("unroll") for (int p = 0; p < 2; ++p) {                                      \
        float o[8];                                                                        \
        _Pragma("unroll") for (int u = 0; u < 8; ++u) {                                    \
          const int q = 8 * p + u; /* accumulator element: g = 2p + u/4 */                 \
          if constexpr (DUAL) o[u] = silu(acc[i][j][q]) * acc2[i][j][q];                   \
          else o[u] = apply_act(acc[i][j][q], ACT);                                        \
        }                                                                                  \
        const uint32_t lo0 = pack_bf16x2(o[0], o[1]), lo1 = pack_bf16x2(o[2], o[3]);        \
        const uint32_t hi0 = pack_bf16x2(o[4], o[5]), hi1 = pack_bf16x2(o[6], o[7]);        \
        const auto s0 = __builtin_amdgcn_permlane32_swap(lo0, hi0, false, false);          \
        const auto s1 = __builtin_amdgcn_permlane32_swap(lo1, hi1, false, false);          \
        const int col = n0 + wn * WN + j * 32 + 16 * p + 8 * (lane >> 5);                  \
        if (row < r1 && col < N) {                                                         \
          const u32x4 v = {s0[0], s1[0], s0[1], s1[1]};                                    \
          if (MODE == kUpGemm) {                                                           \
            const int r16 = lr % 16, pos = 4 * r16 + (((col % 32) / 8) ^ swz4(r16));        \
            *reinterpret_cast<u32x4*>(C + ((size_t)(col / 32) * ldg + g0 + lr / 16) * 512 + \
                                      pos * 8) = v;                                        \
          } else {                                                                         \
            *reinterpret_cast<u32x4*>(C + (size_t)row * N + col) = v;                      \
          }                                                                                \
        }                                                                                  \
      }                                                                                    \
    }                                                                                      \
  } while (0)
  // Fused combine epilogue (operands swapped): accumulator element q of lane l
  // is output column l & 31 of fragment row 8 (q / 4) + 4 (l >> 5) + q % 4.
  // Per row: its token and routing weight (rows without a token add nothing),
  // then w * bf16(O) into y_acc[token] (y_acc rows are N = d wide).
#define MOE_EPILOGUE_FUSED(FA_)                                                            \
  do {                                                                                     \
    _Pragma("unroll") for (int i = 0; i < (FA_); ++i)                                      \
    _Pragma("unroll") for (int q = 0; q < 16; ++q) {                                       \
      const int row = r0 + (2 * i + wm) * 32 + 8 * (q >> 2) + 4 * (lane >> 5) + (q & 3);    \
      int tok = -1;                                                                        \
      float wt = 0.f;                                                                      \
      if (row < r1) {                                                                      \
        tok = fc.token_of_row[row];                                                        \
        if (tok >= 0) wt = fc.topk_w[(size_t)tok * fc.k + fc.slot_of_row[row]];            \
      }                                                                                    \
      _Pragma("unroll") for (int j = 0; j < FN; ++j) {                                     \
        const int col = n0 + wn * WN + j * 32 + (lane & 31);                               \
        if (tok >= 0 && col < N) {                                                         \
          const float o = bf16_to_f32(pack_bf16x2(acc[i][j][q], 0.f) & 0xffffu);           \
          unsafeAtomicAdd(fc.y_acc + (size_t)tok * N + col, wt * o);                       \
        }                                                                                  \
      }                                                                                    \
    }                                                                                      \
  } while (0)
  // fp32 epilogue (kUpRawF32): lane l holds columns 8g + 4(l>>5) + 0..3 of
  // row l&31 for g = 0..3, stored as they are.
#define MOE_EPILOGUE_RAW(FA_)                                                              \
  do {                                                                                     \
    _Pragma("unroll") for (int i = 0; i < (FA_); ++i) {                                    \
      const int row = r0 + (2 * i + wm) * 32 + (lane & 31);                                \
      _Pragma("unroll") for (int j = 0; j < FN; ++j)                                       \
      _Pragma("unroll") for (int g = 0; g < 4; ++g) {                                      \
        const int col = n0 + wn * WN + j * 32 + 8 * g + 4 * (lane >> 5);                   \
        if (row < r1 && col < N) {                                                         \
          const size_t o_ = (size_t)row * N + col;                                         \
          *reinterpret_cast<floatx4*>(be.U + o_) =                                         \
              floatx4{acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2],        \
                      acc[i][j][4 * g + 3]};                                               \
          if constexpr (DUAL)                                                              \
            *reinterpret_cast<floatx4*>(be.V + o_) =                                       \
                floatx4{acc2[i][j][4 * g], acc2[i][j][4 * g + 1], acc2[i][j][4 * g + 2],   \
                        acc2[i][j][4 * g + 3]};                                            \
        }                                                                                  \
      }                                                                                    \
    }                                                                                      \
  } while (0)
  // Activation-gradient epilogue (kBwdG), four consecutive columns at a time;
  // the packed store of 4 elements is half of a 16-byte position: row r16 of
  // the tile's group, logical chunk (col % 32) / 8, elements col % 8 on.
  // Units (i, j) of four column groups run as a two-stage pipeline: the u (v)
  // loads of the next unit are issued before this unit's arithmetic and
  // stores.  The vector memory counter retires loads and stores in issue
  // order, and a wait after a branch must assume the fewest operations in
  // flight of any path into it, so the epilogue has no branches: u, v, H and
  // G go through buffer resources based at the tile's first row (rows past
  // the tile fall outside the range), the packed G through one based at the
  // tile's first group of the column block, and a lane outside the tile or
  // the matrix takes an offset past every range, which the hardware answers
  // with zeros (loads) or drops (stores).  Each wait then leaves the previous
  // unit's stores and the next unit's loads in flight.
#define MOE_BWDG_LOAD(n_, b_)                                                              \
  do {                                                                                     \
    const int i_ = (n_) / FN, j_ = (n_) % FN;                                              \
    const int lr_ = (2 * i_ + wm) * 32 + (lane & 31);                                      \
    const int cb_ = n0 + wn * WN + j_ * 32;                                                \
    const bool ok_ = lr_ < rows_t && cb_ < N;                                              \
    _Pragma("unroll") for (int g = 0; g < 4; ++g) {                                        \
      const int col_ = cb_ + 8 * g + 4 * (lane >> 5);                                      \
      const uint32_t o_ = ok_ ? (uint32_t)(lr_ * N + col_) * 4u : kBwdOut;                 \
      ub_[b_][g] = __builtin_bit_cast(floatx4, __builtin_amdgcn_raw_buffer_load_b128(rs_u, o_, 0, 0)); \
      if constexpr (ACT == ACT_SWIGLU)                                                     \
        vb_[b_][g] = __builtin_bit_cast(floatx4, __builtin_amdgcn_raw_buffer_load_b128(rs_v, o_, 0, 0)); \
    }                                                                                      \
  } while (0)
#define MOE_EPILOGUE_BWDG(FA_)                                                             \
  do {                                                                                     \
    constexpr int NU_ = (FA_) * FN;                                                        \
    constexpr uint32_t kBwdOut = 0x80000000u;                                              \
    const int rows_t = r1 - r0;                                                            \
    const auto rs_u = buffer_rsrc(be.U + (size_t)r0 * N, (uint32_t)rows_t * (uint32_t)N * 4u); \
    const auto rs_v = buffer_rsrc((ACT == ACT_SWIGLU ? be.V : be.U) + (size_t)r0 * N,        \
                                  (uint32_t)rows_t * (uint32_t)N * 4u);                    \
    const auto rs_h = buffer_rsrc(be.H + (size_t)r0 * N, (uint32_t)rows_t * (uint32_t)N * 2u); \
    const auto rs_g = buffer_rsrc(be.G + (size_t)r0 * be.kg,                               \
                                  (uint32_t)rows_t * (uint32_t)be.kg * 2u);                \
    floatx4 ub_[2][4], vb_[2][4];                                                          \
    if constexpr (NU_ > 0) MOE_BWDG_LOAD(0, 0);                                            \
    _Pragma("unroll") for (int n = 0; n < NU_; ++n) {                                      \
      if (n + 1 < NU_) MOE_BWDG_LOAD(n + 1, (n + 1) & 1);                                  \
      const int i = n / FN, j = n % FN;                                                    \
      const int lr = (2 * i + wm) * 32 + (lane & 31);                                      \
      const int r16 = lr % 16;                                                             \
      const int cb = n0 + wn * WN + j * 32;                                                \
      const bool ok = lr < rows_t && cb < N;                                               \
      /* packed G: column block cb (du) and N + cb (dv), from the tile's first group */    \
      const auto rs_c = buffer_rsrc(C + ((size_t)(cb / 32) * ldg + g0) * 512, 0x7fffffffu); \
      const int cb2 = ACT == ACT_SWIGLU ? N + cb : cb; /* dv's column block (SwiGLU) */     \
      const auto rs_c2 = buffer_rsrc(C + ((size_t)(cb2 / 32) * ldg + g0) * 512, 0x7fffffffu); \
      _Pragma("unroll") for (int g = 0; g < 4; ++g) {                                      \
        const int col = cb + 8 * g + 4 * (lane >> 5);                                      \
        const floatx4 uu = ub_[n & 1][g];                                                  \
        floatx4 vv = floatx4{0.f, 0.f, 0.f, 0.f};                                          \
        if constexpr (ACT == ACT_SWIGLU) vv = vb_[n & 1][g];                               \
        float hv[4], gu[4], gv[4];                                                         \
        _Pragma("unroll") for (int q = 0; q < 4; ++q)                                      \
          bwd_act_grad<ACT>(uu[q], vv[q], acc[i][j][4 * g + q], hv[q], gu[q], gv[q]);      \
        const u32x2 hb = {pack_bf16x2(hv[0], hv[1]), pack_bf16x2(hv[2], hv[3])};           \
        const u32x2 ubv = {pack_bf16x2(gu[0], gu[1]), pack_bf16x2(gu[2], gu[3])};          \
        const int pos = 4 * r16 + (((col % 32) / 8) ^ swz4(r16));                          \
        const uint32_t oh = ok ? (uint32_t)(lr * N + col) * 2u : kBwdOut;                  \
        const uint32_t og = ok ? (uint32_t)(lr * be.kg + col) * 2u : kBwdOut;              \
        const uint32_t oc = ok ? (uint32_t)((lr / 16) * 512 + pos * 8 + col % 8) * 2u : kBwdOut; \
        __builtin_amdgcn_raw_buffer_store_b64(hb, rs_h, oh, 0, 0);                         \
        __builtin_amdgcn_raw_buffer_store_b64(ubv, rs_g, og, 0, 0);                        \
        __builtin_amdgcn_raw_buffer_store_b64(ubv, rs_c, oc, 0, 0);                        \
        if constexpr (ACT == ACT_SWIGLU) {                                                 \
          const u32x2 vbv = {pack_bf16x2(gv[0], gv[1]), pack_bf16x2(gv[2], gv[3])};        \
          const uint32_t og2 = ok ? (uint32_t)(lr * be.kg + N + col) * 2u : kBwdOut;       \
          __builtin_amdgcn_raw_buffer_store_b64(vbv, rs_g, og2, 0, 0);                     \
          __builtin_amdgcn_raw_buffer_store_b64(vbv, rs_c2, oc, 0, 0);                     \
        }                                                                                  \
      }                                                                                    \
    }                                                                                      \
  } while (0)
  // Weight-gradient epilogue (kWgrad): fp32, rows split between the outputs.
#define MOE_EPILOGUE_WG(FA_)                                                               \
  do {                                                                                     \
    _Pragma("unroll") for (int i = 0; i < (FA_); ++i) {                                    \
      const int m = r0 + (2 * i + wm) * 32 + (lane & 31);                                  \
      float* orow_ = m < be.kg ? be.U + ((size_t)e * be.kg + m) * N                        \
                               : be.V + ((size_t)e * (be.M - be.kg) + (m - be.kg)) * N;     \
      _Pragma("unroll") for (int j = 0; j < FN; ++j)                                       \
      _Pragma("unroll") for (int g = 0; g < 4; ++g) {                                      \
        const int col = n0 + wn * WN + j * 32 + 8 * g + 4 * (lane >> 5);                   \
        if (m < r1 && col < N)                                                             \
          *reinterpret_cast<floatx4*>(orow_ + col) =                                       \
              floatx4{acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2],        \
                      acc[i][j][4 * g + 3]};                                               \
      }                                                                                    \
    }                                                                                      \
  } while (0)
  // One self-contained copy (accumulators, K loop, epilogue) per number of
  // live fragments, so no accumulator value crosses from one copy to another.
#define MOE_TILE(FA_)                                                                      \
  do {                                                                                     \
    floatx16 acc[(FA_) > 0 ? (FA_) : 1][FN];                                               \
    floatx16 acc2[DUAL && (FA_) > 0 ? (FA_) : 1][FN2];                                     \
    MOE_K_LOOP(FA_);                                                                       \
    if constexpr (FUSED) MOE_EPILOGUE_FUSED(FA_);                                          \
    else if constexpr (MODE == kUpRawF32) MOE_EPILOGUE_RAW(FA_);                           \
    else if constexpr (MODE == kBwdG) MOE_EPILOGUE_BWDG(FA_);                              \
    else if constexpr (MODE == kWgrad) MOE_EPILOGUE_WG(FA_);                               \
    else MOE_EPILOGUE(FA_);                                                                \
  } while (0)

  static_assert(FM >= 2 && FM <= 5, "one copy per live-fragment count 0..FM");
  switch (fa) {
    case 0: MOE_TILE(0); break;
    case 1: MOE_TILE(1); break;
    case 2: if constexpr (FM >= 2) MOE_TILE(2); break;
    case 3: if constexpr (FM >= 3) MOE_TILE(3); break;
    case 4: if constexpr (FM >= 4) MOE_TILE(4); break;
    default: if constexpr (FM >= 5) MOE_TILE(5); break;
  }
#undef MOE_TILE
#undef MOE_EPILOGUE
#undef MOE_EPILOGUE_FUSED
#undef MOE_EPILOGUE_RAW
#undef MOE_EPILOGUE_BWDG
#undef MOE_BWDG_LOAD
#undef MOE_EPILOGUE_WG
#undef MOE_K_LOOP
#undef MOE_LOAD_KK
#undef MOE_MFMA_KK
#undef MOE_SYNC_STAGE
#undef MOE_STAGE_HEAD
#undef MOE_STAGE_NEXT
#undef MOE_STAGE_TAIL
#undef MOE_RING_ISSUE
#undef MOE_ISSUE_W
#undef MOE_ISSUE_A
}

template <int BM, int BN, int ACT, int MODE>
__global__ __launch_bounds__(kGemmWaves * 64, 1) __attribute__((amdgpu_waves_per_eu(2, 2)))
void grouped_gemm_bf16(
    const bf16_t* __restrict__ A, const bf16_t* __restrict__ B, const bf16_t* __restrict__ B2,
    bf16_t* __restrict__ C, int K, int N, const int4* __restrict__ tiles,
    const int32_t* __restrict__ tile_count, int n_tiles, int ldg, int gm, FusedCombineArgs fc,
    BwdEpiArgs be) {
  __shared__ __attribute__((aligned(1024))) char smem[GemmLds<BM, BN, ACT, MODE>::bytes];
  gemm_bf16_body<BM, BN, ACT, MODE>(smem, A, B, B2, C, K, N, tiles, tile_count[0], n_tiles, ldg,
                                    gm > 0 ? gm : tile_count[1], fc, be);
}

// Two tile configurations in one kernel: the tile plan has chosen the row
// tile height from the batch's row counts (tile_count[2]), so the block runs
// BM1 x BN1 tiles (n_tiles1 column tiles) when it is BM1, else BM2 x BN2.
// The LDS array is the larger ring; registers are those of the larger body.
template <int BM1, int BN1, int BM2, int BN2, int ACT, int MODE>
__global__ __launch_bounds__(kGemmWaves * 64, 1) __attribute__((amdgpu_waves_per_eu(2, 2)))
void grouped_gemm_bf16_pick(
    const bf16_t* __restrict__ A, const bf16_t* __restrict__ B, const bf16_t* __restrict__ B2,
    bf16_t* __restrict__ C, int K, int N, const int4* __restrict__ tiles,
    const int32_t* __restrict__ tile_count, int n_tiles1, int n_tiles2, int ldg,
    FusedCombineArgs fc) {
  constexpr int L1 = GemmLds<BM1, BN1, ACT, MODE>::bytes, L2 = GemmLds<BM2, BN2, ACT, MODE>::bytes;
  __shared__ __attribute__((aligned(1024))) char smem[L1 > L2 ? L1 : L2];
  // The plan's tile count, group size and row tile height in one load (the
  // plan sits at the 256-aligned start of the workspace).
  const int4 plan = *reinterpret_cast<const int4*>(tile_count);
  if (plan.z == BM1)
    gemm_bf16_body<BM1, BN1, ACT, MODE>(smem, A, B, B2, C, K, N, tiles, plan.x, n_tiles1, ldg,
                                        plan.y, fc, BwdEpiArgs{});
  else
    gemm_bf16_body<BM2, BN2, ACT, MODE>(smem, A, B, B2, C, K, N, tiles, plan.x, n_tiles2, ldg,
                                        plan.y, fc, BwdEpiArgs{});
}

// Weight packing for the bf16 kernel: W [E, N, K] row-major -> slabs of SR
// rows (SR = packed_slab_rows(N)); slab (e, s) holds K/32 stages of SR*32
// elements, each stage SR/16 blocks of 1 KB laid out exactly as
// grouped_gemm_bf16 stages 16 weight rows in LDS: 16-byte position L of block
// g holds row 16g + L/4 of the slab, logical chunk (L % 4) ^ swz4(L / 4).  One
// thread per 16-byte output chunk, so the writes are contiguous.
__global__ __launch_bounds__(256) void pack_weights_bf16(const bf16_t* __restrict__ w,
                                                         bf16_t* __restrict__ wp, int N, int K,
                                                         size_t chunks) {
  const int SR = packed_slab_rows(N), kts = K / 32;
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t q = (size_t)blockIdx.x * blockDim.x + threadIdx.x; q < chunks; q += stride) {
    const int L = (int)(q % 64);
    const size_t blk = q / 64;                 // 1-KB block index
    const int g = (int)(blk % (SR / 16));      // 16-row group in the slab stage
    const size_t st = blk / (SR / 16);         // slab stage: (e * N/SR + s) * kts + kt
    const int kt = (int)(st % kts);
    const size_t es = st / kts;                // e * (N / SR) + s: slabs are contiguous rows
    const int r = L / 4, c = (L % 4) ^ swz4(r);
    const size_t row = es * SR + g * 16 + r;
    *reinterpret_cast<u32x4*>(wp + q * 8) =
        *reinterpret_cast<const u32x4*>(w + row * K + kt * 32 + c * 8);
  }
}

hipError_t launch_pack_weights(int E, int N, int K, const void* w, void* wp, hipStream_t st) {
  const size_t chunks = (size_t)E * N * K / 8;
  const int blocks = (int)std::min<size_t>((chunks + 255) / 256, 8192);
  pack_weights_bf16<<<blocks, 256, 0, st>>>(static_cast<const bf16_t*>(w),
                                            static_cast<bf16_t*>(wp), N, K, chunks);
  return hipGetLastError();
}

// The same packed layout for a matrix given transposed: the [N, K] matrix
// whose columns k < KA are rows k of wa[e] ([E, KA, N] row-major) and whose
// columns k >= KA are rows k - KA of wb[e] ([E, K - KA, N]).  The backward
// takes W2^T (N = h, K = d, from W2 [E, d, h]) and [W1^T | W3^T] (N = d,
// K = h or 2h, from W1, W3 [E, h, d]) this way.  One thread per 16-byte
// output chunk, eight gathered elements each (a one-time repacking).
__global__ __launch_bounds__(256) void pack_weights_t_bf16(const bf16_t* __restrict__ wa,
                                                           const bf16_t* __restrict__ wb,
                                                           bf16_t* __restrict__ wp, int N, int KA,
                                                           int K, size_t chunks) {
  const int SR = packed_slab_rows(N), kts = K / 32, KB = K - KA;
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t q = (size_t)blockIdx.x * blockDim.x + threadIdx.x; q < chunks; q += stride) {
    const int L = (int)(q % 64);
    const size_t blk = q / 64;
    const int g = (int)(blk % (SR / 16));
    const size_t st = blk / (SR / 16);
    const int kt = (int)(st % kts);
    const size_t es = st / kts;
    const int r = L / 4, c = (L % 4) ^ swz4(r);
    const size_t row = es * SR + g * 16 + r;
    const size_t e = row / N;
    const int n = (int)(row % N), k0 = kt * 32 + c * 8;
    uint32_t v[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      uint32_t lh[2];
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        const int k = k0 + 2 * t + b;
        lh[b] = k < KA ? wa[(e * KA + k) * N + n] : wb[(e * KB + (k - KA)) * N + n];
      }
      v[t] = lh[0] | (lh[1] << 16);
    }
    *reinterpret_cast<u32x4*>(wp + q * 8) = u32x4{v[0], v[1], v[2], v[3]};
  }
}

hipError_t launch_pack_weights_t(int E, int N, int KA, int K, const void* wa, const void* wb,
                                 void* wp, hipStream_t st) {
  const size_t chunks = (size_t)E * N * K / 8;
  const int blocks = (int)std::min<size_t>((chunks + 255) / 256, 8192);
  pack_weights_t_bf16<<<blocks, 256, 0, st>>>(static_cast<const bf16_t*>(wa),
                                              static_cast<const bf16_t*>(wb),
                                              static_cast<bf16_t*>(wp), N, KA, K, chunks);
  return hipGetLastError();
}

// ------------------------------------------------------------- fp32 MFMA ---

// FUSEDC: the down GEMM with the combine folded in (as kDownFused above): each
// output element, scaled by its row's routing weight, is added into the
// token's fp32 accumulator row instead of being stored.
template <int ACT, bool FUSEDC>
__global__ __launch_bounds__(256) void grouped_gemm_f32(
    const float* __restrict__ A, const float* __restrict__ B, const float* __restrict__ B2,
    float* __restrict__ C, int K, int N, const int4* __restrict__ tiles,
    const int32_t* __restrict__ tile_count, int n_tiles, FusedCombineArgs fc) {
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
        if constexpr (FUSEDC) {
          if (row < r1 && col < N) {
            const int tok = fc.token_of_row[row];
            if (tok >= 0)
              unsafeAtomicAdd(fc.y_acc + (size_t)tok * N + col,
                              fc.topk_w[(size_t)tok * fc.k + fc.slot_of_row[row]] * o);
          }
        } else {
          if (row < r1 && col < N) C[(size_t)row * N + col] = o;
        }
      }
    }
}

// ---------------------------------------------------------------- launch ---

constexpr int kF32BM = 64, kF32BN = 64;

static size_t align256(size_t x) { return (x + 255) / 256 * 256; }

// Row-tile height.  bf16: 320 rows, which take a whole expert at capacity
// factor 1.25 of 256 rows.  128 rows when experts average at most 32 rows
// (decode-sized batches): such tiles hold two live fragments per wave instead
// of five, which leaves the accumulators for twice the columns (half the
// column tiles, so half the prologues and epilogues) and drops the requests
// for rows past a 320-row tile.  Only where one tile per expert is all but
// certain: an expert of more rows than a tile is split, and each of its row
// tiles streams the expert's weights again (DeepSeek-like layer, 128 rows per
// expert on average but spread around that: 5.75 -> 6.63 ms per step with
// 128-row tiles; decode, ~8 rows per expert: 3.77 -> 3.64 ms).
// 192 rows when experts average at most 128 rows: an expert of up to 192 rows
// (all but a few at 128 on average) still takes one tile, and the smaller A
// slots leave LDS and registers for 512 weight rows per stage where the
// matrices are wide enough (SwiGLU with h >= 2048, the down GEMM with
// d >= 4096), which halves the A rows' L2 reads against 256.
// 192 rows also when experts average at least kLargeRowsPerExpert rows: every
// expert then spans many row tiles anyway, its last partial tile wastes less
// of a 192-row tile than of a 320-row one (2048 rows: 97% of the tile rows
// live against 91%), and the wide 96 x 128 wave tile reads fewer LDS bytes
// per MFMA (3 + 4 fragments for 12 MFMAs against 5 + 2 for 10).  Same-box
// A/B on the Mixtral-like layer (2048 rows per expert): up GEMM 3607 ->
// 3427 us, down unchanged (1724 us), step 5.50 -> 5.34 ms.  Only with at least
// kLargeMinRows rows in all: fewer give too few blocks to fill the chip (one
// expert of 4096 rows, the DeepSeek-like shared expert: 176 up blocks for 256
// CUs, 420 against 372 us alone, and the layer's step ~30 us slower).
constexpr int kLargeRowsPerExpert = 1024, kLargeMinRows = 8192;
static int ffn_bm(int dtype, int E, int max_rows) {
  if (dtype == 0) return kF32BM;
  if ((long long)max_rows <= 32LL * E) return kGemmBMSmall;
  if ((long long)max_rows <= (long long)kMidRowsPerExpert * E) return kGemmBMMid;
  if ((long long)max_rows >= (long long)kLargeRowsPerExpert * E && max_rows >= kLargeMinRows)
    return kGemmBMMid;
  return kGemmBM;
}

// Where the bound max_rows asks for 320-row tiles but is within 4x of the
// 192-row threshold, the batch may still hold few enough rows for 192-row
// tiles (a capacity-bound layer whose hot experts drop most of their slots):
// the forward's tile plan then picks the height from the real counts
// (ffn_plan_tiles, BMalt) and the GEMMs serve both (grouped_gemm_bf16_pick).
// Skewed-load layer (15.6 k of 65.5 k slots admitted, 640-row cap): FFN 709 ->
// 567 us.  Far above it (Mixtral-like: 2048 rows per expert) the two-height
// kernel cost 1.3% against the 320-row one and the choice is not offered.
// 0 when there is no choice.
static int ffn_bm_alt(int dtype, int E, int max_rows) {
  return dtype == 1 && ffn_bm(dtype, E, max_rows) == kGemmBM &&
                 (long long)max_rows <= 4LL * kMidRowsPerExpert * E
             ? kGemmBMMid
             : 0;
}
// The smallest row tile a plan may use (it sizes the plan and the groups).
static int ffn_bm_min(int dtype, int E, int max_rows) {
  const int alt = ffn_bm_alt(dtype, E, max_rows);
  return alt ? alt : ffn_bm(dtype, E, max_rows);
}

// Upper bound of row tiles: every expert may end in a partial tile.
static int max_m_tiles(int max_rows, int BM, int E) { return (max_rows + BM - 1) / BM + E; }

static size_t ffn_plan_bytes(int E, int max_rows, int dtype) {
  return align256(sizeof(int32_t)) +
         align256((size_t)max_m_tiles(max_rows, ffn_bm_min(dtype, E, max_rows), E) *
                  sizeof(int4));
}

// 16-row groups of the packed bf16 hidden buffer: each tile rounds its rows up
// to whole groups, so at most one partial group per tile.
static int ffn_groups(int E, int max_rows) {
  return (max_rows + 15) / 16 + max_m_tiles(max_rows, ffn_bm_min(1, E, max_rows), E);
}

size_t ffn_workspace_bytes(int E, int max_rows, int d, int h, int act, int dtype) {
  (void)d;
  (void)act;
  const size_t hidden = dtype == 0 ? (size_t)max_rows * h * 4
                                   : (size_t)ffn_groups(E, max_rows) * 16 * h * 2;
  return ffn_plan_bytes(E, max_rows, dtype) + align256(hidden);
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
  const int bm = ffn_bm(a.dtype, a.E, a.max_rows);
  ffn_plan_tiles<<<1, 1024, 0, st>>>(a.offsets, nullptr, a.E, bm,
                                     ffn_bm_alt(a.dtype, a.E, a.max_rows), a.max_rows,
                                     max_m_tiles(a.max_rows, ffn_bm_min(a.dtype, a.E, a.max_rows),
                                                 a.E),
                                     ffn_groups(a.E, a.max_rows), ffn_tiles(a), ffn_count(a));
  return hipGetLastError();
}

template <int BM, int BN, int ACT, int MODE>
static void launch_bf16(const bf16_t* A, const bf16_t* B, const bf16_t* B2, bf16_t* C, int K,
                        int N, const FfnArgs& a, hipStream_t st, BwdEpiArgs be = {}) {
  const int nt = (N + BN - 1) / BN;
  const int g = grid_of(max_m_tiles(a.max_rows, BM, a.E), nt);
  // Block order from the plan (gm 0): groups of 4 row tiles once a quarter of
  // the row tiles belong to experts of two or more; an XCD's 32 concurrent
  // blocks then cover 4 x 8 tiles, so an expert's row tiles read its weight
  // slabs from that XCD's L2, and its L2 misses per K stage fall from 1 A tile
  // + 32 weight slabs to 4 A tiles + 8 weight slabs.
  grouped_gemm_bf16<BM, BN, ACT, MODE><<<g, kGemmWaves * 64, 0, st>>>(
      A, B, B2, C, K, N, ffn_tiles(a), ffn_count(a), nt, ffn_groups(a.E, a.max_rows), 0,
      MODE == kDownFused ? *a.fused : FusedCombineArgs{}, be);
}

// The forward GEMMs where the plan picks the row tile height (ffn_bm_alt):
// BM1 x BN1 (192-row tiles) or BM2 x BN2 (320-row tiles).
template <int BM1, int BN1, int BM2, int BN2, int ACT, int MODE>
static void launch_bf16_pick(const bf16_t* A, const bf16_t* B, const bf16_t* B2, bf16_t* C,
                             int K, int N, const FfnArgs& a, hipStream_t st) {
  const int nt1 = (N + BN1 - 1) / BN1, nt2 = (N + BN2 - 1) / BN2;
  const int g = std::max(grid_of(max_m_tiles(a.max_rows, BM1, a.E), nt1),
                         grid_of(max_m_tiles(a.max_rows, BM2, a.E), nt2));
  grouped_gemm_bf16_pick<BM1, BN1, BM2, BN2, ACT, MODE><<<g, kGemmWaves * 64, 0, st>>>(
      A, B, B2, C, K, N, ffn_tiles(a), ffn_count(a), nt1, nt2, ffn_groups(a.E, a.max_rows),
      MODE == kDownFused ? *a.fused : FusedCombineArgs{});
}

template <int ACT, bool FUSEDC = false>
static void launch_f32(const float* A, const float* B, const float* B2, float* C, int K, int N,
                       const FfnArgs& a, hipStream_t st) {
  const int nt = (N + kF32BN - 1) / kF32BN;
  const int g = grid_of(max_m_tiles(a.max_rows, kF32BM, a.E), nt);
  grouped_gemm_f32<ACT, FUSEDC><<<g, 256, 0, st>>>(A, B, B2, C, K, N, ffn_tiles(a), ffn_count(a),
                                                   nt, FUSEDC ? *a.fused : FusedCombineArgs{});
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
    const int bm = ffn_bm(1, a.E, a.max_rows);
    if (bm == kGemmBMMid) {
      constexpr int S = kGemmBMMid;
      if (a.act == ACT_SWIGLU) {
        if (a.h >= 2048) launch_bf16<S, 256, ACT_SWIGLU, kUpGemm>(X, W1, W3, H, a.d, a.h, a, st);
        else launch_bf16<S, 128, ACT_SWIGLU, kUpGemm>(X, W1, W3, H, a.d, a.h, a, st);
      } else if (a.h >= 2048) {
        if (a.act == ACT_RELU) launch_bf16<S, 256, ACT_RELU, kUpGemm>(X, W1, nullptr, H, a.d, a.h, a, st);
        else launch_bf16<S, 256, ACT_GELU, kUpGemm>(X, W1, nullptr, H, a.d, a.h, a, st);
      } else {
        if (a.act == ACT_RELU) launch_bf16<S, 128, ACT_RELU, kUpGemm>(X, W1, nullptr, H, a.d, a.h, a, st);
        else launch_bf16<S, 128, ACT_GELU, kUpGemm>(X, W1, nullptr, H, a.d, a.h, a, st);
      }
    } else if (bm == kGemmBMSmall) {
      // 128-row tiles: twice the columns per tile for the same accumulators.
      constexpr int S = kGemmBMSmall;
      if (a.act == ACT_SWIGLU) {
        if (a.h >= 1024) launch_bf16<S, 256, ACT_SWIGLU, kUpGemm>(X, W1, W3, H, a.d, a.h, a, st);
        else launch_bf16<S, 128, ACT_SWIGLU, kUpGemm>(X, W1, W3, H, a.d, a.h, a, st);
      } else if (a.h >= 2048) {
        if (a.act == ACT_RELU) launch_bf16<S, 512, ACT_RELU, kUpGemm>(X, W1, nullptr, H, a.d, a.h, a, st);
        else launch_bf16<S, 512, ACT_GELU, kUpGemm>(X, W1, nullptr, H, a.d, a.h, a, st);
      } else {
        if (a.act == ACT_RELU) launch_bf16<S, 256, ACT_RELU, kUpGemm>(X, W1, nullptr, H, a.d, a.h, a, st);
        else launch_bf16<S, 256, ACT_GELU, kUpGemm>(X, W1, nullptr, H, a.d, a.h, a, st);
      }
    } else if (ffn_bm_alt(1, a.E, a.max_rows) == 0) {
      if (a.act == ACT_SWIGLU) {
        launch_bf16<kGemmBM, 128, ACT_SWIGLU, kUpGemm>(X, W1, W3, H, a.d, a.h, a, st);
      } else if (a.h >= 2048) {
        if (a.act == ACT_RELU) launch_bf16<kGemmBM, 256, ACT_RELU, kUpGemm>(X, W1, nullptr, H, a.d, a.h, a, st);
        else launch_bf16<kGemmBM, 256, ACT_GELU, kUpGemm>(X, W1, nullptr, H, a.d, a.h, a, st);
      } else {
        if (a.act == ACT_RELU) launch_bf16<kGemmBM, 128, ACT_RELU, kUpGemm>(X, W1, nullptr, H, a.d, a.h, a, st);
        else launch_bf16<kGemmBM, 128, ACT_GELU, kUpGemm>(X, W1, nullptr, H, a.d, a.h, a, st);
      }
    } else if (a.act == ACT_SWIGLU) {
      // 320-row tiles, or the 192-row ones the mid branch above would take.
      constexpr int M = kGemmBMMid, L = kGemmBM;
      if (a.h >= 2048) launch_bf16_pick<M, 256, L, 128, ACT_SWIGLU, kUpGemm>(X, W1, W3, H, a.d, a.h, a, st);
      else launch_bf16_pick<M, 128, L, 128, ACT_SWIGLU, kUpGemm>(X, W1, W3, H, a.d, a.h, a, st);
    } else if (a.h >= 2048) {
      constexpr int M = kGemmBMMid, L = kGemmBM;
      if (a.act == ACT_RELU) launch_bf16_pick<M, 256, L, 256, ACT_RELU, kUpGemm>(X, W1, nullptr, H, a.d, a.h, a, st);
      else launch_bf16_pick<M, 256, L, 256, ACT_GELU, kUpGemm>(X, W1, nullptr, H, a.d, a.h, a, st);
    } else {
      constexpr int M = kGemmBMMid, L = kGemmBM;
      if (a.act == ACT_RELU) launch_bf16_pick<M, 128, L, 128, ACT_RELU, kUpGemm>(X, W1, nullptr, H, a.d, a.h, a, st);
      else launch_bf16_pick<M, 128, L, 128, ACT_GELU, kUpGemm>(X, W1, nullptr, H, a.d, a.h, a, st);
    }
  }
  return hipGetLastError();
}

// Zero fill of the fused combine's fp32 accumulator (a kernel, not a memset,
// so a captured graph replays it as a kernel node).
__global__ __launch_bounds__(256) void zero_f32x4(floatx4* __restrict__ p, size_t n4) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += stride)
    p[i] = floatx4{0.f, 0.f, 0.f, 0.f};
}

template <int MODE>
static void launch_down_bf16(const FfnArgs& a, hipStream_t st) {
  auto H = static_cast<const bf16_t*>(ffn_hidden_buf(a));
  auto W2 = static_cast<const bf16_t*>(a.w2);
  auto Y = static_cast<bf16_t*>(a.y_rows);
  const int bm = ffn_bm(1, a.E, a.max_rows);
  if (bm == kGemmBMMid) {
    if (a.d >= 4096) launch_bf16<kGemmBMMid, 512, ACT_NONE, MODE>(H, W2, nullptr, Y, a.h, a.d, a, st);
    else if (a.d >= 1024) launch_bf16<kGemmBMMid, 256, ACT_NONE, MODE>(H, W2, nullptr, Y, a.h, a.d, a, st);
    else launch_bf16<kGemmBMMid, 128, ACT_NONE, MODE>(H, W2, nullptr, Y, a.h, a.d, a, st);
  } else if (bm == kGemmBMSmall) {
    constexpr int S = kGemmBMSmall;
    if (a.d >= 2048) launch_bf16<S, 512, ACT_NONE, MODE>(H, W2, nullptr, Y, a.h, a.d, a, st);
    else launch_bf16<S, 256, ACT_NONE, MODE>(H, W2, nullptr, Y, a.h, a.d, a, st);
  } else if (ffn_bm_alt(1, a.E, a.max_rows) == 0) {
    if (a.d >= 1024) launch_bf16<kGemmBM, 256, ACT_NONE, MODE>(H, W2, nullptr, Y, a.h, a.d, a, st);
    else launch_bf16<kGemmBM, 128, ACT_NONE, MODE>(H, W2, nullptr, Y, a.h, a.d, a, st);
  } else {
    // 320-row tiles, or the 192-row ones the mid branch above would take.
    constexpr int M = kGemmBMMid, L = kGemmBM;
    if (a.d >= 4096) launch_bf16_pick<M, 512, L, 256, ACT_NONE, MODE>(H, W2, nullptr, Y, a.h, a.d, a, st);
    else if (a.d >= 1024) launch_bf16_pick<M, 256, L, 256, ACT_NONE, MODE>(H, W2, nullptr, Y, a.h, a.d, a, st);
    else launch_bf16_pick<M, 128, L, 128, ACT_NONE, MODE>(H, W2, nullptr, Y, a.h, a.d, a, st);
  }
}

hipError_t launch_ffn_zero_acc(const FfnArgs& a, hipStream_t st) {
  const size_t n4 = (size_t)a.fused->N * a.d / 4;  // d is a multiple of 64
  if (n4 > 0) {
    const int blocks = (int)std::min<size_t>((n4 + 255) / 256, 4096);
    zero_f32x4<<<blocks, 256, 0, st>>>(reinterpret_cast<floatx4*>(a.fused->y_acc), n4);
  }
  return hipGetLastError();
}

hipError_t launch_ffn_down(const FfnArgs& a, hipStream_t st) {
  if (a.fused) {
    const hipError_t e = launch_ffn_zero_acc(a, st);
    if (e != hipSuccess) return e;
  }
  if (a.dtype == 0) {
    auto H = static_cast<const float*>(ffn_hidden_buf(a));
    auto W2 = static_cast<const float*>(a.w2);
    auto Y = static_cast<float*>(a.y_rows);
    if (a.fused) launch_f32<ACT_NONE, true>(H, W2, nullptr, Y, a.h, a.d, a, st);
    else launch_f32<ACT_NONE, false>(H, W2, nullptr, Y, a.h, a.d, a, st);
  } else if (a.fused) {
    launch_down_bf16<kDownFused>(a, st);
  } else {
    launch_down_bf16<kDownGemm>(a, st);
  }
  return hipGetLastError();
}

// ------------------------------------------------------- backward GEMMs ---

// Workspace of the backward on the grouped GEMM: the tile plan (as the
// forward's), G = [du | dv] in the packed layout (K = kg = h or 2h), u (and v)
// in fp32, then G and H row-major for the weight gradients.
namespace {
struct BwdLayout {
  size_t gpk, u, v, grm, hrm, total;
};
BwdLayout bwd_layout(int E, int max_rows, int h, int act) {
  const size_t kg = act == ACT_SWIGLU ? 2 * (size_t)h : (size_t)h;
  BwdLayout l;
  l.gpk = ffn_plan_bytes(E, max_rows, 1);
  l.u = l.gpk + align256((size_t)ffn_groups(E, max_rows) * 16 * kg * 2);
  l.v = l.u + align256((size_t)max_rows * h * 4);
  l.grm = l.v + (act == ACT_SWIGLU ? align256((size_t)max_rows * h * 4) : 0);
  l.hrm = l.grm + align256((size_t)max_rows * kg * 2);
  l.total = l.hrm + align256((size_t)max_rows * h * 2);
  return l;
}
}  // namespace

size_t ffn_bwd_gemms_workspace_bytes(int E, int max_rows, int d, int h, int act) {
  (void)d;
  return bwd_layout(E, max_rows, h, act).total;
}

size_t ffn_bwd_packed_workspace_bytes(int E, int max_rows, int d, int h, int act) {
  return ffn_bwd_gemms_workspace_bytes(E, max_rows, d, h, act) +
         ffn_bwd_wgrad_workspace_bytes(E, max_rows, d, h, act);
}

hipError_t launch_zero_f32(float* p, size_t n, hipStream_t st) {
  const size_t n4 = n / 4;  // n is a multiple of 64 here
  if (n4 > 0) {
    const int blocks = (int)std::min<size_t>((n4 + 255) / 256, 4096);
    zero_f32x4<<<blocks, 256, 0, st>>>(reinterpret_cast<floatx4*>(p), n4);
  }
  return hipGetLastError();
}

hipError_t launch_ffn_bwd_packed_gemms(const FfnBwdPackedArgs& a, void** g_rm, void** h_rm,
                                       hipStream_t st) {
  const BwdLayout l = bwd_layout(a.E, a.max_rows, a.h, a.act);
  char* ws = static_cast<char*>(a.ws);
  const bool dual = a.act == ACT_SWIGLU;
  const int kg = dual ? 2 * a.h : a.h;
  BwdEpiArgs be{reinterpret_cast<float*>(ws + l.u), dual ? reinterpret_cast<float*>(ws + l.v) : nullptr,
                reinterpret_cast<bf16_t*>(ws + l.grm), reinterpret_cast<bf16_t*>(ws + l.hrm), kg};
  *g_rm = be.G;
  *h_rm = be.H;
  if (a.max_rows == 0) return hipGetLastError();
  FfnArgs f{a.E, a.max_rows, a.d, a.h, a.act, 1, a.x_rows, a.offsets, a.w1p, a.w3p, nullptr,
            nullptr, a.ws};
  const int bm = ffn_bm(1, a.E, a.max_rows);
  ffn_plan_tiles<<<1, 1024, 0, st>>>(a.offsets, a.group_rows, a.E, bm, 0, a.max_rows,
                                     max_m_tiles(a.max_rows, bm, a.E), ffn_groups(a.E, a.max_rows),
                                     ffn_tiles(f), ffn_count(f));
  auto X = static_cast<const bf16_t*>(a.x_rows);
  auto DY = static_cast<const bf16_t*>(a.dy_rows);
  auto W1 = static_cast<const bf16_t*>(a.w1p);
  auto W3 = static_cast<const bf16_t*>(a.w3p);
  auto W2T = static_cast<const bf16_t*>(a.w2tp);
  auto W13T = static_cast<const bf16_t*>(a.w13tp);
  auto GP = reinterpret_cast<bf16_t*>(ws + l.gpk);
  auto DX = static_cast<bf16_t*>(a.dx_rows);
  // u (v): the forward's up GEMM shape; g: an up GEMM of dy with W2^T, one
  // B operand; dx: the forward's down GEMM shape over G (K = kg).
  const bool wide = a.h >= 2048;
#define MOE_BWD_TILES(S_)                                                                  \
  do {                                                                                     \
    constexpr int S = (S_);                                                                \
    if (dual) {                                                                            \
      if constexpr (S != kGemmBM) {                                                        \
        if (wide)                                                                          \
          launch_bf16<S, 256, ACT_SWIGLU, kUpRawF32>(X, W1, W3, nullptr, a.d, a.h, f, st, be); \
        else                                                                               \
          launch_bf16<S, 128, ACT_SWIGLU, kUpRawF32>(X, W1, W3, nullptr, a.d, a.h, f, st, be); \
      } else {                                                                             \
        launch_bf16<S, 128, ACT_SWIGLU, kUpRawF32>(X, W1, W3, nullptr, a.d, a.h, f, st, be); \
      }                                                                                    \
    } else if (wide) {                                                                     \
      launch_bf16<S, 256, ACT_NONE, kUpRawF32>(X, W1, nullptr, nullptr, a.d, a.h, f, st, be); \
    } else {                                                                               \
      launch_bf16<S, 128, ACT_NONE, kUpRawF32>(X, W1, nullptr, nullptr, a.d, a.h, f, st, be); \
    }                                                                                      \
    switch (a.act) {                                                                       \
      case ACT_RELU:                                                                       \
        if (wide) launch_bf16<S, 256, ACT_RELU, kBwdG>(DY, W2T, nullptr, GP, a.d, a.h, f, st, be); \
        else launch_bf16<S, 128, ACT_RELU, kBwdG>(DY, W2T, nullptr, GP, a.d, a.h, f, st, be); \
        break;                                                                             \
      case ACT_GELU:                                                                       \
        if (wide) launch_bf16<S, 256, ACT_GELU, kBwdG>(DY, W2T, nullptr, GP, a.d, a.h, f, st, be); \
        else launch_bf16<S, 128, ACT_GELU, kBwdG>(DY, W2T, nullptr, GP, a.d, a.h, f, st, be); \
        break;                                                                             \
      default:                                                                             \
        if (wide) launch_bf16<S, 256, ACT_SWIGLU, kBwdG>(DY, W2T, nullptr, GP, a.d, a.h, f, st, be); \
        else launch_bf16<S, 128, ACT_SWIGLU, kBwdG>(DY, W2T, nullptr, GP, a.d, a.h, f, st, be); \
        break;                                                                             \
    }                                                                                      \
    if constexpr (S == kGemmBMMid) {                                                       \
      if (a.d >= 4096) {                                                                   \
        launch_bf16<S, 512, ACT_NONE, kDownGemm>(GP, W13T, nullptr, DX, kg, a.d, f, st);   \
        break;                                                                             \
      }                                                                                    \
    }                                                                                      \
    if (a.d >= 1024)                                                                       \
      launch_bf16<S, 256, ACT_NONE, kDownGemm>(GP, W13T, nullptr, DX, kg, a.d, f, st);     \
    else                                                                                   \
      launch_bf16<S, 128, ACT_NONE, kDownGemm>(GP, W13T, nullptr, DX, kg, a.d, f, st);     \
  } while (0)
  if (bm == kGemmBMMid) MOE_BWD_TILES(kGemmBMMid);
  else if (bm == kGemmBMSmall) MOE_BWD_TILES(kGemmBMSmall);
  else MOE_BWD_TILES(kGemmBM);
#undef MOE_BWD_TILES
  return hipGetLastError();
}

// ------------------------------------------------- weight gradients ---

// Segments as the backward clamps them (to max_rows and, when given, to the
// first group_rows[e] rows), their stage offsets kst[e] (sum of ceil(rows /
// 32) before e; kst[E] = the total), and the tiles of the two weight-gradient
// GEMMs: BM rows of M1 (= kg) or M2 (= d) for every expert, {e, m0, m1,
// kst[e] M / 16 + m0 / 16}.
__global__ __launch_bounds__(1024) void wgrad_plan(const int32_t* __restrict__ offsets,
                                                   const int32_t* __restrict__ group_rows, int E,
                                                   int max_rows, int BM, int M1, int M2,
                                                   int2* __restrict__ seg, int32_t* __restrict__ kst,
                                                   int4* __restrict__ tiles1,
                                                   int4* __restrict__ tiles2,
                                                   int32_t* __restrict__ counts) {
  __shared__ int32_t wsum[16];
  const int e = threadIdx.x;
  int lo = 0, hi = 0;
  if (e < E) {
    lo = min(offsets[e], max_rows);
    hi = min(offsets[e + 1], max_rows);
    if (group_rows) hi = min(hi, lo + max(group_rows[e], 0));
    hi = max(hi, lo);
  }
  const int n = (hi - lo + 31) / 32;
  const int incl = block_scan_1024(n, wsum);
  if (e < E) {
    seg[e] = make_int2(lo, hi);
    kst[e] = incl - n;
    if (e == E - 1) kst[E] = incl;
    const int mt1 = (M1 + BM - 1) / BM, mt2 = (M2 + BM - 1) / BM;
    for (int i = 0; i < mt1; ++i)
      tiles1[e * mt1 + i] = make_int4(e, i * BM, min(M1, (i + 1) * BM),
                                      (incl - n) * (M1 / 16) + i * BM / 16);
    for (int i = 0; i < mt2; ++i)
      tiles2[e * mt2 + i] = make_int4(e, i * BM, min(M2, (i + 1) * BM),
                                      (incl - n) * (M2 / 16) + i * BM / 16);
    if (e == 0) {
      counts[0] = E * mt1;
      counts[1] = E * mt2;
    }
  }
}

// Row-major activations src [rows, C] (bf16) of every expert's segment, in
// stages of 32 rows (zero past the segment), transposed into 1-KB blocks of
// 16 columns x 32 rows laid out as the GEMM stages them (16-byte position L:
// column 16q + L/4, logical chunk (L % 4) ^ swz4(L/4) of the 32 rows): the
// packed-A order (block (kst[e] + t) C/16 + q) or, with layoutB, the weights'
// slab order (slab s = q / (SR/16) of the expert at s kt_e SR/16 blocks, then
// stage t, then the block in the slab).  One block of 256 threads per stage
// and 256 columns, through an LDS tile.
__global__ __launch_bounds__(256) void pack_rows_t_bf16(const bf16_t* __restrict__ src, int C,
                                                        const int2* __restrict__ seg,
                                                        const int32_t* __restrict__ kst, int E,
                                                        int layoutB, bf16_t* __restrict__ out) {
  __shared__ __attribute__((aligned(16))) bf16_t tile[32][256 + 8];
  const int sg = blockIdx.x;
  if (sg >= kst[E]) return;
  int lo = 0, hi = E - 1;  // the expert e with kst[e] <= sg < kst[e + 1]
  while (lo < hi) {
    const int mid = (lo + hi + 1) / 2;
    if (kst[mid] <= sg) lo = mid; else hi = mid - 1;
  }
  const int e = lo, t = sg - kst[e], kte = kst[e + 1] - kst[e];
  const int2 sgm = seg[e];
  const int r0 = sgm.x + 32 * t;
  const int c0 = blockIdx.y * 256;
  const int tid = threadIdx.x;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int id = tid + 256 * u, row = id / 32, cc = id % 32, col = c0 + cc * 8;
    u32x4 v = {0u, 0u, 0u, 0u};
    if (r0 + row < sgm.y && col < C) v = *reinterpret_cast<const u32x4*>(src + (size_t)(r0 + row) * C + col);
    *reinterpret_cast<u32x4*>(&tile[row][cc * 8]) = v;
  }
  __syncthreads();
  const int SR = packed_slab_rows(C), bps = SR / 16;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int id = tid + 256 * u, ql = id / 64, L = id % 64;
    const int cl = 16 * ql + L / 4;
    if (c0 + 16 * ql >= C) continue;
    const int k0 = 8 * ((L % 4) ^ swz4(L / 4));
    uint32_t w4[4];
#pragma unroll
    for (int q2 = 0; q2 < 4; ++q2)
      w4[q2] = (uint32_t)tile[k0 + 2 * q2][cl] | ((uint32_t)tile[k0 + 2 * q2 + 1][cl] << 16);
    const int q = (c0 >> 4) + ql;
    const size_t blk = layoutB ? (size_t)kst[e] * (C / 16) + (size_t)(q / bps) * kte * bps +
                                     (size_t)t * bps + (q % bps)
                               : ((size_t)kst[e] + t) * (C / 16) + q;
    *reinterpret_cast<u32x4*>(out + blk * 512 + L * 8) = u32x4{w4[0], w4[1], w4[2], w4[3]};
  }
}

namespace {
constexpr int kWgBM = 128;
struct WgLayout {
  size_t seg, kst, counts, tiles1, tiles2, gt, xt, dyt, ht, total;
};
WgLayout wg_layout(size_t base, int E, int max_rows, int d, int h, int act) {
  const int kg = act == ACT_SWIGLU ? 2 * h : h;
  const size_t stages = (size_t)(max_rows + 31) / 32 + E;
  WgLayout l;
  l.seg = base;
  l.kst = l.seg + align256((size_t)E * sizeof(int2));
  l.counts = l.kst + align256((size_t)(E + 1) * sizeof(int32_t));
  l.tiles1 = l.counts + align256(2 * sizeof(int32_t));
  l.tiles2 = l.tiles1 + align256((size_t)E * ((kg + kWgBM - 1) / kWgBM) * sizeof(int4));
  l.gt = l.tiles2 + align256((size_t)E * ((d + kWgBM - 1) / kWgBM) * sizeof(int4));
  l.xt = l.gt + align256(stages * 32 * kg * 2);
  l.dyt = l.xt + align256(stages * 32 * d * 2);
  l.ht = l.dyt + align256(stages * 32 * d * 2);
  l.total = l.ht + align256(stages * 32 * h * 2);
  return l;
}

template <int BN>
void launch_wgrad_gemm(const bf16_t* A, const bf16_t* B, int N, const int4* tiles,
                       const int32_t* count, int m_tiles_max, int ldg, BwdEpiArgs be,
                       hipStream_t st) {
  const int nt = (N + BN - 1) / BN;
  grouped_gemm_bf16<kWgBM, BN, ACT_NONE, kWgrad><<<grid_of(m_tiles_max, nt), kGemmWaves * 64, 0,
                                                   st>>>(A, B, nullptr, nullptr, 0, N, tiles,
                                                         count, nt, ldg, 1, FusedCombineArgs{}, be);
}
}  // namespace

size_t ffn_bwd_wgrad_workspace_bytes(int E, int max_rows, int d, int h, int act) {
  return wg_layout(0, E, max_rows, d, h, act).total;
}

hipError_t launch_ffn_bwd_wgrad(const FfnBwdPackedArgs& a, const void* g_rm, const void* h_rm,
                                void* ws, float* dw1, float* dw3, float* dw2, hipStream_t st) {
  const int kg = a.act == ACT_SWIGLU ? 2 * a.h : a.h;
  const WgLayout l = wg_layout(0, a.E, a.max_rows, a.d, a.h, a.act);
  char* w = static_cast<char*>(ws);
  int2* seg = reinterpret_cast<int2*>(w + l.seg);
  int32_t* kst = reinterpret_cast<int32_t*>(w + l.kst);
  int32_t* counts = reinterpret_cast<int32_t*>(w + l.counts);
  int4* tiles1 = reinterpret_cast<int4*>(w + l.tiles1);
  int4* tiles2 = reinterpret_cast<int4*>(w + l.tiles2);
  bf16_t* GT = reinterpret_cast<bf16_t*>(w + l.gt);
  bf16_t* XT = reinterpret_cast<bf16_t*>(w + l.xt);
  bf16_t* DYT = reinterpret_cast<bf16_t*>(w + l.dyt);
  bf16_t* HT = reinterpret_cast<bf16_t*>(w + l.ht);
  wgrad_plan<<<1, 1024, 0, st>>>(a.offsets, a.group_rows, a.E, a.max_rows, kWgBM, kg, a.d, seg,
                                 kst, tiles1, tiles2, counts);
  if (a.max_rows > 0) {
    const int stages = (a.max_rows + 31) / 32 + a.E;
    auto pack = [&](const void* src, int C, int layoutB, bf16_t* out) {
      pack_rows_t_bf16<<<dim3(stages, (C + 255) / 256), 256, 0, st>>>(
          static_cast<const bf16_t*>(src), C, seg, kst, a.E, layoutB, out);
    };
    pack(g_rm, kg, 0, GT);
    pack(a.x_rows, a.d, 1, XT);
    pack(a.dy_rows, a.d, 0, DYT);
    pack(h_rm, a.h, 1, HT);
  }
  const int mt1 = (kg + kWgBM - 1) / kWgBM, mt2 = (a.d + kWgBM - 1) / kWgBM;
  // dW1 | dW3 [kg, d] = G^T x; dW2 [d, h] = dy^T H.
  BwdEpiArgs b1{dw1, dw3, nullptr, nullptr, a.h, kg, kst};
  BwdEpiArgs b2{dw2, nullptr, nullptr, nullptr, a.d, a.d, kst};
  if (a.d >= 1024)
    launch_wgrad_gemm<512>(GT, XT, a.d, tiles1, counts, a.E * mt1, kg / 16, b1, st);
  else
    launch_wgrad_gemm<256>(GT, XT, a.d, tiles1, counts, a.E * mt1, kg / 16, b1, st);
  if (a.h >= 1024)
    launch_wgrad_gemm<512>(DYT, HT, a.h, tiles2, counts + 1, a.E * mt2, a.d / 16, b2, st);
  else
    launch_wgrad_gemm<256>(DYT, HT, a.h, tiles2, counts + 1, a.E * mt2, a.d / 16, b2, st);
  return hipGetLastError();
}

}  // namespace moe
