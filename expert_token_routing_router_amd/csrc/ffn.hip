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
__device__ __forceinline__ float gelu_as7126(float u) {
  const float a = fabsf(u);
  const float t = __builtin_amdgcn_rcpf(fmaf(0.3275911f * 0.70710678118654752440f, a, 1.0f));
  float q = fmaf(0.5f * 1.061405429f, t, 0.5f * -1.453152027f);
  q = fmaf(q, t, 0.5f * 1.421413741f);
  q = fmaf(q, t, 0.5f * -0.284496736f);
  q = fmaf(q, t, 0.5f * 0.254829592f);
  const float e = __builtin_amdgcn_exp2f(u * u * -0.72134752044448170368f);
  return fmaf(-(a * t), q * e, fmaxf(u, 0.f));
}

__device__ __forceinline__ float apply_act(float u, int act) {
  if (act == ACT_RELU) return fmaxf(u, 0.f);
  if (act == ACT_GELU) return gelu_as7126(u);
  return u;
}

// g sigmoid(g); v_rcp_f32 (within 2 ulp) in place of an IEEE divide.
__device__ __forceinline__ float silu(float g) { return g * __builtin_amdgcn_rcpf(1.f + __expf(-g)); }

// ------------------------------------------------------------- tile plan ---

// One block of 1024 threads (E <= 1024): expert e owns n_e = ceil(rows_e / BM)
// row tiles of equal height, rounded up to whole 32-row MFMA fragments
// (chunk_e = 32 ceil(ceil(rows_e / n_e) / 32) <= BM; since (n_e - 1) BM <
// rows_e, no tile is empty).  Tile q of the batch is tiles[q] = {e, first
// row, row end, first 16-row group}, and *count = number of tiles.  The group
// numbering gives every tile ceil(rows / 16) groups of its own, in tile order:
// the packed hidden buffer of the bf16 FFN stores a tile's rows there.  Rows
// are clamped to max_rows.
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

__global__ __launch_bounds__(1024) void ffn_plan_tiles(const int32_t* __restrict__ offsets,
                                                       int E, int BM, int max_rows,
                                                       int4* __restrict__ tiles,
                                                       int32_t* __restrict__ count) {
  __shared__ int32_t wsum[16];
  __shared__ int32_t total_s;
  const int e = threadIdx.x;
  int32_t lo = 0, hi = 0, n = 0, chunk = BM;
  if (e < E) {
    lo = min(offsets[e], max_rows);
    hi = min(offsets[e + 1], max_rows);
    n = hi > lo ? (hi - lo + BM - 1) / BM : 0;
    if (n > 0) chunk = ((hi - lo + n - 1) / n + 31) / 32 * 32;
  }
  const int32_t n_incl = block_scan_1024(n, wsum);
  const int32_t start = n_incl - n;
  if (e == E - 1) total_s = n_incl;
  // 16-row groups of this expert's tiles, then their exclusive prefix.
  int32_t ng = 0;
  for (int q = 0; q < n; ++q) ng += (min(hi, lo + (q + 1) * chunk) - (lo + q * chunk) + 15) / 16;
  int32_t g0 = block_scan_1024(ng, wsum) - ng;
  for (int q = 0; q < n; ++q) {
    const int32_t r0 = lo + q * chunk, r1 = min(hi, r0 + chunk);
    tiles[start + q] = make_int4(e, r0, r1, g0);
    g0 += (r1 - r0 + 15) / 16;
  }
  if (e == 0) *count = total_s;  // written by thread E-1 before the second scan's barriers
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
// tiles (160 accumulators) leave room for two waves per SIMD.
//
// MFMA v_mfma_f32_32x32x16_bf16 with the weight fragment as the first operand,
// so a lane's accumulator holds 4 consecutive output columns of one row.
// DUAL (SwiGLU): the B stage holds BN rows of W1 (gate) and BN rows of W3
// (up); the wave keeps both accumulators and combines them in the epilogue.
//
// Operands reach LDS by global_load_lds_dwordx4 (16 bytes per lane, 1 KB =
// 16 rows of 64 bytes per instruction) into a ring of NS stages; waves 0-3
// fetch the A rows (XOR swizzle applied through the choice of source address),
// waves 4-7 the weight rows.  Weights come packed (moe_expert_ffn_pack_weights)
// so that one stage of a slab of 64 or 256 weight rows is one contiguous run
// already in LDS order: the weight stream reads long sequential runs of HBM.
// The epilogue converts to bf16 in registers (v_cvt_pk_bf16_f32), swaps
// half-rows between lanes l and l+32 (v_permlane32_swap) so each lane owns 8
// consecutive columns, and stores 16 bytes per lane straight to global memory.
constexpr int kGemmBM = 320, kGemmBMSmall = 128, kGemmWaves = 8;
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
// so a down tile's K stage is one contiguous run.
enum { kUpGemm = 0, kDownGemm = 1 };

template <int BM, int BN, int ACT, int MODE>
__global__ __launch_bounds__(kGemmWaves * 64, 1) __attribute__((amdgpu_waves_per_eu(2, 2)))
void grouped_gemm_bf16(
    const bf16_t* __restrict__ A, const bf16_t* __restrict__ B, const bf16_t* __restrict__ B2,
    bf16_t* __restrict__ C, int K, int N, const int4* __restrict__ tiles,
    const int32_t* __restrict__ tile_count, int n_tiles, int ldg, int gm) {
  constexpr bool DUAL = ACT == ACT_SWIGLU;
  constexpr int BK = 32, RB = BK * 2;  // RB: bytes per staged row
  constexpr int CH = BK / 8;                         // 16-byte chunks per row
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
  constexpr bool AP = MODE == kUpGemm;
  constexpr int ASLOT = BM * 2 * RB;                   // bytes of one A pair slot
  constexpr int WST = BROWS * RB;                      // bytes of one weight stage
  constexpr int NW_ = (kLdsBytes - 2 * ASLOT) / WST;
  constexpr int NW = AP ? (NW_ < 6 ? NW_ : 6) : NS;    // weight ring depth
  constexpr int LA2 = BM / 8 / 4;                      // A loads per pair, A waves (0-3)
  constexpr int LDSB = AP ? 2 * ASLOT + NW * WST : NS * STAGE;
  static_assert(!AP || (NW >= 4 && NW - 2 <= 4 && (NW - 1) * LB < 64 && 2 * LA2 < 64),
                "pair ring: A pairs two stages ahead, weight waits covered below");
  static_assert(NS >= 3, "the ring needs three stages");
  static_assert(KK == 2, "register sets alternate per K step");
  static_assert(BM % (4 * RPL) == 0 && BROWS % (4 * RPL) == 0, "loads split over 4 waves");
  static_assert(WN % 32 == 0, "wave tile must be whole 32-column MFMA blocks");
  static_assert((NS - 1) * LMAX < 64, "loads in flight must fit the 6-bit vmcnt");
  __shared__ __attribute__((aligned(1024))) char smem[LDSB];

  const int m_tiles = *tile_count;
  const int logical = xcd_logical(blockIdx.x, m_tiles * n_tiles);
  if (logical < 0) return;
  int mt, nt;
  tile_of(logical, n_tiles, m_tiles, gm, mt, nt);
  const int4 tile = tiles[mt];
  const int e = tile.x, r0 = tile.y, r1 = tile.z, g0 = tile.w;
  const int n0 = nt * BN;
  // wave is uniform: readfirstlane lets every per-wave index live in SGPRs.
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / 4, wn = wave % 4;
  const bool a_wave = wave < 4;
  const int grp = wave % 4;

  // Per-lane source pointers of this wave's loads (16 stage rows each) and the
  // element step from one K stage to the next: BK along an A row, one slab
  // stage (SR * BK elements) in the packed weights.
  const bf16_t* src[LMAX];
  int ldst;  // LDS byte offset (within a stage) of this wave's first load
  size_t kstep;
  int arow = 0, ach0 = 0, ach1 = 0;  // AP A waves: first row, logical chunk offsets
  if (a_wave && MODE == kDownGemm) {
    ldst = grp * LA * 1024;
    kstep = (size_t)ldg * 512;
    const int last = (r1 - r0 - 1) / RPL;  // the tile's last 16-row group
#pragma unroll
    for (int i = 0; i < LMAX; ++i) {
      const int g = min(grp * LA + (i < LA ? i : 0), last);  // groups past the tile: fetched, never used
      src[i] = A + (size_t)(g0 + g) * 512 + lane * 8;
    }
  } else if (a_wave) {
    // Load i of a pair: tile rows (grp * LA2 + i) * 8 + lane / 8, physical
    // 16-byte chunk lane % 8 of the row's 128 bytes, which holds logical chunk
    // (lane % 8) ^ swz8(row % 16); row % 16 = 8 (i % 2) + lane / 8.
    ldst = 0;
    kstep = 0;
    arow = r0 + grp * LA2 * 8 + lane / 8;
    ach0 = ((lane & 7) ^ swz8(lane >> 3)) * 8;
    ach1 = ((lane & 7) ^ swz8(8 + (lane >> 3))) * 8;
  } else {
    ldst = (AP ? 0 : BM * RB) + grp * LB * 1024;
    const int SR = packed_slab_rows(N);
    kstep = (size_t)SR * BK;
#pragma unroll
    for (int i = 0; i < LMAX; ++i) {
      const int br = (grp * LB + (i < LB ? i : 0)) * RPL;  // first weight row in the stage
      const bf16_t* W = (DUAL && br >= BN) ? B2 : B;
      const int n = min(n0 + (DUAL ? br % BN : br), N - RPL);  // 16-row group, clamped
      src[i] = W + ((size_t)e * (N / SR) + n / SR) * (size_t)(K / BK) * SR * BK +
               (n % SR) / RPL * 512 + lane * 8;
    }
  }
  const int nl = a_wave ? LA : LB;

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
  const int ktiles = K / BK;

  // Issue the global->LDS loads of K tile kt_ into ring slot slot_.
#define MOE_RING_ISSUE(kt_, slot_)                                                         \
  do {                                                                                     \
    char* base_ = smem + (slot_) * STAGE + ldst;                                           \
    if (a_wave) {                                                                          \
      _Pragma("unroll") for (int i = 0; i < LMAX; ++i) if (LA == LB || i < nl)             \
          __builtin_amdgcn_global_load_lds((void*)(src[i] + (size_t)(kt_) * kstep),        \
                                           (lds_ptr_t)(base_ + i * 1024), 16, 0, 0);       \
    } else { /* weights are read once per launch: non-temporal, system scope */            \
      _Pragma("unroll") for (int i = 0; i < LMAX; ++i) if (LA == LB || i < nl)             \
          __builtin_amdgcn_global_load_lds((void*)(src[i] + (size_t)(kt_) * kstep),        \
                                           (lds_ptr_t)(base_ + i * 1024), 16, 0, kWeightCpol); \
    }                                                                                      \
  } while (0)
  // AP: weight stage kt_ into its ring slot (weight waves), A pair p_ into
  // pair slot p_ & 1 (A waves).
#define MOE_ISSUE_W(kt_)                                                                   \
  do {                                                                                     \
    char* base_ = smem + 2 * ASLOT + ((kt_) % NW) * WST + ldst;                            \
    _Pragma("unroll") for (int i = 0; i < LB; ++i)                                         \
        __builtin_amdgcn_global_load_lds((void*)(src[i] + (size_t)(kt_) * kstep),          \
                                         (lds_ptr_t)(base_ + i * 1024), 16, 0, kWeightCpol); \
  } while (0)
#define MOE_ISSUE_A(p_)                                                                    \
  do {                                                                                     \
    char* base_ = smem + ((p_) & 1) * ASLOT + grp * LA2 * 1024;                            \
    _Pragma("unroll") for (int i = 0; i < LA2; ++i) {                                      \
      const int row_ = min(arow + 8 * i, r1 - 1); /* rows past the tile: never used */     \
      __builtin_amdgcn_global_load_lds(                                                    \
          (void*)(A + (size_t)row_ * K + ((i & 1) ? ach1 : ach0) + (size_t)(p_) * 2 * BK), \
          (lds_ptr_t)(base_ + i * 1024), 16, 0, 0);                                        \
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
      acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf##S[j], xf##S[i], acc[i][j],   \
                                                          0, 0, 0);                        \
      if constexpr (DUAL)                                                                  \
        acc2[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf##S[j], xf##S[i],           \
                                                             acc2[i][j], 0, 0, 0);         \
    }                                                                                      \
  } while (0)
  // Wait until the next stage's loads have landed in every wave: at most
  // `later_` younger stages of this wave may still be in flight (vmcnt counts
  // this wave's 1-KB loads, nl per stage).
#define MOE_WAIT_STAGE(later_)                                                             \
  do {                                                                                     \
    if (a_wave) {                                                                          \
      switch (later_) {                                                                    \
        case 0: wait_vmcnt<0>(); break;                                                    \
        case 1: wait_vmcnt<LA>(); break;                                                   \
        case 2: wait_vmcnt<2 * LA>(); break;                                               \
        default: wait_vmcnt<3 * LA>(); break;                                              \
      }                                                                                    \
    } else {                                                                               \
      switch (later_) {                                                                    \
        case 0: wait_vmcnt<0>(); break;                                                    \
        case 1: wait_vmcnt<LB>(); break;                                                   \
        case 2: wait_vmcnt<2 * LB>(); break;                                               \
        default: wait_vmcnt<3 * LB>(); break;                                              \
      }                                                                                    \
    }                                                                                      \
    ring_barrier();                                                                        \
  } while (0)
  // AP weight waits: at most later_ younger weight stages of this wave in flight.
#define MOE_WAIT_W(later_)                                                                 \
  do {                                                                                     \
    switch (later_) {                                                                      \
      case 0: wait_vmcnt<0>(); break;                                                      \
      case 1: wait_vmcnt<LB>(); break;                                                     \
      case 2: wait_vmcnt<2 * LB>(); break;                                                 \
      case 3: wait_vmcnt<3 * LB>(); break;                                                 \
      default: wait_vmcnt<4 * LB>(); break;                                                \
    }                                                                                      \
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
      /* A pairs 0 and 1, weight stages 0 .. NW-2; stage 0 landed.          */            \
      if (a_wave) {                                                                        \
        MOE_ISSUE_A(0);                                                                    \
        if (ktiles > 2) {                                                                  \
          MOE_ISSUE_A(1);                                                                  \
          wait_vmcnt<LA2>();                                                               \
        } else {                                                                           \
          wait_vmcnt<0>();                                                                 \
        }                                                                                  \
      } else {                                                                             \
        _Pragma("unroll") for (int s = 0; s < NW - 1; ++s) if (s < ktiles) MOE_ISSUE_W(s); \
        MOE_WAIT_W(min(NW - 2, ktiles - 1));                                               \
      }                                                                                    \
      ring_barrier();                                                                      \
      MOE_LOAD_KK(FA_, 0, 0, 0);                                                           \
      /* Steady state: the weight refill and the next A pair are in range.  */            \
      /* The wait at stage kt is for stage kt+1: for the A waves a new pair  */            \
      /* when kt is odd (issued two stages ago, the only A loads in flight), */            \
      /* after which pair (kt+3)/2 goes into the slot of stages kt-1 and kt. */            \
      for (; kt + NW - 1 < ktiles; ++kt) {                                                 \
        MOE_LOAD_KK(FA_, kt, 1, 1);                                                        \
        MOE_MFMA_KK(FA_, 0);                                                               \
        if (a_wave) {                                                                      \
          if (kt & 1) wait_vmcnt<0>();                                                     \
        } else {                                                                           \
          wait_vmcnt<(NW - 3) * LB>();                                                     \
        }                                                                                  \
        ring_barrier();                                                                    \
        if (a_wave) {                                                                      \
          if (kt & 1) MOE_ISSUE_A((kt + 3) >> 1);                                          \
        } else {                                                                           \
          MOE_ISSUE_W(kt + NW - 1);                                                        \
        }                                                                                  \
        MOE_LOAD_KK(FA_, kt + 1, 0, 0);                                                    \
        MOE_MFMA_KK(FA_, 1);                                                               \
      }                                                                                    \
      for (; kt < ktiles; ++kt) {                                                          \
        MOE_LOAD_KK(FA_, kt, 1, 1);                                                        \
        MOE_MFMA_KK(FA_, 0);                                                               \
        if (kt + 1 < ktiles) {                                                             \
          if (a_wave) {                                                                    \
            if (kt & 1) wait_vmcnt<0>();                                                   \
          } else {                                                                         \
            MOE_WAIT_W(min(NW - 3, ktiles - kt - 2));                                      \
          }                                                                                \
          ring_barrier();                                                                  \
          if (a_wave) {                                                                    \
            if ((kt & 1) && kt + 3 < ktiles) MOE_ISSUE_A((kt + 3) >> 1);                   \
          } else if (kt + NW - 1 < ktiles) {                                               \
            MOE_ISSUE_W(kt + NW - 1);                                                      \
          }                                                                                \
          MOE_LOAD_KK(FA_, kt + 1, 0, 0);                                                  \
        }                                                                                  \
        MOE_MFMA_KK(FA_, 1);                                                               \
      }                                                                                    \
    } else {                                                                               \
      _Pragma("unroll") for (int s = 0; s < NS - 1; ++s) if (s < ktiles) MOE_RING_ISSUE(s, s); \
      MOE_WAIT_STAGE(min(NS - 2, ktiles - 1));                                             \
      MOE_LOAD_KK(FA_, 0, 0, 0);                                                           \
      /* Steady state: the refill is always in range and the wait count is  */            \
      /* fixed, so the loop body has no branches besides the wave role.     */            \
      for (; kt + NS - 1 < ktiles; ++kt) {                                                 \
        MOE_LOAD_KK(FA_, kt, 1, 1);                                                        \
        MOE_MFMA_KK(FA_, 0);                                                               \
        if (a_wave) wait_vmcnt<(NS - 3) * LA>(); else wait_vmcnt<(NS - 3) * LB>();         \
        ring_barrier();                                                                    \
        MOE_RING_ISSUE(kt + NS - 1, (kt + NS - 1) % NS);                                   \
        MOE_LOAD_KK(FA_, kt + 1, 0, 0);                                                    \
        MOE_MFMA_KK(FA_, 1);                                                               \
      }                                                                                    \
      /* The last NS - 1 stages: nothing left to issue.                     */            \
      for (; kt < ktiles; ++kt) {                                                          \
        MOE_LOAD_KK(FA_, kt, 1, 1);                                                        \
        MOE_MFMA_KK(FA_, 0);                                                               \
        if (kt + 1 < ktiles) {                                                             \
          /* Stage kt+1 visible to all waves; every wave is past its reads of */          \
          /* stage kt-1, so that slot can be refilled.                         */          \
          MOE_WAIT_STAGE(min(NS - 3, ktiles - kt - 2));                                    \
          if (kt + NS - 1 < ktiles) MOE_RING_ISSUE(kt + NS - 1, (kt + NS - 1) % NS);       \
          MOE_LOAD_KK(FA_, kt + 1, 0, 0);                                                  \
        }                                                                                  \
        MOE_MFMA_KK(FA_, 1);                                                               \
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
  // One self-contained copy (accumulators, K loop, epilogue) per number of
  // live fragments, so no accumulator value crosses from one copy to another.
#define MOE_TILE(FA_)                                                                      \
  do {                                                                                     \
    floatx16 acc[(FA_) > 0 ? (FA_) : 1][FN];                                               \
    floatx16 acc2[DUAL && (FA_) > 0 ? (FA_) : 1][FN2];                                     \
    MOE_K_LOOP(FA_);                                                                       \
    MOE_EPILOGUE(FA_);                                                                     \
  } while (0)

  static_assert(FM == 5 || FM == 2, "one copy per live-fragment count 0..FM");
  if constexpr (FM == 5) {
    switch (fa) {
      case 0: MOE_TILE(0); break;
      case 1: MOE_TILE(1); break;
      case 2: MOE_TILE(2); break;
      case 3: MOE_TILE(3); break;
      case 4: MOE_TILE(4); break;
      default: MOE_TILE(5); break;
    }
  } else {
    switch (fa) {
      case 0: MOE_TILE(0); break;
      case 1: MOE_TILE(1); break;
      default: MOE_TILE(2); break;
    }
  }
#undef MOE_TILE
#undef MOE_EPILOGUE
#undef MOE_K_LOOP
#undef MOE_LOAD_KK
#undef MOE_MFMA_KK
#undef MOE_WAIT_STAGE
#undef MOE_RING_ISSUE
#undef MOE_ISSUE_W
#undef MOE_ISSUE_A
#undef MOE_WAIT_W
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
static int ffn_bm(int dtype, int E, int max_rows) {
  if (dtype == 0) return kF32BM;
  return (long long)max_rows <= 32LL * E ? kGemmBMSmall : kGemmBM;
}

// Upper bound of row tiles: every expert may end in a partial tile.
static int max_m_tiles(int max_rows, int BM, int E) { return (max_rows + BM - 1) / BM + E; }

static size_t ffn_plan_bytes(int E, int max_rows, int dtype) {
  return align256(sizeof(int32_t)) +
         align256((size_t)max_m_tiles(max_rows, ffn_bm(dtype, E, max_rows), E) * sizeof(int4));
}

// 16-row groups of the packed bf16 hidden buffer: each tile rounds its rows up
// to whole groups, so at most one partial group per tile.
static int ffn_groups(int E, int max_rows) {
  return (max_rows + 15) / 16 + max_m_tiles(max_rows, ffn_bm(1, E, max_rows), E);
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
  ffn_plan_tiles<<<1, 1024, 0, st>>>(a.offsets, a.E, ffn_bm(a.dtype, a.E, a.max_rows), a.max_rows,
                                     ffn_tiles(a),
                                     ffn_count(a));
  return hipGetLastError();
}

template <int BM, int BN, int ACT, int MODE>
static void launch_bf16(const bf16_t* A, const bf16_t* B, const bf16_t* B2, bf16_t* C, int K,
                        int N, const FfnArgs& a, hipStream_t st) {
  const int nt = (N + BN - 1) / BN;
  const int g = grid_of(max_m_tiles(a.max_rows, BM, a.E), nt);
  // Groups of 4 row tiles once experts average two or more row tiles: an XCD's
  // 32 concurrent blocks then cover 4 x 8 tiles, and its L2 misses per K stage
  // fall from 1 A tile + 32 weight slabs to 4 A tiles + 8 weight slabs.
  const int gm = a.max_rows / a.E >= 2 * BM ? 4 : 1;
  grouped_gemm_bf16<BM, BN, ACT, MODE><<<g, kGemmWaves * 64, 0, st>>>(
      A, B, B2, C, K, N, ffn_tiles(a), ffn_count(a), nt, ffn_groups(a.E, a.max_rows), gm);
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
    if (ffn_bm(1, a.E, a.max_rows) == kGemmBMSmall) {
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
    } else if (a.act == ACT_SWIGLU) {
      launch_bf16<kGemmBM, 128, ACT_SWIGLU, kUpGemm>(X, W1, W3, H, a.d, a.h, a, st);
    } else if (a.h >= 2048) {
      if (a.act == ACT_RELU) launch_bf16<kGemmBM, 256, ACT_RELU, kUpGemm>(X, W1, nullptr, H, a.d, a.h, a, st);
      else launch_bf16<kGemmBM, 256, ACT_GELU, kUpGemm>(X, W1, nullptr, H, a.d, a.h, a, st);
    } else {
      if (a.act == ACT_RELU) launch_bf16<kGemmBM, 128, ACT_RELU, kUpGemm>(X, W1, nullptr, H, a.d, a.h, a, st);
      else launch_bf16<kGemmBM, 128, ACT_GELU, kUpGemm>(X, W1, nullptr, H, a.d, a.h, a, st);
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
    if (ffn_bm(1, a.E, a.max_rows) == kGemmBMSmall) {
      constexpr int S = kGemmBMSmall;
      if (a.d >= 2048) launch_bf16<S, 512, ACT_NONE, kDownGemm>(H, W2, nullptr, Y, a.h, a.d, a, st);
      else launch_bf16<S, 256, ACT_NONE, kDownGemm>(H, W2, nullptr, Y, a.h, a.d, a, st);
    } else if (a.d >= 1024) {
      launch_bf16<kGemmBM, 256, ACT_NONE, kDownGemm>(H, W2, nullptr, Y, a.h, a.d, a, st);
    } else {
      launch_bf16<kGemmBM, 128, ACT_NONE, kDownGemm>(H, W2, nullptr, Y, a.h, a.d, a, st);
    }
  }
  return hipGetLastError();
}

}  // namespace moe
