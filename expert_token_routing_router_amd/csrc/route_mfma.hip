// route_mfma.hip -- certified router scoring for bf16 inputs on gfx950.
//
// The router logit is defined exactly (fp64 sum left to right of exact
// products, bias added in fp64, one rounding to fp32).  Computing that for
// every (token, expert) costs 2*N*d*E fp64 operations, which is far above the
// memory time of reading x once when E >= 64.  Selection only needs exact
// values where they decide something, so:
//
//  1. logits_mfma      z~ = sum over K chunks of 64 of the bf16 MFMA chunk sum
//                      (fp32 accumulation, exact products), added up in fp64,
//                      plus the bias; also sum_i x_ti^2 and sum_i w_ei^2 in fp64.
//                      Error bound: each fp32 rounding in a chunk of 64 exact
//                      products is at most 2^-23 of a partial sum bounded by
//                      S_c = sum over the chunk of |x_i w_i|; with at most 64
//                      roundings per chunk the chunk error is <= 2^-17 S_c, so
//                      |z~ - exact| <= 2^-17 S with S <= |x_t| |w_e| (Cauchy-
//                      Schwarz).  The definition's own fp64 summation and fp32
//                      rounding add at most 2^-40 S + 2^-24 |z|.  The margin
//                      used is m = 2^-16 |x_t| |w_e| + 2^-22 |z~| + 2^-90.
//  2. route_certify    one wave per token: selection-score intervals (the score
//                      map -- identity or sigmoid, then + selection bias in
//                      fp32 -- is monotone, so the interval ends map through
//                      it); groups that are certainly kept / certainly dropped
//                      / undecided; the experts that can still be selected or
//                      can still be the maximum of an undecided group.  Those
//                      (token, expert) pairs go to a list.
//  3. route_exact      the exact definition for every listed pair (one lane,
//                      one sequential fp64 chain), overwriting z~.
//  4. route_finalize   one wave per token: group and top-k selection from exact
//                      values (every expert left out of the list is certainly
//                      not selected), combine weights, per-expert counts.
//
// Passages: glossary "Expert Parallelism", "How tokens travel between GPUs"
// (step 1 and the snippet's Linear router) and "Load balancing and capacity"
// (selection-only bias; node-limited routing as the group limit).
#include "device.h"
#include "kernels.h"

namespace moe {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int kRouteTokTile = 64;   // tokens per block in logits_mfma
constexpr int kRouteExpTile = 64;   // experts per block (4 waves x 16)
constexpr int kRouteKChunk = 64;    // K chunk accumulated in fp32

// ------------------------------------------------------------ 1. scores ---

// Grid (ceil(N/64), ceil(E/64)); 256 threads.  Wave w covers the block's 64
// tokens x experts [16w, 16w+16) with four 16x16 MFMA blocks
// (v_mfma_f32_16x16x32_bf16, tokens as rows).  LDS rows are 64 bf16 = eight
// 16-byte chunks, chunk c of row r stored at c ^ (r & 7).
__global__ __launch_bounds__(256) void logits_mfma(const bf16_t* __restrict__ x,
                                                   const bf16_t* __restrict__ w, int N, int d,
                                                   int E, const float* __restrict__ router_bias,
                                                   float* __restrict__ logits,
                                                   double* __restrict__ sumsq_x,
                                                   double* __restrict__ sumsq_w,
                                                   int32_t* __restrict__ zero_counts,
                                                   int32_t* __restrict__ zero_pairs) {
  __shared__ u32x4 xs[kRouteTokTile * 8];
  __shared__ u32x4 ws[kRouteExpTile * 8];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int t0 = blockIdx.x * kRouteTokTile, e0 = blockIdx.y * kRouteExpTile;
  if (blockIdx.x == 0 && blockIdx.y == 0) {
    for (int e = tid; e < E; e += 256) zero_counts[e] = 0;
    if (tid == 0) *zero_pairs = 0;
  }

  // Each thread stages 2 x-chunks and 2 w-chunks per K chunk: rows tid/8 and
  // tid/8 + 32, chunk tid % 8.  It also accumulates their squares.
  const int cr = tid >> 3, cc = tid & 7;
  double sx[2] = {0.0, 0.0}, sw[2] = {0.0, 0.0};
  floatx4 acc32[4];
  double acc[4][4];
#pragma unroll
  for (int b = 0; b < 4; ++b)
#pragma unroll
    for (int v = 0; v < 4; ++v) acc[b][v] = 0.0;

  const u32x4 zero4 = {0u, 0u, 0u, 0u};
  // The next chunk's global loads are issued before the current chunk's
  // MFMAs (two register sets, loop unrolled by two).
  u32x4 rx0[2], rw0[2], rx1[2], rw1[2];
#define MOE_LOGITS_LOAD(k0_, RX, RW)                                                        \
  do {                                                                                      \
    _Pragma("unroll") for (int h = 0; h < 2; ++h) {                                         \
      const int r = cr + 32 * h, kc = (k0_) + cc * 8;                                       \
      RX[h] = (t0 + r < N && kc < d) ? *reinterpret_cast<const u32x4*>(x + (size_t)(t0 + r) * d + kc) \
                                     : zero4;                                              \
      RW[h] = (e0 + r < E && kc < d) ? *reinterpret_cast<const u32x4*>(w + (size_t)(e0 + r) * d + kc) \
                                     : zero4;                                              \
    }                                                                                       \
  } while (0)
#define MOE_LOGITS_CHUNK(RX, RW)                                                            \
  do {                                                                                      \
    __syncthreads();                                                                        \
    _Pragma("unroll") for (int h = 0; h < 2; ++h) {                                         \
      const int r = cr + 32 * h;                                                            \
      xs[r * 8 + (cc ^ (r & 7))] = RX[h];                                                   \
      ws[r * 8 + (cc ^ (r & 7))] = RW[h];                                                   \
      _Pragma("unroll") for (int q = 0; q < 4; ++q) {                                       \
        const uint32_t a_ = RX[h][q], b_ = RW[h][q];                                        \
        const double a0 = bf16_to_f32(a_ & 0xffffu), a1 = bf16_to_f32(a_ >> 16);            \
        const double b0 = bf16_to_f32(b_ & 0xffffu), b1 = bf16_to_f32(b_ >> 16);            \
        sx[h] = fma(a0, a0, fma(a1, a1, sx[h]));                                            \
        sw[h] = fma(b0, b0, fma(b1, b1, sw[h]));                                            \
      }                                                                                     \
    }                                                                                       \
    __syncthreads();                                                                        \
  } while (0)
#define MOE_LOGITS_MFMA()                                                                   \
  do {                                                                                      \
    _Pragma("unroll") for (int b = 0; b < 4; ++b) acc32[b] = floatx4{0.f, 0.f, 0.f, 0.f};   \
    _Pragma("unroll") for (int ks = 0; ks < kRouteKChunk / 32; ++ks) {                      \
      const int c = ks * 4 + (lane >> 4);                                                   \
      const int er = wave * 16 + (lane & 15);                                               \
      const bf16x8_t bw = __builtin_bit_cast(bf16x8_t, ws[er * 8 + (c ^ (er & 7))]);        \
      _Pragma("unroll") for (int b = 0; b < 4; ++b) {                                       \
        const int tr = b * 16 + (lane & 15);                                                \
        const bf16x8_t ax = __builtin_bit_cast(bf16x8_t, xs[tr * 8 + (c ^ (tr & 7))]);      \
        acc32[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ax, bw, acc32[b], 0, 0, 0);      \
      }                                                                                     \
    }                                                                                       \
    _Pragma("unroll") for (int b = 0; b < 4; ++b)                                           \
        _Pragma("unroll") for (int v = 0; v < 4; ++v) acc[b][v] += (double)acc32[b][v];     \
  } while (0)

  MOE_LOGITS_LOAD(0, rx0, rw0);
  for (int k0 = 0; k0 < d; k0 += 2 * kRouteKChunk) {
    MOE_LOGITS_CHUNK(rx0, rw0);
    if (k0 + kRouteKChunk < d) MOE_LOGITS_LOAD(k0 + kRouteKChunk, rx1, rw1);
    MOE_LOGITS_MFMA();
    if (k0 + kRouteKChunk >= d) break;
    MOE_LOGITS_CHUNK(rx1, rw1);
    if (k0 + 2 * kRouteKChunk < d) MOE_LOGITS_LOAD(k0 + 2 * kRouteKChunk, rx0, rw0);
    MOE_LOGITS_MFMA();
  }
#undef MOE_LOGITS_LOAD
#undef MOE_LOGITS_CHUNK
#undef MOE_LOGITS_MFMA

  // Sums of squares: the 8 threads of a row (consecutive lanes) combine.
#pragma unroll
  for (int h = 0; h < 2; ++h) {
#pragma unroll
    for (int o = 1; o < 8; o <<= 1) {
      sx[h] += __shfl_xor(sx[h], o, 64);
      sw[h] += __shfl_xor(sw[h], o, 64);
    }
    const int r = cr + 32 * h;
    if (cc == 0) {
      if (blockIdx.y == 0 && t0 + r < N) sumsq_x[t0 + r] = sx[h];
      if (blockIdx.x == 0 && e0 + r < E) sumsq_w[e0 + r] = sw[h];
    }
  }

  // C block b: lane holds expert (lane & 15) of this wave, tokens 4*(lane>>4)+v.
  const int e = e0 + wave * 16 + (lane & 15);
  if (e < E) {
    const double bias = router_bias ? (double)router_bias[e] : 0.0;
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int t = t0 + b * 16 + 4 * (lane >> 4) + v;
        if (t < N) logits[(size_t)t * E + e] = (float)(acc[b][v] + bias);
      }
  }
}

// ----------------------------------------------------------- 2. certify ---

__device__ __forceinline__ float sigmoid_affinity_v2(float z) {
  return __double2float_rn(1.0 / (1.0 + exp(-(double)z)));
}

// Selection score of an fp32 logit, exactly as the definition computes it.
__device__ __forceinline__ float sel_score(float z, int score_fn, float bias) {
  const float a = score_fn == 2 ? sigmoid_affinity_v2(z) : z;
  return a + bias;
}

// Does (sa, a) certainly rank before (sb, b) when only sa >= lower end of a's
// score and sb <= upper end of b's are known?  Called with lo(a), hi(b).
__device__ __forceinline__ bool certainly_before(float lo_a, int a, float hi_b, int b) {
  return lo_a > hi_b || (lo_a == hi_b && a < b);
}

constexpr int kCertTokensPerBlock = 64;
constexpr int kCertWaves = 16;  // 4 tokens per wave; occupancy hides per-token latency

// One wave per token.  Lane l holds experts l, l+64, l+128, l+192.
// Outputs per token: cand[t][4] (bit e set: e needs its exact logit),
// gmask[t][2] = {certainly kept groups, undecided groups}; pairs appended.
__global__ __launch_bounds__(kCertWaves * 64) void route_certify(
    const float* __restrict__ logits, const double* __restrict__ sumsq_x,
    const double* __restrict__ sumsq_w, const float* __restrict__ sel_bias, int N, int E, int k,
    int G, int kg, int score_fn, uint64_t* __restrict__ cand, uint64_t* __restrict__ gmask,
    int32_t* __restrict__ pairs, int32_t* __restrict__ pair_count) {
  static_assert(kCertTokensPerBlock == 64, "the pair scan is one wave wide");
  __shared__ float glo_s[kCertWaves][64], ghi_s[kCertWaves][64];
  __shared__ float lo_s[kCertWaves][256], hi_s[kCertWaves][256];
  __shared__ uint64_t cand_s[kCertTokensPerBlock][4];  // this block's candidate masks
  __shared__ int32_t cnt_s[kCertTokensPerBlock];       // candidates per token, then offsets
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int per = E / G;
  const int t_begin = blockIdx.x * kCertTokensPerBlock;
  const int t_end = min(N, t_begin + kCertTokensPerBlock);
  double nw[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int e = lane + 64 * j;
    nw[j] = e < E ? sqrt(sumsq_w[e]) : 0.0;
  }
  for (int t = t_begin + wave; t < t_end; t += kCertWaves) {
    const double nx = sqrt(sumsq_x[t]);
    float lo[4], hi[4];
    bool ok[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = lane + 64 * j;
      ok[j] = e < E;
      lo[j] = -INFINITY;
      hi[j] = -INFINITY;
      if (ok[j]) {
        const double zt = (double)logits[(size_t)t * E + e];
        // 2^-16 |x||w| (with a relative pad for the rounded norms), 2^-22 |z|.
        const double m = 1.52587890625e-05 * (nx * nw[j]) * (1.0 + 1e-12) +
                         2.384185791015625e-07 * fabs(zt) + 1e-27;
        const float zlo = __double2float_rd(zt - m), zhi = __double2float_ru(zt + m);
        const float b = sel_bias ? sel_bias[e] : 0.f;
        lo[j] = sel_score(zlo, score_fn, b);
        hi[j] = sel_score(zhi, score_fn, b);
      }
    }

    // Groups: certainly kept, undecided (bit masks over G <= 64 groups).
    uint64_t kept_c = ~0ull, undecided = 0ull;
    if (G > 1) {
      // Group maxima of the lower and upper ends: lane g < G scans group g.
      float gl = -INFINITY, gh = -INFINITY;
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (ok[j]) {
          lo_s[wave][lane + 64 * j] = lo[j];
          hi_s[wave][lane + 64 * j] = hi[j];
        }
      __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
      __builtin_amdgcn_wave_barrier();
      if (lane < G) {
        for (int e = lane * per; e < (lane + 1) * per; ++e) {
          gl = fmaxf(gl, lo_s[wave][e]);
          gh = fmaxf(gh, hi_s[wave][e]);
        }
        glo_s[wave][lane] = gl;
        ghi_s[wave][lane] = gh;
      }
      __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
      __builtin_amdgcn_wave_barrier();
      bool keep = false, drop = false;
      if (lane < G) {
        int could_beat = 0, beaten = 0;
        for (int h = 0; h < G; ++h) {
          if (h == lane) continue;
          const float glh = glo_s[wave][h], ghh = ghi_s[wave][h];
          if (!certainly_before(gl, lane, ghh, h)) ++could_beat;
          if (certainly_before(glh, h, gh, lane)) ++beaten;
        }
        keep = could_beat <= kg - 1;
        drop = beaten >= kg;
      }
      kept_c = __ballot(lane < G && keep);
      undecided = __ballot(lane < G && !keep && !drop);
      __builtin_amdgcn_wave_barrier();
    }

    // k-th largest lower end among experts of certainly kept groups.
    bool comp[4], elig[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int g = (lane + 64 * j) / per;
      comp[j] = ok[j] && ((kept_c >> g) & 1ull);
      elig[j] = ok[j] && (((kept_c | undecided) >> g) & 1ull);
    }
    float thr = -INFINITY;
    {
      bool used[4] = {false, false, false, false};
      float tv = -INFINITY;
      int ti = -1;
      for (int r = 0; r < k; ++r) {
        float bs = 0.f;
        int bi = -1;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int e = lane + 64 * j;
          if (comp[j] && !used[j] && (bi < 0 || lo[j] > bs)) {
            bs = lo[j];
            bi = e;
          }
        }
        wave_argmax(bs, bi);
        if (bi < 0) {  // fewer than k competitors: nobody is certainly out
          ti = -1;
          break;
        }
        tv = bs;
        ti = bi;
        if (lane == (bi & 63)) {
#pragma unroll
          for (int j = 0; j < 4; ++j)
            if (bi == lane + 64 * j) used[j] = true;
        }
      }
      thr = ti < 0 ? -INFINITY : tv;
    }

    // Candidates: eligible experts that are not certainly out, plus possible
    // maxima of undecided groups.
    uint64_t cw[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = lane + 64 * j;
      bool c = elig[j] && hi[j] >= thr;
      if (ok[j] && G > 1) {
        const int g = e / per;
        if ((undecided >> g) & 1ull) c = c || hi[j] >= glo_s[wave][g];
      }
      cw[j] = __ballot(c);
    }
    if (lane < 4) {
      uint64_t v = cw[0];
#pragma unroll
      for (int j = 1; j < 4; ++j)
        if (lane == j) v = cw[j];
      cand[(size_t)t * 4 + lane] = v;
    }
    if (lane == 0) {
      gmask[(size_t)t * 2 + 0] = kept_c;
      gmask[(size_t)t * 2 + 1] = undecided;
    }
    int n = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) n += __popcll(cw[j]);
    if (lane < 4) {
      uint64_t v = cw[0];
#pragma unroll
      for (int j = 1; j < 4; ++j)
        if (lane == j) v = cw[j];
      cand_s[t - t_begin][lane] = v;
    }
    if (lane == 0) cnt_s[t - t_begin] = n;
  }

  // Append this block's (t, e) pairs with one global atomic: an exclusive
  // scan of the per-token counts (64 entries, one wave), then each wave
  // writes the pairs of its tokens.
  __syncthreads();
  const int nt = t_end - t_begin;
  if (wave == 0) {
    int c = lane < nt ? cnt_s[lane] : 0;
    int incl = c;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int v = __shfl_up(incl, o, 64);
      if (lane >= o) incl += v;
    }
    const int total = __shfl(incl, 63, 64);
    int base = 0;
    if (lane == 0) base = atomicAdd(pair_count, total);
    base = __shfl(base, 0, 64);
    if (lane < nt) cnt_s[lane] = base + incl - c;
  }
  __syncthreads();
  for (int tl = wave; tl < nt; tl += kCertWaves) {
    const int t = t_begin + tl;
    int base = cnt_s[tl];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint64_t m = cand_s[tl][j];
      const uint64_t below = lane == 0 ? 0ull : (m << (64 - lane));
      if ((m >> lane) & 1ull) pairs[base + __popcll(below)] = (t << 8) | (lane + 64 * j);
      base += __popcll(m);
    }
  }
}

// ------------------------------------------------------------- 3. exact ---

// The definition for every listed pair: fp64 sum, left to right, of the exact
// products x_ti w_ei, + bias, one rounding to fp32.  The sum is one
// sequential chain per pair (its rounding order is part of the definition),
// so a lane owns a pair; what the 64 lanes of a wave share is the memory
// traffic.  A one-wave block takes groups of 64 consecutive list entries and
// streams their x and w rows through LDS in chunks of 32 elements (64 bytes
// of each row, 8 KB per chunk for the group) with global_load_lds_dwordx4,
// up to kExactRing - 1 chunks ahead of the chains.  Load i of a chunk covers
// the rows of pairs 16(i%4) .. 16(i%4)+15 (x for i < 4, w after); lane L
// fetches row L/4 of those, logical 16-byte chunk (L % 4) ^ swz4(L / 4), so
// the chains' 16-byte LDS reads of one chunk spread over the banks.  Needs
// d % 32 == 0 (the launcher checks).
constexpr int kExactRing = 8;    // LDS chunk slots per wave, 8 KB each
constexpr int kExactBlocks = 2048;

__global__ __launch_bounds__(64) void route_exact(const bf16_t* __restrict__ x,
                                                  const bf16_t* __restrict__ w, int d, int E,
                                                  const float* __restrict__ router_bias,
                                                  const int32_t* __restrict__ pairs,
                                                  const int32_t* __restrict__ pair_count,
                                                  float* __restrict__ logits) {
  __shared__ __attribute__((aligned(1024))) char ring[kExactRing][8192];
  const int lane = threadIdx.x;
  const int n = *pair_count;
  const int nch = d / 32;
  const int mine = (lane & 15) * 4;  // this lane's row inside its 1-KB block: byte offset / 16
  const int msw = swz4(lane & 15);
  for (int g0 = blockIdx.x * 64; g0 < n; g0 += gridDim.x * 64) {
    const bool live = g0 + lane < n;
    const int v = pairs[live ? g0 + lane : g0];  // idle lanes shadow a listed pair
    const int t = v >> 8, e = v & 255;
    const u32x4* src[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int q = 16 * i + lane / 4;  // pair whose rows this lane fetches
      const int tq = __shfl(t, q, 64), eq = __shfl(e, q, 64);
      const int c = (lane % 4) ^ swz4(lane / 4);
      src[i] = reinterpret_cast<const u32x4*>(x + (size_t)tq * d) + c;
      src[4 + i] = reinterpret_cast<const u32x4*>(w + (size_t)eq * d) + c;
    }
#define MOE_EXACT_ISSUE(ch_)                                                                \
  do {                                                                                      \
    char* slot_ = ring[(ch_) % kExactRing];                                                 \
    _Pragma("unroll") for (int i = 0; i < 8; ++i)                                           \
        __builtin_amdgcn_global_load_lds((void*)(src[i] + (size_t)(ch_) * 4),               \
                                         (lds_ptr_t)(slot_ + i * 1024), 16, 0, 0);          \
  } while (0)
#pragma unroll
    for (int c = 0; c < kExactRing - 1; ++c)
      if (c < nch) MOE_EXACT_ISSUE(c);
    double acc = 0.0;
    for (int ch = 0; ch < nch; ++ch) {
      // Chunk ch has landed once at most `later` younger chunks (8 loads
      // each) are still in flight.
      switch (min(kExactRing - 2, nch - 1 - ch)) {
        case 0: wait_vmcnt<0>(); break;
        case 1: wait_vmcnt<8>(); break;
        case 2: wait_vmcnt<16>(); break;
        case 3: wait_vmcnt<24>(); break;
        case 4: wait_vmcnt<32>(); break;
        case 5: wait_vmcnt<40>(); break;
        default: wait_vmcnt<48>(); break;
      }
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
      // The slot of chunk ch-1 was consumed by the previous iteration.
      if (ch + kExactRing - 1 < nch) MOE_EXACT_ISSUE(ch + kExactRing - 1);
      const char* slot = ring[ch % kExactRing];
      const char* xb = slot + (lane >> 4) * 1024;
      const char* wb = slot + 4096 + (lane >> 4) * 1024;
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) {
        const int pos = (mine + (qq ^ msw)) * 16;
        const u32x4 a = *reinterpret_cast<const u32x4*>(xb + pos);
        const u32x4 b = *reinterpret_cast<const u32x4*>(wb + pos);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          acc = __fma_rn((double)bf16_to_f32(a[q] & 0xffffu), (double)bf16_to_f32(b[q] & 0xffffu),
                         acc);
          acc = __fma_rn((double)bf16_to_f32(a[q] >> 16), (double)bf16_to_f32(b[q] >> 16), acc);
        }
      }
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
    }
#undef MOE_EXACT_ISSUE
    if (live) {
      if (router_bias) acc = acc + (double)router_bias[e];
      logits[(size_t)t * E + e] = __double2float_rn(acc);
    }
  }
}

// ---------------------------------------------------------- 4. finalize ---

__global__ __launch_bounds__(kCertWaves * 64) void route_finalize(
    const float* __restrict__ logits, const float* __restrict__ sel_bias,
    const uint64_t* __restrict__ cand, const uint64_t* __restrict__ gmask, int N, int E, int k,
    int G, int kg, int score_fn, int32_t* __restrict__ topk_idx, float* __restrict__ topk_w,
    int32_t* __restrict__ counts) {
  __shared__ int32_t hist[256];
  __shared__ float s_s[kCertWaves][256];
  for (int e = threadIdx.x; e < E; e += blockDim.x) hist[e] = 0;
  __syncthreads();
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int per = E / G;
  const int t_begin = blockIdx.x * kCertTokensPerBlock;
  const int t_end = min(N, t_begin + kCertTokensPerBlock);
  for (int t = t_begin + wave; t < t_end; t += kCertWaves) {
    float z[4], s[4];
    bool is_c[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = lane + 64 * j;
      const bool okj = e < E;
      z[j] = okj ? logits[(size_t)t * E + e] : 0.f;
      is_c[j] = okj && ((cand[(size_t)t * 4 + j] >> lane) & 1ull);
      s[j] = is_c[j] ? sel_score(z[j], score_fn, sel_bias ? sel_bias[e] : 0.f) : -INFINITY;
    }
    uint64_t kept = ~0ull;
    if (G > 1) {
      const uint64_t kept_c = gmask[(size_t)t * 2 + 0], undecided = gmask[(size_t)t * 2 + 1];
      kept = kept_c;
      const int need = kg - __popcll(kept_c);
      if (need > 0 && undecided) {
        // Exact maxima of undecided groups (all their possible maxima are
        // candidates, so the maximum over candidates is the group score).
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (lane + 64 * j < E) s_s[wave][lane + 64 * j] = s[j];
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
        __builtin_amdgcn_wave_barrier();
        float gs = 0.f;
        int gi = -1;
        if (lane < G && ((undecided >> lane) & 1ull)) {
          float m = -INFINITY;
          for (int e = lane * per; e < (lane + 1) * per; ++e) m = fmaxf(m, s_s[wave][e]);
          gs = m;
          gi = lane;
        }
        for (int r = 0; r < need; ++r) {
          float bs = gs;
          int bi = gi;
          wave_argmax(bs, bi);
          if (bi < 0) break;
          kept |= 1ull << bi;
          if (lane == bi) gi = -1;
        }
        __builtin_amdgcn_wave_barrier();
      }
    }
    bool elig[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) elig[j] = is_c[j] && ((kept >> ((lane + 64 * j) / per)) & 1ull);

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
        for (int j = 0; j < 4; ++j) {
          const int e = lane + 64 * j;
          if (elig[j] && (bi < 0 || s[j] > bs)) {
            bs = s[j];
            bi = e;
          }
        }
        wave_argmax(bs, bi);
        sel[r] = bi;
        const int owner = bi & 63, jj = bi >> 6;
        float zv = z[0];
#pragma unroll
        for (int j = 1; j < 4; ++j)
          if (jj == j) zv = z[j];
        zsel[r] = __shfl(zv, owner, 64);
        if (lane == owner) {
#pragma unroll
          for (int j = 0; j < 4; ++j)
            if (jj == j) elig[j] = false;
        }
      }
    }

    double wsum = 0.0, wv[8];
    if (score_fn == 0) {
      double zmax = (double)zsel[0];
#pragma unroll
      for (int r = 1; r < 8; ++r)
        if (r < k) zmax = fmax(zmax, (double)zsel[r]);
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        wv[r] = r < k ? exp((double)zsel[r] - zmax) : 0.0;
        wsum += wv[r];
      }
    } else if (score_fn == 1) {
      float m = -INFINITY;
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (lane + 64 * j < E) m = fmaxf(m, z[j]);
      const double zmax = (double)wave_max(m);
      double part = 0.0;
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (lane + 64 * j < E) part += exp((double)z[j] - zmax);
      wsum = wave_sum(part);
#pragma unroll
      for (int r = 0; r < 8; ++r) wv[r] = r < k ? exp((double)zsel[r] - zmax) : 0.0;
    } else {
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        wv[r] = r < k ? (double)sigmoid_affinity_v2(zsel[r]) : 0.0;
        wsum += wv[r];
      }
    }
    int my_e = sel[0];
    double my_w = wv[0];
#pragma unroll
    for (int r = 1; r < 8; ++r)
      if (lane == r) {
        my_e = sel[r];
        my_w = wv[r];
      }
    if (lane < k) {
      topk_idx[(size_t)t * k + lane] = my_e;
      topk_w[(size_t)t * k + lane] = (float)(my_w / wsum);
      if (my_e >= 0) atomicAdd(&hist[my_e], 1);
    }
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += blockDim.x)
    if (hist[e]) atomicAdd(&counts[e], hist[e]);
}

// ---------------------------------------------------------------- launch ---

static size_t a256(size_t v) { return (v + 255) / 256 * 256; }

struct CertWs {
  double* sumsq_x;
  double* sumsq_w;
  uint64_t* cand;
  uint64_t* gmask;
  int32_t* pairs;
  int32_t* pair_count;
};

static CertWs cert_layout(void* ws, int N, int E) {
  char* p = static_cast<char*>(ws);
  CertWs c;
  c.sumsq_x = reinterpret_cast<double*>(p);
  p += a256((size_t)N * 8);
  c.sumsq_w = reinterpret_cast<double*>(p);
  p += a256((size_t)E * 8);
  c.cand = reinterpret_cast<uint64_t*>(p);
  p += a256((size_t)N * 4 * 8);
  c.gmask = reinterpret_cast<uint64_t*>(p);
  p += a256((size_t)N * 2 * 8);
  c.pairs = reinterpret_cast<int32_t*>(p);
  p += a256((size_t)N * E * 4);
  c.pair_count = reinterpret_cast<int32_t*>(p);
  return c;
}

size_t route_certified_workspace_bytes(int N, int E) {
  if (N <= 0) return 0;
  return a256((size_t)N * 8) + a256((size_t)E * 8) + a256((size_t)N * 32) + a256((size_t)N * 16) +
         a256((size_t)N * E * 4) + 256;
}

hipError_t launch_route_certified(const RouteArgs& a, hipStream_t st) {
  const CertWs c = cert_layout(a.ws, a.N, a.E);
  const bf16_t* x = static_cast<const bf16_t*>(a.x);
  const bf16_t* w = static_cast<const bf16_t*>(a.w_router);
  dim3 g1((a.N + kRouteTokTile - 1) / kRouteTokTile, (a.E + kRouteExpTile - 1) / kRouteExpTile);
  logits_mfma<<<g1, 256, 0, st>>>(x, w, a.N, a.d, a.E, a.router_bias, a.logits, c.sumsq_x,
                                   c.sumsq_w, a.counts, c.pair_count);
  const int blocks = (a.N + kCertTokensPerBlock - 1) / kCertTokensPerBlock;
  route_certify<<<blocks, kCertWaves * 64, 0, st>>>(a.logits, c.sumsq_x, c.sumsq_w, a.sel_bias, a.N, a.E,
                                        a.k, a.G, a.kg, a.score_fn, c.cand, c.gmask, c.pairs,
                                        c.pair_count);
  route_exact<<<kExactBlocks, 64, 0, st>>>(x, w, a.d, a.E, a.router_bias, c.pairs,
                                           c.pair_count, a.logits);
  route_finalize<<<blocks, kCertWaves * 64, 0, st>>>(a.logits, a.sel_bias, c.cand, c.gmask, a.N, a.E, a.k,
                                         a.G, a.kg, a.score_fn, a.topk_idx, a.topk_w, a.counts);
  return hipGetLastError();
}

}  // namespace moe
