// route_mfma.hip -- certified router scoring for bf16 inputs on gfx950.
//
// The router logit is defined exactly (fp64 sum left to right of exact
// products, bias added in fp64, one rounding to fp32).  Computing that for
// every (token, expert) costs 2*N*d*E fp64 operations, far above the memory
// time of reading x once when E >= 64.  Selection only needs exact values
// where they decide something, so the scores come from bf16 MFMAs with a
// proven error bound, and only the (token, expert) pairs the bound cannot
// settle are recomputed by the definition.  One kernel does all of it per
// tile of tokens (see route_fused).
#include "device.h"
#include "kernels.h"

namespace moe {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

// Fused per-tile routing.  One block of 8 waves owns kFuseTok consecutive
// tokens and runs every step for them, so the approximate logits, the
// candidate sets and the exact values never leave LDS:
//
//  1. scores     for each tile of 64 experts, stream the tokens' x rows and
//                the experts' w rows through an LDS ring in chunks of 32
//                elements (global_load_lds_dwordx4); wave w multiplies tokens
//                16(w/4).. by experts 16(w%4).. of the tile with
//                v_mfma_f32_16x16x32_bf16 (fp32 within 64-element chunks, fp64
//                across); upper bounds of sum x_ti^2 and sum w_ei^2 come from
//                the diagonals of X X^T and W W^T by the same MFMA on the same
//                operands (fp32 per 64 elements, padded by 2^-17 relative and
//                2^-120 absolute, summed in fp64).  z~ = that sum + bias, kept
//                as fp32.  Error bound: each fp32 rounding in a chunk of at
//                most 64 exact products is at most 2^-23 of a partial sum
//                bounded by S_c = sum over the chunk of |x_i w_i|, so the
//                chunk error is <= 2^-17 S_c and |z~ - exact| <= 2^-17 S with
//                S <= |x_t| |w_e| (Cauchy-Schwarz); the definition's own fp64
//                summation and fp32 rounding add at most 2^-40 S + 2^-24 |z|.
//                Margin used: m = 2^-16 |x_t| |w_e| + 2^-22 |z~| + 1e-27.
//  2. certify    one wave per token: selection-score intervals (the score map
//                -- identity or sigmoid, then + selection bias in fp32 -- is
//                monotone, so the interval ends map through it); groups that
//                are certainly kept / certainly dropped / undecided; the
//                experts that can still be selected or can still be the
//                maximum of an undecided group become (token, expert) pairs.
//  3. exact      the definition for every pair -- fp64 sum left to right of
//                exact products, + bias, one rounding.  Where a test on the
//                products' exponents proves that chain rounds nowhere, 16
//                lanes sum the pair's products in any order (same bits);
//                otherwise one lane runs the chain itself;
//                the rows were streamed in step 1, so they come from L2.
//  4. finalize   one wave per token: group and top-k selection from exact
//                values (every expert outside the candidate set is certainly
//                not selected), combine weights; then the tile's logits, its
//                top-k rows and its per-expert counts go out.
//
// Passages: glossary "Expert Parallelism", "How tokens travel between GPUs"
// (step 1 and the snippet's Linear router) and "Load balancing and capacity"
// (selection-only bias; node-limited routing as the group limit).
constexpr int kFuseTok = 32;                     // tokens per block
constexpr int kFuseWaves = 8;
constexpr int kFuseRing = 6;  // LDS chunk slots in step 1 (11 measured slower)
// Pair slots (two chunks each) of step 1: 4 in the one-launch route, 6 in the
// scoring launch of a split route (it holds no candidate lists or per-token
// state, so two blocks per CU still fit); the tail launch keeps the ring of
// kFuseRing chunks as scratch only.
constexpr int kFusePairs = 4;
constexpr int kScorePairs = 6;
constexpr int kFuseSlot = (kFuseTok + 64) * 64;  // bytes: 32 x rows + 64 w rows of 64 B

__device__ __forceinline__ float sigmoid_affinity_v2(float z) {
  return __double2float_rn(1.0 / (1.0 + exp(-(double)z)));
}

// Selection score of an fp32 logit, exactly as the definition computes it.
__device__ __forceinline__ float sel_score(float z, int score_fn, float bias) {
  const float a = score_fn == 2 ? sigmoid_affinity_v2(z) : z;
  return a + bias;
}

// Exponent of the lowest set bit of a nonzero finite fp64 value: v is an
// integer multiple of 2^lowbit_exp(v) (significand m, with the implicit bit
// for normal values, times 2^(biased exponent - 1075); subnormals 2^-1074).
__device__ __forceinline__ int lowbit_exp(double v) {
  const uint64_t b = (uint64_t)__double_as_longlong(v);
  const int be = (int)((b >> 52) & 0x7ff);
  const uint64_t m = (b & 0xfffffffffffffull) | (be ? (1ull << 52) : 0ull);
  return (be ? be : 1) - 1075 + __builtin_ctzll(m);
}

// Does (sa, a) certainly rank before (sb, b) when only sa >= lower end of a's
// score and sb <= upper end of b's are known?  Called with lo(a), hi(b).
__device__ __forceinline__ bool certainly_before(float lo_a, int a, float hi_b, int b) {
  return lo_a > hi_b || (lo_a == hi_b && a < b);
}

// Steps 2-4 of one tile of nt <= kFuseTok tokens starting at t0, given the
// approximate logits in zs and the squared norms sx (tokens) and sw (experts):
// certify, exact values for the candidate pairs, selection and weights, the
// tile's logits, and per-expert counts added to hist.  scratch (LDS) holds
// the pair lists and the group-limit scratch: at least
// max(4 * kFuseTok * ZW, 8 * kFuseWaves * ZW + 512 * kFuseWaves) bytes.
template <int NJ, int ZW>
__device__ __forceinline__ void route_tile_tail(
    const bf16_t* __restrict__ x, const bf16_t* __restrict__ w, int d, int E, int k, int G,
    int kg, int score_fn, const float* __restrict__ router_bias,
    const float* __restrict__ sel_bias, float* __restrict__ logits,
    int32_t* __restrict__ topk_idx, float* __restrict__ topk_w, int t0, int nt,
    float (*zs)[ZW], char* scratch, const double* sx, const double* sw,
    uint64_t (*cand_s)[4], uint64_t (*gm_s)[2], int32_t* cnt_s, int32_t* hist,
    int32_t& npairs_s, int32_t& nfb_s) {
  static_assert(ZW >= 64 * NJ, "a zs row holds every expert");
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  uint16_t* plist = reinterpret_cast<uint16_t*>(scratch);  // (t_local << 8) | e
  typedef float ExpRow[ZW];
  typedef float GroupRows[2][64];
  ExpRow* wsc = reinterpret_cast<ExpRow*>(scratch);                            // [8][E]: lower ends / scores
  ExpRow* wsc2 = reinterpret_cast<ExpRow*>(scratch + kFuseWaves * ZW * 4);     // [8][E]: upper ends
  GroupRows* gsc = reinterpret_cast<GroupRows*>(scratch + 2 * kFuseWaves * ZW * 4);
  // ---- 2. certify -------------------------------------------------------
  const int per = E / G;
  double nw[NJ];
  float sb[NJ];  // this lane's selection biases, read once per block
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int e = lane + 64 * j;
    nw[j] = e < E ? sqrt(sw[e]) : 0.0;
    sb[j] = (sel_bias && e < E) ? sel_bias[e] : 0.f;
  }
  for (int tl = wave; tl < nt; tl += kFuseWaves) {
    const double nx = sqrt(sx[tl]);
    float lo[NJ], hi[NJ];
    bool ok[NJ];
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int e = lane + 64 * j;
      ok[j] = e < E;
      lo[j] = -INFINITY;
      hi[j] = -INFINITY;
      if (ok[j]) {
        const double zt = (double)zs[tl][e];
        // 2^-16 |x||w| (with a relative pad for the rounded norms), 2^-22 |z|.
        const double m = 1.52587890625e-05 * (nx * nw[j]) * (1.0 + 1e-12) +
                         2.384185791015625e-07 * fabs(zt) + 1e-27;
        // Outward by one ulp after rounding to nearest: still an enclosure.
        const float zlo = nextafterf(__double2float_rn(zt - m), -INFINITY);
        const float zhi = nextafterf(__double2float_rn(zt + m), INFINITY);
        const float b = sb[j];
        lo[j] = sel_score(zlo, score_fn, b);
        hi[j] = sel_score(zhi, score_fn, b);
      }
    }
    // Groups: certainly kept, undecided (bit masks over G <= 64 groups).
    uint64_t kept_c = ~0ull, undecided = 0ull;
    if (G > 1) {
      float gl = -INFINITY, gh = -INFINITY;
#pragma unroll
      for (int j = 0; j < NJ; ++j)
        if (ok[j]) {
          wsc[wave][lane + 64 * j] = lo[j];
          wsc2[wave][lane + 64 * j] = hi[j];
        }
      __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
      __builtin_amdgcn_wave_barrier();
      if (lane < G) {
        for (int e = lane * per; e < (lane + 1) * per; ++e) {
          gl = fmaxf(gl, wsc[wave][e]);
          gh = fmaxf(gh, wsc2[wave][e]);
        }
        gsc[wave][0][lane] = gl;
        gsc[wave][1][lane] = gh;
      }
      __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
      __builtin_amdgcn_wave_barrier();
      bool keep = false, drop = false;
      if (lane < G) {
        int could_beat = 0, beaten = 0;
        for (int h = 0; h < G; ++h) {
          if (h == lane) continue;
          const float glh = gsc[wave][0][h], ghh = gsc[wave][1][h];
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
    bool comp[NJ], elig[NJ];
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int g = (lane + 64 * j) / per;
      comp[j] = ok[j] && ((kept_c >> g) & 1ull);
      elig[j] = ok[j] && (((kept_c | undecided) >> g) & 1ull);
    }
    float thr = -INFINITY;
    {
      bool used[NJ] = {};
      float tv = -INFINITY;
      int ti = -1;
      for (int r = 0; r < k; ++r) {
        float bs = 0.f;
        int bi = -1;
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
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
          for (int j = 0; j < NJ; ++j)
            if (bi == lane + 64 * j) used[j] = true;
        }
      }
      thr = ti < 0 ? -INFINITY : tv;
    }
    // Candidates: eligible experts that are not certainly out, plus possible
    // maxima of undecided groups.
    uint64_t cw[NJ];
    int n = 0;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int e = lane + 64 * j;
      bool c = elig[j] && hi[j] >= thr;
      if (ok[j] && G > 1) {
        const int g = e / per;
        if ((undecided >> g) & 1ull) c = c || hi[j] >= gsc[wave][0][g];
      }
      cw[j] = __ballot(c);
      n += __popcll(cw[j]);
    }
    if (lane < NJ) {
      uint64_t v = cw[0];
#pragma unroll
      for (int j = 1; j < NJ; ++j)
        if (lane == j) v = cw[j];
      cand_s[tl][lane] = v;
    }
    if (lane == 0) {
      gm_s[tl][0] = kept_c;
      gm_s[tl][1] = undecided;
      cnt_s[tl] = n;
    }
  }
  __syncthreads();
  // Pair list in LDS: exclusive scan of the per-token counts, then each wave
  // writes the pairs of its tokens.
  if (wave == 0) {
    const int c = lane < nt ? cnt_s[lane] : 0;
    int incl = c;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int v = __shfl_up(incl, o, 64);
      if (lane >= o) incl += v;
    }
    if (lane < nt) cnt_s[lane] = incl - c;
    if (lane == 63) {
      npairs_s = incl;
      nfb_s = 0;
    }
  }
  __syncthreads();
  for (int tl = wave; tl < nt; tl += kFuseWaves) {
    int base = cnt_s[tl];
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const uint64_t m = cand_s[tl][j];
      const uint64_t below = lane == 0 ? 0ull : (m << (64 - lane));
      if ((m >> lane) & 1ull) plist[base + __popcll(below)] = (uint16_t)((tl << 8) | (lane + 64 * j));
      base += __popcll(m);
    }
  }
  __syncthreads();

  // ---- 3. exact ---------------------------------------------------------
  // The definition sums exact products left to right in fp64.  Every
  // partial sum of that chain is exact when all products are multiples of
  // 2^m and sum |x_i w_i| < 2^(m+53): then the fp64 result is the exact dot
  // product, and any order of summation gives the same bits.  A product p of
  // two bf16 values is a multiple of 2^(frexp_exp(p) - 16) (8-bit
  // significands, so its lowest bit sits at most 16 places below its top
  // bit, which is frexp_exp(p) - 1); a zero product reports exponent 0,
  // which can only lower the minimum.  Cauchy-Schwarz bounds sum |x_i w_i|
  // by sqrt(sum x^2 * sum w^2), both already summed in step 1 (their fp64
  // rounding is covered by the 2^-20 pad).  So: 16 lanes per pair, each
  // summing a strided share of the products; the pair's lanes reduce the
  // sum and the minimum exponent; pairs that pass the test are done, the
  // others go to a list and run the chain one lane each below.
  const int np = npairs_s;
  uint16_t* fb = plist + kFuseTok * ZW;  // pairs that need the chain
  {
    const int q = tid >> 4, s16 = tid & 15;
    const int nv = d / 8;  // 16-byte vectors per row
    for (int p = q; p - q < np; p += kFuseWaves * 4) {
      // Four partial sums (exact, so they may be split and regrouped freely)
      // keep the fp64 adds off one dependency chain; loads run 4 vectors
      // ahead of the arithmetic.
      constexpr int AHEAD = 4;
      double acc4[4] = {0.0, 0.0, 0.0, 0.0};
      int emin = 0x7fffffff;
      int tl = 0, e = 0;
      if (p < np) {
        const int v = plist[p];
        tl = v >> 8;
        e = v & 255;
        const u32x4* xr = reinterpret_cast<const u32x4*>(x + (size_t)(t0 + tl) * d);
        const u32x4* wr = reinterpret_cast<const u32x4*>(w + (size_t)e * d);
        u32x4 xa[AHEAD], wa[AHEAD];
#pragma unroll
        for (int u = 0; u < AHEAD; ++u) {
          const int i = s16 + 16 * u;
          xa[u] = i < nv ? xr[i] : u32x4{0u, 0u, 0u, 0u};
          wa[u] = i < nv ? wr[i] : u32x4{0u, 0u, 0u, 0u};
        }
        for (int i0 = s16; i0 < nv; i0 += 16 * AHEAD) {
#pragma unroll
          for (int u = 0; u < AHEAD; ++u) {
            const u32x4 a = xa[u], b = wa[u];
            const int nxt = i0 + 16 * (AHEAD + u);
            if (nxt < nv) {
              xa[u] = xr[nxt];
              wa[u] = wr[nxt];
            }
            if (i0 + 16 * u < nv) {
#pragma unroll
              for (int h = 0; h < 4; ++h) {
                const double p0 =
                    (double)bf16_to_f32(a[h] & 0xffffu) * (double)bf16_to_f32(b[h] & 0xffffu);
                const double p1 = (double)bf16_to_f32(a[h] >> 16) * (double)bf16_to_f32(b[h] >> 16);
                acc4[h] += p0;
                acc4[h] += p1;
                emin = min(emin, min(__builtin_amdgcn_frexp_exp(p0), __builtin_amdgcn_frexp_exp(p1)));
              }
            }
          }
        }
      }
      double acc = (acc4[0] + acc4[1]) + (acc4[2] + acc4[3]);
#pragma unroll
      for (int o = 8; o >= 1; o >>= 1) {
        acc += __shfl_xor(acc, o, 64);
        emin = min(emin, __shfl_xor(emin, o, 64));
      }
      if (p < np && s16 == 0) {
        const double bound = sqrt(sx[tl] * sw[e]) * (1.0 + 0x1p-20);
        if (bound < ldexp(1.0, min(emin, 1000) - 16 + 53)) {
          if (router_bias) acc = acc + (double)router_bias[e];
          zs[tl][e] = __double2float_rn(acc);
        } else {
          fb[atomicAdd(&nfb_s, 1)] = (uint16_t)((tl << 8) | e);
        }
      }
    }
  }
  __syncthreads();
  // The chain itself for the pairs the test did not settle, one wave per pair,
  // walked a segment of `seg` consecutive products at a time.  First every
  // lane forms the data of up to four segments j: T_j, the fp64 sum of the
  // segment's exact products in any order; A_j, an upper bound of the sum of
  // their magnitudes (the fp64 sum of the magnitudes, at most 2^11 terms, so
  // within a factor 1 + 2^-42; padded by 2^-40); m_j, the least frexp
  // exponent of its products minus 16 (each product is a multiple of 2^m_j,
  // a zero product counting as exponent 0 only lowers it).  Then all lanes
  // walk the segments in order with the chain's running value s, a multiple
  // of 2^lowbit_exp(s).  With q = min(m_j, that exponent), if
  // |s| + A_j < 2^(q + 53), every partial sum of the chain inside segment j
  // is a multiple of 2^q below 2^(q + 53) in magnitude, hence representable:
  // the chain does not round there, and it leaves the segment at s + T_j
  // exactly (T_j is then exact as well, by the same bound, and so is the one
  // add).  Otherwise the chain runs element by element through segment j,
  // each product broadcast from its lane: the definition's rounded adds in
  // its order.  Segments hold 64 products up to d = 16384 (at most 256
  // segments, four per lane).
  const int nfb = nfb_s;
  {
    const int seg = 64 * ((d + 64 * 256 - 1) / (64 * 256));
    const int nseg = (d + seg - 1) / seg;
    for (int p = wave; p < nfb; p += kFuseWaves) {
      const int v = fb[p];
      const int tl = v >> 8, e = v & 255;
      const bf16_t* xr = x + (size_t)(t0 + tl) * d;
      const bf16_t* wr = w + (size_t)e * d;
      double T[4], A[4];
      int M[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        T[u] = 0.0;
        A[u] = 0.0;
        M[u] = 0x7fffffff;
        const int j = lane + 64 * u;
        if (j < nseg) {
          const int i1 = min(d, (j + 1) * seg);
          for (int i = j * seg; i < i1; i += 8) {  // d % 32 == 0: whole 8-element pieces
            const u32x4 a = *reinterpret_cast<const u32x4*>(xr + i);
            const u32x4 b = *reinterpret_cast<const u32x4*>(wr + i);
#pragma unroll
            for (int h = 0; h < 4; ++h) {
              const double p0 =
                  (double)bf16_to_f32(a[h] & 0xffffu) * (double)bf16_to_f32(b[h] & 0xffffu);
              const double p1 = (double)bf16_to_f32(a[h] >> 16) * (double)bf16_to_f32(b[h] >> 16);
              T[u] += p0;
              T[u] += p1;
              A[u] += fabs(p0);
              A[u] += fabs(p1);
              M[u] = min(M[u], min(__builtin_amdgcn_frexp_exp(p0), __builtin_amdgcn_frexp_exp(p1)));
            }
          }
          A[u] *= 1.0 + 0x1p-40;
        }
      }
      double acc = 0.0;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        for (int ln = 0; ln < 64 && 64 * u + ln < nseg; ++ln) {
          const double tj = bcast_lane(T[u], ln), aj = bcast_lane(A[u], ln);
          int q = __builtin_amdgcn_readlane(M[u], ln) - 16;
          if (acc != 0.0) q = min(q, lowbit_exp(acc));
          // |s| + A_j rounded up (the fp64 add loses at most 2^-53 of it).
          const double lhs = (fabs(acc) + aj) * (1.0 + 0x1p-50);
          if (lhs < ldexp(1.0, min(q + 53, 1023))) {
            acc = acc + tj;
          } else {
            const int j = 64 * u + ln;
            const int i1 = min(d, (j + 1) * seg);
            for (int b0 = j * seg; b0 < i1; b0 += 64) {
              const int i = b0 + lane;
              double pv = 0.0;
              if (i < i1) pv = (double)bf16_to_f32(xr[i]) * (double)bf16_to_f32(wr[i]);
              const int n = min(64, i1 - b0);
              for (int r = 0; r < n; ++r) acc = acc + bcast_lane(pv, r);
            }
          }
        }
      }
      if (lane == 0) {
        if (router_bias) acc = acc + (double)router_bias[e];
        zs[tl][e] = __double2float_rn(acc);
      }
    }
  }
  __syncthreads();

  // ---- 4. finalize ------------------------------------------------------
  for (int tl = wave; tl < nt; tl += kFuseWaves) {
    const int t = t0 + tl;
    float z[NJ], s[NJ];
    bool is_c[NJ];
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int e = lane + 64 * j;
      const bool okj = e < E;
      z[j] = okj ? zs[tl][e] : 0.f;
      is_c[j] = okj && ((cand_s[tl][j] >> lane) & 1ull);
      s[j] = is_c[j] ? sel_score(z[j], score_fn, sb[j]) : -INFINITY;
    }
    uint64_t kept = ~0ull;
    if (G > 1) {
      const uint64_t kept_c = gm_s[tl][0], undecided = gm_s[tl][1];
      kept = kept_c;
      const int need = kg - __popcll(kept_c);
      if (need > 0 && undecided) {
        // Exact maxima of undecided groups (all their possible maxima are
        // candidates, so the maximum over candidates is the group score).
#pragma unroll
        for (int j = 0; j < NJ; ++j)
          if (lane + 64 * j < E) wsc[wave][lane + 64 * j] = s[j];
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
        __builtin_amdgcn_wave_barrier();
        float gs = 0.f;
        int gi = -1;
        if (lane < G && ((undecided >> lane) & 1ull)) {
          float m = -INFINITY;
          for (int e = lane * per; e < (lane + 1) * per; ++e) m = fmaxf(m, wsc[wave][e]);
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
    bool elig[NJ];
#pragma unroll
    for (int j = 0; j < NJ; ++j) elig[j] = is_c[j] && ((kept >> ((lane + 64 * j) / per)) & 1ull);

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
        for (int j = 1; j < NJ; ++j)
          if (jj == j) zv = z[j];
        zsel[r] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(zv), owner));
        if (lane == owner) {
#pragma unroll
          for (int j = 0; j < NJ; ++j)
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
      for (int j = 0; j < NJ; ++j)
        if (lane + 64 * j < E) m = fmaxf(m, z[j]);
      const double zmax = (double)wave_max(m);
      double part = 0.0;
#pragma unroll
      for (int j = 0; j < NJ; ++j)
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
  // The tile's logits (exact for candidates, z~ elsewhere) and counts.
  for (int i = tid; i < nt * E; i += kFuseWaves * 64) logits[(size_t)t0 * E + i] = zs[i / E][i % E];
}

// NJ = ceil(E / 64) expert slots per lane in steps 2 and 4.  SPLIT 0 runs
// every step; with several expert tiles the work is split in two launches so
// that the expert tiles of step 1 run in parallel: SPLIT 1 is step 1 for one
// expert tile (blockIdx.y) per block, writing z~ to `logits` and the squared
// norms to ws_sx / ws_sw; SPLIT 2 reads them back and runs steps 2-4.
template <int NJ, int SPLIT>
__global__ __launch_bounds__(kFuseWaves * 64, 4) void route_fused(
    const bf16_t* __restrict__ x, const bf16_t* __restrict__ w, int N, int d, int E, int k,
    int G, int kg, int score_fn, const float* __restrict__ router_bias,
    const float* __restrict__ sel_bias, float* __restrict__ logits,
    int32_t* __restrict__ topk_idx, float* __restrict__ topk_w, int32_t* __restrict__ counts,
    double* __restrict__ ws_sx, double* __restrict__ ws_sw, double* __restrict__ ws_part,
    int ksplit, int tail_tpb) {
  constexpr int ZW = 64 * NJ;
  // Pair slots of step 1 (the tail launch runs no step 1: its ring is scratch).
  constexpr int RINGP = SPLIT == 1 ? kScorePairs : kFusePairs;
  constexpr int NSLOT = SPLIT == 2 ? kFuseRing / 2 : RINGP;
  // The block's LDS is one object, carved at fixed offsets: the ring first
  // (1-KB aligned), then the 8-byte and the 4-byte arrays.  With several LDS
  // objects the compiler tags each with its own alias scope, and before every
  // read of the ring it then waits for all of the ring's direct-to-LDS loads,
  // the refills just issued included (s_waitcnt vmcnt(0)), so no load
  // overlapped the arithmetic.  As one object the reads are ordered only by
  // the ring's own waits and barriers (each wave waits for its loads of the
  // pairs it is about to read, then the barrier), as in the grouped GEMM.
  // The scoring launch (SPLIT == 1) uses the ring alone.
  constexpr bool TAIL = SPLIT != 1;
  constexpr int kRingB = NSLOT * 2 * kFuseSlot;
  constexpr int kSxO = kRingB, kSwO = kSxO + (TAIL ? kFuseTok * 8 : 0);
  constexpr int kCandO = kSwO + (TAIL ? ZW * 8 : 0);
  constexpr int kGmO = kCandO + (TAIL ? kFuseTok * 4 * 8 : 0);
  constexpr int kZsO = kGmO + (TAIL ? kFuseTok * 2 * 8 : 0);
  constexpr int kCntO = kZsO + (TAIL ? kFuseTok * ZW * 4 : 0);
  constexpr int kHistO = kCntO + (TAIL ? kFuseTok * 4 : 0);
  constexpr int kNpO = kHistO + (TAIL ? ZW * 4 : 0);
  constexpr int kLdsB = kNpO + (TAIL ? 8 : 0);
  __shared__ __attribute__((aligned(1024))) char lds[kLdsB];
  auto& ring = *reinterpret_cast<char (*)[NSLOT][2 * kFuseSlot]>(lds);  // step 1; then pairs
  auto& zs = *reinterpret_cast<float (*)[kFuseTok][ZW]>(lds + kZsO);  // z~, then exact values
  auto& sx = *reinterpret_cast<double (*)[kFuseTok]>(lds + kSxO);
  auto& sw = *reinterpret_cast<double (*)[ZW]>(lds + kSwO);
  auto& cand_s = *reinterpret_cast<uint64_t (*)[kFuseTok][4]>(lds + kCandO);
  auto& gm_s = *reinterpret_cast<uint64_t (*)[kFuseTok][2]>(lds + kGmO);
  auto& cnt_s = *reinterpret_cast<int32_t (*)[kFuseTok]>(lds + kCntO);
  auto& hist = *reinterpret_cast<int32_t (*)[ZW]>(lds + kHistO);
  int32_t& npairs_s = *reinterpret_cast<int32_t*>(lds + kNpO);
  int32_t& nfb_s = *reinterpret_cast<int32_t*>(lds + kNpO + 4);
  // After step 1 the ring holds, at different times, the per-wave scratch of
  // the group limit (steps 2 and 4) and the pair lists (end of 2, step 3).
  static_assert(2 * kFuseTok * ZW * 2 <= kFuseRing * kFuseSlot,
                "pair list and fallback list fit the ring");
  static_assert(2 * kFuseWaves * ZW * 4 + kFuseWaves * 512 <= kFuseRing * kFuseSlot,
                "group-limit scratch fits the ring");
  static_assert(kFuseTok <= 64 && ZW <= 256, "pair encoding and one-wave token scan");

  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // The tail launch takes tail_tpb (1..16) tokens per block, so that the few
  // token tiles of a split launch still cover every CU.
  const int TPB = SPLIT == 2 ? tail_tpb : kFuseTok;
  const int t0 = blockIdx.x * TPB;
  const int nt = min(TPB, N - t0);
  // Chunks of 32 elements this block sums.  A K-split scoring launch
  // (ksplit > 1, grid.z = split) gives split z the even-aligned chunk range
  // [c0, c0 + nch); its fp64 partial sums go to ws_part.
  int c0 = 0, nch = d / 32;
  if (SPLIT == 1 && ksplit > 1) {
    const int z = blockIdx.z, pairs = nch / 2;
    c0 = 2 * (pairs * z / ksplit);
    const int c1 = z + 1 == ksplit ? nch : 2 * (pairs * (z + 1) / ksplit);
    nch = c1 - c0;
  }
  if constexpr (TAIL)
    for (int e = tid; e < E; e += kFuseWaves * 64) hist[e] = 0;
  // The scoring launch of the split route clears the counts its tail launch
  // adds to (stream order runs the whole tail after it).
  if (SPLIT == 1 && blockIdx.x == 0 && blockIdx.y == 0 && blockIdx.z == 0)
    for (int e = tid; e < E; e += kFuseWaves * 64) counts[e] = 0;

  // ---- 1. scores --------------------------------------------------------
  // The ring holds pairs of chunks (64 elements) as 128-byte row pieces: 12
  // loads of 1 KB per pair, j < 4 the x rows 8j.. of the token block, j >= 4
  // the w rows 8(j - 4).. of the expert tile; wave w issues load w, and waves
  // 0-3 also load w + 8.  Lane L fetches row 8j' + L/8 of its load, logical
  // 16-byte chunk (L % 8) ^ swz8(row % 16), into physical chunk L % 8.  The
  // loads are buffer loads over the block's own x rows and expert rows, so the
  // second chunk of a last pair past the row end (d an odd number of chunks)
  // reads zeros instead of past the buffers; every offset that varies sits in
  // the per-lane offset, which the range check covers.
  const int nx = min(kFuseTok, N - t0);  // token rows the block may read
  const int nl = wave < 4 ? 2 : 1;       // loads per pair of this wave
  // Squared norms from the diagonal of X X^T and W W^T, one extra MFMA per
  // chunk on the operands already in registers (waves 0 and 4 for the two
  // token blocks, waves 0-3 for the expert blocks).  In the 16x16 output lane
  // l holds rows 4(l/16) + v of column l % 16, so the diagonal element of row
  // i = l % 16 is in lanes with l / 16 = i / 4, at v = i % 4.
  const bool diag_lane = (lane >> 4) == ((lane & 15) >> 2);
  const int diag_v = lane & 3;
  double sxp = 0.0;  // waves 0 and 4, diagonal lanes: sum x^2 of token 16(wave/4) + lane%16
  floatx4 sq32x = floatx4{0.f, 0.f, 0.f, 0.f};
  const int et_begin = SPLIT == 1 ? 64 * (int)blockIdx.y : 0;
  const int et_end = SPLIT == 1 ? et_begin + 64 : (SPLIT == 2 ? 0 : E);
  const int npair = (nch + 1) / 2;
  for (int et = et_begin; et < et_end; et += 64) {
    const int ne = min(64, E - et);
    const auto rs_x = buffer_rsrc(x + (size_t)t0 * d, (uint32_t)nx * (uint32_t)d * 2u);
    const auto rs_w = buffer_rsrc(w + (size_t)et * d, (uint32_t)ne * (uint32_t)d * 2u);
    // Per-lane byte offsets of this wave's loads at pair 0 of the range.
    uint32_t vo[2];
    bool isx[2];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int j = wave + 8 * q;
      const int jj = j < 4 ? j : j - 4;
      const int r = 8 * jj + lane / 8;
      isx[q] = j < 4;
      const int rr = isx[q] ? min(r, nx - 1) : min(r, ne - 1);  // past the end: fetched, unused
      vo[q] = (uint32_t)rr * (uint32_t)d * 2u + (uint32_t)(((lane & 7) ^ swz8(r & 15)) * 16) +
              (uint32_t)c0 * 64u;
    }
#define MOE_FUSE_ISSUE(pr_)                                                                  \
  do {                                                                                       \
    char* slot_ = ring[(pr_) % RINGP];                                                       \
    const uint32_t po_ = (uint32_t)(pr_) * 128u;                                             \
    _Pragma("unroll") for (int q = 0; q < 2; ++q) if (q < nl) {                              \
      const int j = wave + 8 * q;                                                            \
      buffer_load_lds16<0>(isx[q] ? rs_x : rs_w, slot_ + j * 1024, vo[q] + po_, 0u);         \
    }                                                                                        \
  } while (0)
    // Pairs are consumed two per step: one wait and one barrier per two pairs.
    // The prologue issues RINGP - 2 pairs; each step refills the two slots the
    // previous step used.
    static_assert(RINGP >= 4 && 2 * (RINGP - 4) <= 7, "two slots refilled per step");
    for (int c = 0; c < RINGP - 2 && c < npair; ++c) MOE_FUSE_ISSUE(c);
    double swp = 0.0;  // waves 0-3, diagonal lanes: sum w^2 of expert 16 wave + lane%16
    // fp32 sums of the chunks of a step: chunks 0 and 2 go to the first of
    // each pair of accumulators, 1 and 3 to the second (at most 64 products
    // per fp32 sum, and two independent MFMA chains).
    floatx4 sq32w[2] = {floatx4{0.f, 0.f, 0.f, 0.f}, floatx4{0.f, 0.f, 0.f, 0.f}};
    floatx4 sq32x[2] = {floatx4{0.f, 0.f, 0.f, 0.f}, floatx4{0.f, 0.f, 0.f, 0.f}};
    floatx4 acc32[2] = {floatx4{0.f, 0.f, 0.f, 0.f}, floatx4{0.f, 0.f, 0.f, 0.f}};
    double acc[4] = {0.0, 0.0, 0.0, 0.0};
#define MOE_FUSE_CHUNK(pr_, c_, A_)                                                         \
  do {                                                                                      \
    const char* slot = ring[(pr_) % RINGP];                                                 \
    /* MFMA: wave w takes token block w/4 (A = tokens 16(w/4) + (lane & 15)) */            \
    /* and expert block w%4 of the tile (B). */                                             \
    {                                                                                       \
      const int lc = 4 * (c_) + (lane >> 4), r16 = lane & 15;                               \
      const int er = 16 * (wave % 4) + r16, tr = 16 * (wave / 4) + r16;                     \
      const bf16x8_t bw = *reinterpret_cast<const bf16x8_t*>(                               \
          slot + 4096 + er * 128 + ((lc ^ swz8(r16)) << 4));                                \
      const bf16x8_t ax = *reinterpret_cast<const bf16x8_t*>(                               \
          slot + tr * 128 + ((lc ^ swz8(r16)) << 4));                                       \
      acc32[A_] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ax, bw, acc32[A_], 0, 0, 0);      \
      if (wave < 4)                                                                          \
        sq32w[A_] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bw, bw, sq32w[A_], 0, 0, 0);    \
      if (et == 0 && (wave & 3) == 0)                                                        \
        sq32x[A_] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ax, ax, sq32x[A_], 0, 0, 0);    \
    }                                                                                       \
  } while (0)
    // A step's fp32 sums of at most 64 exact products each, summed in fp64;
    // its fp32 sums of at most 64 exact squares as upper bounds in fp64: the
    // rounded sum is at least (1 - 2^-18) of the exact one, and squares below
    // 2^-126 that the MFMA may flush add at most 64 * 2^-126.
#define MOE_FUSE_FOLD()                                                                     \
  do {                                                                                      \
    _Pragma("unroll") for (int a_ = 0; a_ < 2; ++a_) {                                      \
      _Pragma("unroll") for (int v = 0; v < 4; ++v) acc[v] += (double)acc32[a_][v];         \
      acc32[a_] = floatx4{0.f, 0.f, 0.f, 0.f};                                              \
      if (wave < 4) {                                                                       \
        const floatx4 s_ = sq32w[a_];                                                       \
        const float q = diag_v == 0 ? s_[0] : diag_v == 1 ? s_[1] : diag_v == 2 ? s_[2] : s_[3]; \
        if (diag_lane) swp += (double)q * (1.0 + 0x1p-17) + 0x1p-120;                       \
        sq32w[a_] = floatx4{0.f, 0.f, 0.f, 0.f};                                            \
      }                                                                                     \
      if (et == 0 && (wave & 3) == 0) {                                                     \
        const floatx4 s_ = sq32x[a_];                                                       \
        const float q = diag_v == 0 ? s_[0] : diag_v == 1 ? s_[1] : diag_v == 2 ? s_[2] : s_[3]; \
        if (diag_lane) sxp += (double)q * (1.0 + 0x1p-17) + 0x1p-120;                       \
        sq32x[a_] = floatx4{0.f, 0.f, 0.f, 0.f};                                            \
      }                                                                                     \
    }                                                                                       \
  } while (0)
    // Steady state: both refills of the step are in range, so the wait count
    // is a constant and the loop body has no branches besides the wave role.
    int pr = 0;
    for (; pr + RINGP - 1 < npair; pr += 2) {
      // Pairs pr and pr + 1 have landed once at most RINGP - 4 younger pairs
      // of this wave's loads are in flight.
      if (nl == 2) wait_vmcnt<2 * (RINGP - 4)>(); else wait_vmcnt<RINGP - 4>();
      // The pairs are visible to all waves; all waves are done with the
      // previous step's pairs, whose slots are refilled now.
      ring_barrier();
      MOE_FUSE_ISSUE(pr + RINGP - 2);
      MOE_FUSE_ISSUE(pr + RINGP - 1);
      MOE_FUSE_CHUNK(pr, 0, 0);
      MOE_FUSE_CHUNK(pr, 1, 1);
      MOE_FUSE_CHUNK(pr + 1, 0, 0);
      MOE_FUSE_CHUNK(pr + 1, 1, 1);
      MOE_FUSE_FOLD();
    }
    // The last steps: fewer younger pairs in flight, refills only in range;
    // the last step may hold one pair, and the range's last pair one chunk.
    for (; pr < npair; pr += 2) {
      const bool two = pr + 1 < npair;
      const int later = min(npair - 1, pr + RINGP - 3) - (two ? pr + 1 : pr);
      if (nl == 2) wait_stages<2>(later); else wait_stages<1>(later);
      ring_barrier();
      if (pr + RINGP - 2 < npair) MOE_FUSE_ISSUE(pr + RINGP - 2);
      if (pr + RINGP - 1 < npair) MOE_FUSE_ISSUE(pr + RINGP - 1);
      MOE_FUSE_CHUNK(pr, 0, 0);
      if (2 * pr + 1 < nch) MOE_FUSE_CHUNK(pr, 1, 1);
      if (two) {
        MOE_FUSE_CHUNK(pr + 1, 0, 0);
        if (2 * pr + 3 < nch) MOE_FUSE_CHUNK(pr + 1, 1, 1);
      }
      MOE_FUSE_FOLD();
    }
#undef MOE_FUSE_CHUNK
#undef MOE_FUSE_FOLD
#undef MOE_FUSE_ISSUE
    // z~: lane holds expert (lane & 15) of block w%4, tokens 16(w/4) + 4*(lane>>4)+v.
    const int e = et + 16 * (wave % 4) + (lane & 15);
    if (e < E) {
      const double bias = router_bias ? (double)router_bias[e] : 0.0;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int tl = 16 * (wave / 4) + 4 * (lane >> 4) + v;
        if constexpr (SPLIT == 1) {
          if (tl < nt) {
            if (ksplit > 1)
              ws_part[((size_t)blockIdx.z * N + t0 + tl) * E + e] = acc[v];
            else
              logits[(size_t)(t0 + tl) * E + e] = (float)(acc[v] + bias);
          }
        } else {
          zs[tl][e] = (float)(acc[v] + bias);
        }
      }
    }
    // sum w^2: from the diagonal lanes of waves 0-3.
    if (wave < 4 && diag_lane && et + 16 * wave + (lane & 15) < E) {
      if constexpr (SPLIT == 1) {
        if (blockIdx.x == 0) ws_sw[(size_t)blockIdx.z * E + et + 16 * wave + (lane & 15)] = swp;
      } else {
        sw[et + 16 * wave + (lane & 15)] = swp;
      }
    }
    __syncthreads();  // ring slots are reused by the next expert tile
  }
  if constexpr (SPLIT == 1) {
    const int tl = 16 * (wave >> 2) + (lane & 15);
    if (blockIdx.y == 0 && (wave & 3) == 0 && diag_lane && tl < nt)
      ws_sx[(size_t)blockIdx.z * N + t0 + tl] = sxp;
  } else {
  if constexpr (SPLIT == 2) {
    // The tile's z~ and norms from the scoring launch; after a K split, the
    // sum of the splits' fp64 partials in split order (each partial obeys the
    // chunk bound, and the few fp64 additions are far inside the margin's
    // slack), plus the bias, rounded once.  Sums of the partial squared-norm
    // bounds are bounds.
    if (ksplit > 1) {
      for (int i = tid; i < nt * E; i += kFuseWaves * 64) {
        const int e = i % E;
        double z = 0.0;
        for (int q = 0; q < ksplit; ++q) z += ws_part[((size_t)q * N + t0) * E + i];
        zs[i / E][e] = (float)(z + (router_bias ? (double)router_bias[e] : 0.0));
      }
      for (int tl = tid; tl < nt; tl += kFuseWaves * 64) {
        double q2 = 0.0;
        for (int q = 0; q < ksplit; ++q) q2 += ws_sx[(size_t)q * N + t0 + tl];
        sx[tl] = q2;
      }
      for (int e = tid; e < E; e += kFuseWaves * 64) {
        double q2 = 0.0;
        for (int q = 0; q < ksplit; ++q) q2 += ws_sw[(size_t)q * E + e];
        sw[e] = q2;
      }
    } else {
      for (int i = tid; i < nt * E; i += kFuseWaves * 64)
        zs[i / E][i % E] = logits[(size_t)t0 * E + i];
      for (int tl = tid; tl < nt; tl += kFuseWaves * 64) sx[tl] = ws_sx[t0 + tl];
      for (int e = tid; e < E; e += kFuseWaves * 64) sw[e] = ws_sw[e];
    }
  } else {
    if ((wave & 3) == 0 && diag_lane) sx[16 * (wave >> 2) + (lane & 15)] = sxp;
  }
  __syncthreads();

  route_tile_tail<NJ, ZW>(x, w, d, E, k, G, kg, score_fn, router_bias, sel_bias, logits,
                                 topk_idx, topk_w, t0, nt, zs, &ring[0][0], sx, sw, cand_s, gm_s,
                                 cnt_s, hist, npairs_s, nfb_s);
  __syncthreads();
  for (int e = tid; e < E; e += kFuseWaves * 64)
    if (hist[e]) atomicAdd(&counts[e], hist[e]);
  }
}

// ---------------------------------------------------------------- launch ---

// Split launches (see route_fused) whenever there are several expert tiles
// (measured: Zipf-like 32768 tokens x 128 experts 210 -> 178 us; with one
// expert tile the extra launch costs more than it gains, 42 -> 55 us).
static bool route_split(int N, int E) {
  (void)N;
  return E > 64;
}

// K splits of the scoring launch: when its token tiles x expert tiles give
// fewer blocks than CUs (decode-sized batches), each block sums 1/ks of the
// hidden dimension, up to 8 ways and at least one chunk pair each.
static int route_ksplit(int N, int d, int E) {
  if (!route_split(N, E)) return 1;
  const int base = ((N + kFuseTok - 1) / kFuseTok) * ((E + 63) / 64);
  if (base >= 256) return 1;
  return std::max(1, std::min(std::min(8, 256 / std::max(base, 1)), d / 64));
}

size_t route_certified_workspace_bytes(int N, int d, int E) {
  // The fused kernel keeps everything in LDS; the split one passes the
  // squared norms (per K split) and, when K is split, the fp64 partial
  // logits between its two launches.
  if (!route_split(N, E)) return 0;
  const size_t ks = route_ksplit(N, d, E);
  return ks * (size_t)(N + E) * sizeof(double) +
         (ks > 1 ? ks * (size_t)N * E * sizeof(double) : 0);
}

hipError_t launch_route_certified(const RouteArgs& a, hipStream_t st) {
  const int blocks = (a.N + kFuseTok - 1) / kFuseTok;
  const bool split = route_split(a.N, a.E);
  // The counts start at zero: the split route's scoring launch clears them
  // (its tail launch adds), the one-launch route needs a launch before it.
  if (!split) launch_zero_i32(a.counts, a.E, st);
  const int ks = route_ksplit(a.N, a.d, a.E);
  double* ws_sx = split ? static_cast<double*>(a.ws) : nullptr;
  double* ws_sw = split ? ws_sx + (size_t)ks * a.N : nullptr;
  double* ws_part = ks > 1 ? ws_sw + (size_t)ks * a.E : nullptr;
  // Tail blocks take 16 tokens while that still gives about two blocks per
  // CU (two fit: 128 VGPRs, 75 KB of LDS), fewer for smaller batches: the
  // phases of a block (certify, exact sums, selection) run one after another,
  // so a second block on the CU fills the first one's waits, and the exact
  // sums of a block's candidate pairs stream each pair's x and w rows from
  // L2, which 16 tokens per block would put on N/16 CUs (decode-sized
  // batches).  DeepSeek-like layer (4096 tokens): 8 tokens, 227 -> 206 us.
  const int tail_tpb = std::min(kFuseTok / 2, std::max(1, (a.N + 511) / 512));
  auto launch = [&](auto kernel, dim3 grid) {
    kernel<<<grid, kFuseWaves * 64, 0, st>>>(
        static_cast<const bf16_t*>(a.x), static_cast<const bf16_t*>(a.w_router), a.N, a.d, a.E,
        a.k, a.G, a.kg, a.score_fn, a.router_bias, a.sel_bias, a.logits, a.topk_idx, a.topk_w,
        a.counts, ws_sx, ws_sw, ws_part, ks, tail_tpb);
  };
  const dim3 scores_grid(blocks, (a.E + 63) / 64, ks);
  const dim3 tail_grid((a.N + tail_tpb - 1) / tail_tpb);
  switch ((a.E + 63) / 64) {
    case 1: launch(route_fused<1, 0>, dim3(blocks)); break;
    case 2:
      if (split) {
        launch(route_fused<2, 1>, scores_grid);
        launch(route_fused<2, 2>, tail_grid);
      } else {
        launch(route_fused<2, 0>, dim3(blocks));
      }
      break;
    case 3:
      if (split) {
        launch(route_fused<3, 1>, scores_grid);
        launch(route_fused<3, 2>, tail_grid);
      } else {
        launch(route_fused<3, 0>, dim3(blocks));
      }
      break;
    default:
      if (split) {
        launch(route_fused<4, 1>, scores_grid);
        launch(route_fused<4, 2>, tail_grid);
      } else {
        launch(route_fused<4, 0>, dim3(blocks));
      }
      break;
  }
  return hipGetLastError();
}

}  // namespace moe
