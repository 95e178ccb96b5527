// dispatch.hip -- capacity, admission (token order, or first choice first)
// and the expert/rank-contiguous send-buffer layout, for gfx950.
//
// Glossary "Expert Parallelism": step 2 of "How tokens travel between GPUs"
// (each token's hidden state goes to the rank holding its experts; experts sit
// on ranks in blocks, e / (E/R), as in the routing snippet) and the capacity
// bullet of "Load balancing and capacity" (an expert takes at most cap
// assignments per batch, the rest skip it).  Admission is in token order, so
// the rank of slot (t, j) inside expert e is the number of earlier slots (in
// t-major, j-minor order) that chose e -- a stable counting sort.  On request
// the walk is first choice first (MLSys ch.10, section 10.5: GShard's top-2
// router): j-major, t-minor, the same counting sort over that order.
//
// Kernels (over the N*k positions of the admission walk, in tiles of 1024):
//  count       one block: per-tile, per-expert histogram in LDS and the scan
//              below, when tiles * E fits in LDS (else tile_hist + scan).
//  tile_hist   per-tile, per-expert histogram (LDS atomics).
//  scan        one block: per expert, exclusive prefix of the tile histograms
//              (in place), admitted = min(count, cap), exclusive scan over
//              experts -> expert offsets, rank offsets and counts.
//  assign      per tile: per-wave histograms and their prefix give each wave
//              its base; inside a wave, slots of one 64-slot chunk that chose
//              the same expert are found with one ballot per expert-id bit,
//              and a slot's rank is the popcount of the matching lanes below
//              it.  Writes row_of_slot / token_of_row / slot_of_row.
//  permute     token-major copy: one wave reads x[t] once (16-byte vectors)
//              and writes it to each of its admitted rows.
#include "device.h"
#include "kernels.h"

namespace moe {

constexpr int kTileSlots = 1024;  // 4 waves x 4 chunks x 64 slots

// The admission walk: position q of the walk visits slot walk_slot(q).  Token
// order visits slots in storage order (t-major, j-minor); first choice first
// visits slot j of every token, in token order, before slot j + 1 of any
// (q = j N + t).  Tiles, histograms and ranks are all taken over q, so a
// slot's rank inside its expert is the number of earlier positions of the
// walk that chose the same expert, whichever walk it is.
__device__ __forceinline__ int walk_slot(int q, int N, int k, int first_choice) {
  if (!first_choice) return q;
  const int j = q / N;
  return (q - j * N) * k + j;
}

__global__ __launch_bounds__(256) void dispatch_tile_hist(const int32_t* __restrict__ topk_idx,
                                                          int S, int k, int E, int first_choice,
                                                          int32_t* __restrict__ tile_counts) {
  __shared__ int32_t hist[256];
  for (int e = threadIdx.x; e < E; e += 256) hist[e] = 0;
  __syncthreads();
  const int s0 = blockIdx.x * kTileSlots;
  const int s1 = min(S, s0 + kTileSlots);
  const int N = S / k;
  for (int q = s0 + threadIdx.x; q < s1; q += 256) {
    const int e = topk_idx[walk_slot(q, N, k, first_choice)];
    if ((unsigned)e < (unsigned)E) atomicAdd(&hist[e], 1);  // ids out of range are ignored
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += 256)
    tile_counts[(size_t)blockIdx.x * E + e] = hist[e];
}

// One block of 256 threads; thread e owns expert e.
__global__ __launch_bounds__(256) void dispatch_scan(int32_t* __restrict__ tile_counts,
                                                     int num_tiles, int E, int R, int32_t cap,
                                                     int padded,
                                                     int32_t* __restrict__ expert_offsets,
                                                     int32_t* __restrict__ admitted,
                                                     int32_t* __restrict__ rank_offsets,
                                                     int32_t* __restrict__ rank_counts) {
  __shared__ int32_t scan[256];
  __shared__ int32_t offs[257];
  const int e = threadIdx.x;
  int32_t run = 0;
  if (e < E) {
    for (int t = 0; t < num_tiles; ++t) {
      const size_t q = (size_t)t * E + e;
      const int32_t c = tile_counts[q];
      tile_counts[q] = run;  // becomes the tile's base rank for expert e
      run += c;
    }
  }
  const int32_t adm = e < E ? min(run, cap) : 0;
  if (e < E) admitted[e] = adm;
  // Block-wide exclusive scan of adm (Hillis-Steele in LDS; 256 entries).
  scan[e] = adm;
  __syncthreads();
  for (int o = 1; o < 256; o <<= 1) {
    const int32_t v = e >= o ? scan[e - o] : 0;
    __syncthreads();
    scan[e] += v;
    __syncthreads();
  }
  // Padded layout: expert e owns rows [e cap, (e+1) cap) whatever it admits.
  const int32_t excl = padded ? e * cap : scan[e] - adm;
  const int32_t total = padded ? E * cap : scan[e];
  if (e < E) {
    expert_offsets[e] = excl;
    offs[e] = excl;
  }
  if (e == E - 1) {
    expert_offsets[E] = total;
    offs[E] = total;
  }
  __syncthreads();
  const int per = E / R;
  for (int r = threadIdx.x; r <= R; r += 256) rank_offsets[r] = offs[r * per];
  for (int r = threadIdx.x; r < R; r += 256) rank_counts[r] = offs[(r + 1) * per] - offs[r * per];
}

// Histogram and scan in one block of 1024 threads, for batches whose per-tile
// histograms fit in LDS (tiles * E <= kCountLds): the per-tile, per-expert
// counts are taken with LDS atomics over every slot, then thread e turns
// expert e's column into exclusive tile bases (written for dispatch_assign)
// and the same per-expert / per-rank offsets as dispatch_scan follow.
constexpr int kCountLds = 16384;  // ints

__global__ __launch_bounds__(1024) void dispatch_count(const int32_t* __restrict__ topk_idx,
                                                       int S, int k, int first_choice,
                                                       int num_tiles, int E, int R,
                                                       int32_t cap, int padded,
                                                       int32_t* __restrict__ tile_base,
                                                       int32_t* __restrict__ expert_offsets,
                                                       int32_t* __restrict__ admitted,
                                                       int32_t* __restrict__ rank_offsets,
                                                       int32_t* __restrict__ rank_counts) {
  __shared__ int32_t h[kCountLds];
  __shared__ int32_t scan[16];  // wave totals of the expert scan
  __shared__ int32_t offs[1025];
  const int tid = threadIdx.x;
  const int cells = num_tiles * E;
  for (int q = tid; q < cells; q += 1024) h[q] = 0;
  __syncthreads();
  // Eight loads in flight per thread before their atomics (a block-strided
  // loop would wait for each load in turn).  s is the position in the walk.
  const int N = S / k;
  for (int s0 = 0; s0 < S; s0 += 8 * 1024) {
    int ids[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int s = s0 + u * 1024 + tid;
      ids[u] = s < S ? topk_idx[walk_slot(s, N, k, first_choice)] : -1;
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int s = s0 + u * 1024 + tid;
      if ((unsigned)ids[u] < (unsigned)E)  // ids out of range are ignored
        atomicAdd(&h[(s / kTileSlots) * E + ids[u]], 1);
    }
  }
  __syncthreads();
  int32_t run = 0;
  if (tid < E) {
    for (int t = 0; t < num_tiles; ++t) {
      const int32_t c = h[t * E + tid];
      tile_base[(size_t)t * E + tid] = run;
      run += c;
    }
  }
  const int32_t adm = tid < E ? min(run, cap) : 0;
  if (tid < E) admitted[tid] = adm;
  // Exclusive scan of adm over experts: inclusive scan inside each wave,
  // then the wave totals (E <= 1024: at most 16 waves).
  const int lane = tid & 63, wv = tid >> 6;
  int32_t incl = adm;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int32_t v = __shfl_up(incl, o, 64);
    if (lane >= o) incl += v;
  }
  if (lane == 63) scan[wv] = incl;
  __syncthreads();
  for (int w = 0; w < wv; ++w) incl += scan[w];
  // Padded layout: expert e owns rows [e cap, (e+1) cap) whatever it admits.
  const int32_t excl = padded ? tid * cap : incl - adm;
  if (padded) incl = E * cap;
  if (tid < E) {
    expert_offsets[tid] = excl;
    offs[tid] = excl;
  }
  if (tid == E - 1) {
    expert_offsets[E] = incl;
    offs[E] = incl;
  }
  __syncthreads();
  const int per = E / R;
  for (int r = tid; r <= R; r += 1024) rank_offsets[r] = offs[r * per];
  for (int r = tid; r < R; r += 1024) rank_counts[r] = offs[(r + 1) * per] - offs[r * per];
}

__device__ __forceinline__ uint64_t lanemask_lt(int lane) {
  return lane == 0 ? 0ull : (~0ull >> (64 - lane));
}

__global__ __launch_bounds__(256) void dispatch_assign(
    const int32_t* __restrict__ topk_idx, int S, int k, int first_choice, int E, int32_t cap,
    const int32_t* __restrict__ tile_base, const int32_t* __restrict__ expert_offsets,
    int32_t* __restrict__ row_of_slot, int32_t* __restrict__ token_of_row,
    int8_t* __restrict__ slot_of_row) {
  __shared__ int32_t wcount[4][256];  // per-wave histogram, then per-wave running rank
  __shared__ int32_t eoff[257];
  const int wave = threadIdx.x / 64, lane = threadIdx.x % 64;
  const int s0 = blockIdx.x * kTileSlots;

  // The tile's base ranks are loaded now, with the ids below, rather than
  // after the per-wave counts.
  // Descriptors allow at most 256 experts: thread e owns expert e.
  const int32_t base = threadIdx.x < E ? tile_base[(size_t)blockIdx.x * E + threadIdx.x] : 0;
  for (int q = threadIdx.x; q < 4 * 256; q += 256) (&wcount[0][0])[q] = 0;
  for (int e = threadIdx.x; e <= E; e += 256) eoff[e] = expert_offsets[e];
  __syncthreads();

  const int ws0 = s0 + wave * 256;  // this wave's 256 positions of the walk
  const int N = S / k;
  int my_e[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int q = ws0 + c * 64 + lane;
    int e = q < S ? topk_idx[walk_slot(q, N, k, first_choice)] : E;  // E = "no slot"
    if ((unsigned)e >= (unsigned)E) e = E;  // an out-of-range id is treated as dropped
    my_e[c] = e;
    if (e < E) atomicAdd(&wcount[wave][e], 1);
  }
  __syncthreads();
  // Turn per-wave counts into per-wave base ranks: tile base + earlier waves.
  if (threadIdx.x < E) {
    const int e = threadIdx.x;
    int32_t run = base;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const int32_t c = wcount[w][e];
      wcount[w][e] = run;
      run += c;
    }
  }
  __syncthreads();

  // Bits needed to tell apart expert ids 0..E (E is the "no slot" id).
  const int nbits = 32 - __clz(E);
  const int32_t M = eoff[E];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int q = ws0 + c * 64 + lane;
    const int s = q < S ? walk_slot(q, N, k, first_choice) : q;  // the slot itself
    const int e = my_e[c];
    uint64_t same = ~0ull;
    for (int b = 0; b < nbits; ++b) {
      const uint64_t bal = __ballot((e >> b) & 1);
      same &= ((e >> b) & 1) ? bal : ~bal;
    }
    const int below = __popcll(same & lanemask_lt(lane));
    const int leader = 63 - __clzll(same);  // highest lane with this expert
    int32_t rank = 0;
    if (e < E) rank = wcount[wave][e] + below;
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
    if (e < E && lane == leader) wcount[wave][e] += __popcll(same);
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
    if (e < E) {
      if (rank < cap) {
        const int32_t row = eoff[e] + rank;
        row_of_slot[s] = row;
        token_of_row[row] = s / k;
        slot_of_row[row] = (int8_t)(s % k);
      } else {
        row_of_slot[s] = -1;
      }
    } else if (q < S) {
      row_of_slot[s] = -1;
    }
  }
  // Rows >= M (dropped capacity) are marked unused.
  for (int r = s0 + threadIdx.x; r < min(S, s0 + kTileSlots); r += 256) {
    if (r >= M) {
      token_of_row[r] = -1;
      slot_of_row[r] = -1;
    }
  }
}

// Token-major permute: one wave per token (grid-stride), 16-byte vectors.
// NT: the row stores carry the non-temporal cache policy, for layouts larger
// than the last-level cache (the expert FFN then reads them back from HBM
// either way, and plain stores would only evict other data on their way out).
template <bool NT>
__global__ __launch_bounds__(256) void dispatch_permute(const u32x4* __restrict__ x, int N,
                                                        int vec_per_row, int k,
                                                        const int32_t* __restrict__ row_of_slot,
                                                        u32x4* __restrict__ x_perm) {
  const int lane = threadIdx.x % 64;
  const int gw = blockIdx.x * 4 + threadIdx.x / 64;
  const int nw = gridDim.x * 4;
  for (int t = gw; t < N; t += nw) {
    int my_row = lane < k ? row_of_slot[(size_t)t * k + lane] : -1;
    int rows[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) rows[j] = __shfl(my_row, j, 64);
    const u32x4* src = x + (size_t)t * vec_per_row;
    for (int v0 = 0; v0 < vec_per_row; v0 += 64 * 4) {
      u32x4 buf[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int v = v0 + u * 64 + lane;
        if (v < vec_per_row) buf[u] = src[v];
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        if (j < k && rows[j] >= 0) {
          u32x4* dst = x_perm + (size_t)rows[j] * vec_per_row;
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const int v = v0 + u * 64 + lane;
            if (v < vec_per_row) {
              if constexpr (NT) __builtin_nontemporal_store(buf[u], &dst[v]);
              else dst[v] = buf[u];
            }
          }
        }
      }
    }
  }
}

// INT8 payload of the dispatch exchange (EP notes, "深入推导": INT8-quantised
// communication halves the exchange volume): the permuted rows leave as int8
// codes with one fp32 scale per token.  One wave per token keeps the row in
// registers (VPL 16-byte vectors per lane, a power of two up to kQ8MaxVec,
// chosen from d), takes its absmax with a wave max, and makes every decision
// as one fp32 IEEE operation rounded to nearest even (hipcc divides correctly
// rounded by default):
//   inv = 127 / amax,  q = clamp(rint(x * inv), -127, 127),  scale = amax / 127
// (a zero row gives q = 0 and scale 0).  Codes and scale go to each of the
// token's admitted rows: x is read once, d bytes + 4 written per row.
constexpr int kQ8MaxVec = 16;

__device__ __forceinline__ uint32_t q8_code(float v, float inv) {
  const float c = fminf(fmaxf(rintf(v * inv), -127.f), 127.f);
  return static_cast<uint32_t>(static_cast<int32_t>(c)) & 0xffu;
}

template <int DTYPE, int VPL>
__global__ __launch_bounds__(256) void dispatch_permute_q8(const u32x4* __restrict__ x, int N,
                                                           int vec_per_row, int k,
                                                           const int32_t* __restrict__ row_of_slot,
                                                           uint8_t* __restrict__ xq,
                                                           float* __restrict__ row_scale) {
  constexpr int EPV = DTYPE == 0 ? 4 : 8;  // elements (= code bytes) per 16-byte vector
  const int lane = threadIdx.x % 64;
  const int gw = blockIdx.x * 4 + threadIdx.x / 64;
  const int nw = gridDim.x * 4;
  const size_t d = (size_t)vec_per_row * EPV;
  for (int t = gw; t < N; t += nw) {
    const int my_row = lane < k ? row_of_slot[(size_t)t * k + lane] : -1;
    const u32x4* src = x + (size_t)t * vec_per_row;
    u32x4 buf[VPL];
#pragma unroll
    for (int u = 0; u < VPL; ++u) {
      const int v = u * 64 + lane;
      buf[u] = v < vec_per_row ? src[v] : u32x4{0u, 0u, 0u, 0u};
    }
    float amax = 0.f;
#pragma unroll
    for (int u = 0; u < VPL; ++u) {
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        if constexpr (DTYPE == 0) {
          amax = fmaxf(amax, fabsf(__uint_as_float(buf[u][c])));
        } else {
          amax = fmaxf(amax, fabsf(__uint_as_float(buf[u][c] << 16)));
          amax = fmaxf(amax, fabsf(__uint_as_float(buf[u][c] & 0xffff0000u)));
        }
      }
    }
    amax = wave_max(amax);
    const float inv = amax > 0.f ? 127.f / amax : 0.f;
    const float scale = amax > 0.f ? amax / 127.f : 0.f;
    // Codes of this lane's vectors: 4 (fp32) or 8 (bf16) bytes each.
    uint32_t lo[VPL], hi[VPL];
#pragma unroll
    for (int u = 0; u < VPL; ++u) {
      if constexpr (DTYPE == 0) {
        lo[u] = q8_code(__uint_as_float(buf[u][0]), inv) |
                q8_code(__uint_as_float(buf[u][1]), inv) << 8 |
                q8_code(__uint_as_float(buf[u][2]), inv) << 16 |
                q8_code(__uint_as_float(buf[u][3]), inv) << 24;
        hi[u] = 0;
      } else {
        uint32_t w[2] = {0u, 0u};
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const uint32_t pair = q8_code(__uint_as_float(buf[u][c] << 16), inv) |
                                q8_code(__uint_as_float(buf[u][c] & 0xffff0000u), inv) << 8;
          w[c / 2] |= pair << (16 * (c % 2));
        }
        lo[u] = w[0];
        hi[u] = w[1];
      }
    }
    // Each admitted row: one base address, the lane's vectors at fixed offsets.
    for (int j = 0; j < k; ++j) {
      const int r = __shfl(my_row, j, 64);  // uniform
      if (r < 0) continue;
      uint8_t* base = xq + (size_t)r * d + (size_t)lane * EPV;
#pragma unroll
      for (int u = 0; u < VPL; ++u) {
        if (u * 64 + lane < vec_per_row) {
          if constexpr (DTYPE == 0)
            *reinterpret_cast<uint32_t*>(base + u * 64 * EPV) = lo[u];
          else
            *reinterpret_cast<uint2*>(base + u * 64 * EPV) = make_uint2(lo[u], hi[u]);
        }
      }
    }
    if (lane < k && my_row >= 0) row_scale[my_row] = scale;
  }
}

// Receiver side of the INT8 payload: x_perm[r] = dtype(q[r] * scale[r]) (fp32
// product, then bf16 round-to-nearest-even) for r < *num_rows.  One wave per
// row; each lane turns 8 (bf16) or 4 (fp32) codes into one 16-byte vector.
template <int DTYPE>
__global__ __launch_bounds__(256) void dequantize_q8(const uint8_t* __restrict__ xq,
                                                     const float* __restrict__ row_scale,
                                                     const int32_t* __restrict__ num_rows,
                                                     int max_rows, int vec_per_row,
                                                     u32x4* __restrict__ out) {
  constexpr int EPV = DTYPE == 0 ? 4 : 8;
  const int lane = threadIdx.x % 64;
  const int gw = blockIdx.x * 4 + threadIdx.x / 64;
  const int nw = gridDim.x * 4;
  const int M = min(*num_rows, max_rows);
  const size_t d = (size_t)vec_per_row * EPV;
  for (int r = gw; r < M; r += nw) {
    const float sc = row_scale[r];
    const uint8_t* src = xq + (size_t)r * d;
    u32x4* dst = out + (size_t)r * vec_per_row;
    for (int v = lane; v < vec_per_row; v += 64) {
      u32x4 o;
      if constexpr (DTYPE == 0) {
        const uint32_t c4 = *reinterpret_cast<const uint32_t*>(src + (size_t)v * 4);
#pragma unroll
        for (int c = 0; c < 4; ++c)
          o[c] = __float_as_uint((float)(int8_t)(c4 >> (8 * c)) * sc);
      } else {
        const uint2 c8 = *reinterpret_cast<const uint2*>(src + (size_t)v * 8);
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const uint32_t word = c < 2 ? c8.x : c8.y;
          const int sh = 16 * (c % 2);
          o[c] = pack_bf16x2((float)(int8_t)(word >> sh) * sc, (float)(int8_t)(word >> (sh + 8)) * sc);
        }
      }
      dst[v] = o;
    }
  }
}

int q8_max_hidden(int dtype) { return kQ8MaxVec * 64 * (dtype == 0 ? 4 : 8); }

hipError_t launch_dequantize_q8(int max_rows, int d, int dtype, const void* xq,
                                const float* row_scale, const int32_t* num_rows, void* out,
                                hipStream_t st) {
  if (max_rows <= 0) return hipSuccess;
  const int vec_per_row = d * (dtype == 0 ? 4 : 2) / 16;
  const int blocks = std::max(1, std::min((max_rows + 3) / 4, 8192));
  if (dtype == 0)
    dequantize_q8<0><<<blocks, 256, 0, st>>>(static_cast<const uint8_t*>(xq), row_scale, num_rows,
                                              max_rows, vec_per_row, static_cast<u32x4*>(out));
  else
    dequantize_q8<1><<<blocks, 256, 0, st>>>(static_cast<const uint8_t*>(xq), row_scale, num_rows,
                                              max_rows, vec_per_row, static_cast<u32x4*>(out));
  return hipGetLastError();
}

// Padded layout: rows e cap + i with i >= admitted[e] are padding.  The index
// pass marks them (token_of_row = slot_of_row = -1); the row pass zero-fills
// them (x_perm rows, or the INT8 payload's codes and scale).  Admitted rows
// are written by dispatch_assign / the permute and never touched here.
__global__ __launch_bounds__(256) void dispatch_pad_index(const int32_t* __restrict__ admitted,
                                                          int E, int32_t cap,
                                                          int32_t* __restrict__ token_of_row,
                                                          int8_t* __restrict__ slot_of_row) {
  const long long rows = (long long)E * cap;
  for (long long r = (long long)blockIdx.x * 256 + threadIdx.x; r < rows;
       r += (long long)gridDim.x * 256) {
    const int e = (int)(r / cap);
    if (r - (long long)e * cap >= admitted[e]) {
      token_of_row[r] = -1;
      slot_of_row[r] = -1;
    }
  }
}

__global__ __launch_bounds__(256) void dispatch_pad_rows(const int32_t* __restrict__ admitted,
                                                         int E, int32_t cap, int row_bytes,
                                                         u32x4* __restrict__ rows_out,
                                                         float* __restrict__ row_scale) {
  const int lane = threadIdx.x % 64;
  const long long rows = (long long)E * cap;
  const int vec = row_bytes / 16;
  for (long long r = (long long)blockIdx.x * 4 + threadIdx.x / 64; r < rows;
       r += (long long)gridDim.x * 4) {
    const int e = (int)(r / cap);
    if (r - (long long)e * cap < admitted[e]) continue;
    u32x4* dst = rows_out + r * vec;
    for (int v = lane; v < vec; v += 64) dst[v] = u32x4{0u, 0u, 0u, 0u};
    if (row_scale && lane == 0) row_scale[r] = 0.f;
  }
}

size_t dispatch_rows(int N, int k, int E, int32_t cap, int padded) {
  const size_t S = (size_t)N * k;
  if (!padded) return S;
  const size_t P = (size_t)E * (size_t)cap;
  return P > S ? P : S;
}

size_t dispatch_workspace_bytes(int N, int k, int E) {
  const size_t S = (size_t)N * k;
  const size_t tiles = (S + kTileSlots - 1) / kTileSlots;
  return std::max<size_t>(tiles, 1) * (size_t)E * sizeof(int32_t);
}

hipError_t launch_dispatch(const DispatchArgs& a, hipStream_t st, int stages) {
  const int S = a.N * a.k;
  const int tiles = (S + kTileSlots - 1) / kTileSlots;
  int32_t* tile_counts = static_cast<int32_t*>(a.ws);
  if (stages & kDispatchLayout) {
    if (tiles > 0 && (long long)tiles * a.E <= kCountLds && a.E <= 1024) {
      dispatch_count<<<1, 1024, 0, st>>>(a.topk_idx, S, a.k, a.first_choice, tiles, a.E, a.R,
                                         a.cap, a.padded, tile_counts,
                                         a.expert_offsets, a.admitted, a.rank_offsets,
                                         a.rank_counts);
    } else {
      if (tiles > 0)
        dispatch_tile_hist<<<tiles, 256, 0, st>>>(a.topk_idx, S, a.k, a.E, a.first_choice,
                                                  tile_counts);
      dispatch_scan<<<1, 256, 0, st>>>(tile_counts, tiles, a.E, a.R, a.cap, a.padded,
                                       a.expert_offsets, a.admitted, a.rank_offsets,
                                       a.rank_counts);
    }
    if (tiles > 0)
      dispatch_assign<<<tiles, 256, 0, st>>>(a.topk_idx, S, a.k, a.first_choice, a.E, a.cap,
                                             tile_counts, a.expert_offsets, a.row_of_slot,
                                             a.token_of_row, a.slot_of_row);
    if (a.padded) {
      const long long rows = (long long)a.E * a.cap;
      const int blocks = (int)std::min<long long>((rows + 255) / 256, 4096);
      dispatch_pad_index<<<std::max(blocks, 1), 256, 0, st>>>(a.admitted, a.E, a.cap,
                                                              a.token_of_row, a.slot_of_row);
    }
  }
  if (!(stages & kDispatchPermute) || a.N == 0) return hipGetLastError();
  const int elem = a.dtype == 0 ? 4 : 2;
  const int vec_per_row = a.d * elem / 16;
  const int waves_needed = a.N;
  const int blocks = std::max(1, std::min((waves_needed + 3) / 4, 8192));
  if (a.xq) {
    // Vectors per lane the row needs, rounded up to a power of two (<= kQ8MaxVec).
    const int vpl = (vec_per_row + 63) / 64;
    auto go = [&](auto kernel) {
      kernel<<<blocks, 256, 0, st>>>(static_cast<const u32x4*>(a.x), a.N, vec_per_row, a.k,
                                     a.row_of_slot, static_cast<uint8_t*>(a.xq), a.row_scale);
    };
    if (a.dtype == 0) {
      if (vpl <= 1) go(dispatch_permute_q8<0, 1>);
      else if (vpl <= 2) go(dispatch_permute_q8<0, 2>);
      else if (vpl <= 4) go(dispatch_permute_q8<0, 4>);
      else if (vpl <= 8) go(dispatch_permute_q8<0, 8>);
      else go(dispatch_permute_q8<0, 16>);
    } else {
      if (vpl <= 1) go(dispatch_permute_q8<1, 1>);
      else if (vpl <= 2) go(dispatch_permute_q8<1, 2>);
      else if (vpl <= 4) go(dispatch_permute_q8<1, 4>);
      else if (vpl <= 8) go(dispatch_permute_q8<1, 8>);
      else go(dispatch_permute_q8<1, 16>);
    }
  } else {
    // Non-temporal row stores once the rows written (at most N k) exceed the
    // 256 MiB last-level cache.  Measured on MI355X (same-box A/B): DeepSeek-like
    // layer, 470 MB of rows: permute 109 -> 95 us alone and the up GEMM that
    // follows 3011 -> 2896 us in the step; rows that fit the cache (Switch 34 MB,
    // Mixtral-like 134 MB) are read back from it by the up GEMM, and there
    // non-temporal stores cost 3 to 5 us (permute or up GEMM).
    const bool nt = (unsigned long long)a.N * a.k * vec_per_row * 16ull > (256ull << 20);
    auto go = [&](auto kernel) {
      kernel<<<blocks, 256, 0, st>>>(static_cast<const u32x4*>(a.x), a.N, vec_per_row, a.k,
                                     a.row_of_slot, static_cast<u32x4*>(a.x_perm));
    };
    if (nt) go(dispatch_permute<true>);
    else go(dispatch_permute<false>);
  }
  if (a.padded && a.admitted) {  // padding rows of the padded layout: zeros
    const long long rows = (long long)a.E * a.cap;
    const int pblocks = (int)std::max<long long>(1, std::min<long long>((rows + 3) / 4, 8192));
    dispatch_pad_rows<<<pblocks, 256, 0, st>>>(
        a.admitted, a.E, a.cap, a.xq ? a.d : a.d * elem,
        static_cast<u32x4*>(a.xq ? a.xq : a.x_perm), a.xq ? a.row_scale : nullptr);
  }
  return hipGetLastError();
}

}  // namespace moe
