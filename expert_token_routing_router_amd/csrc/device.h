// device.h -- small device helpers shared by the gfx950 kernels of the MoE
// forward library (element conversion, wave reductions, vector types).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

constexpr int kWave = 64;  // CDNA wavefront width

typedef uint16_t bf16_t;  // raw bf16 bits

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));  // one 16-byte vector

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// fp32 -> bf16 bits, round to nearest even, NaN kept quiet: gfx950's
// v_cvt_pk_bf16_f32 (bit-identical to the integer RNE formula on normal,
// subnormal, infinite and NaN inputs).
typedef __bf16 bf16x2_v __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const bf16x2_v v = {static_cast<__bf16>(lo), static_cast<__bf16>(hi)};
  return __builtin_bit_cast(uint32_t, v);
}

// Load element i of a dtype-tagged buffer as fp32 (dtype 0 fp32, 1 bf16).
__device__ __forceinline__ float load_elem(const void* p, int dtype, size_t i) {
  if (dtype == 0) return static_cast<const float*>(p)[i];
  return bf16_to_f32(static_cast<const bf16_t*>(p)[i]);
}

__device__ __forceinline__ int lane_id() { return __lane_id(); }

// Wave reductions through DPP lane exchanges (gfx9 encodings), no LDS
// crossbar: a butterfly inside each row of 16 lanes (quad xor 1, quad xor 2,
// half-row mirror, row mirror), then row broadcasts (lane 15 into rows 1 and
// 3, lane 31 into rows 2 and 3) leave the reduction of all 64 lanes in lane
// 63, which v_readlane hands to every lane.
enum : int {
  kDppXor1 = 0xB1, kDppXor2 = 0x4E, kDppHalfMirror = 0x141, kDppMirror = 0x140,
  kDppBcast15 = 0x142, kDppBcast31 = 0x143
};

template <int CTRL, int ROWS = 0xF>
__device__ __forceinline__ int dpp_i(int old, int v) {
  return __builtin_amdgcn_update_dpp(old, v, CTRL, ROWS, 0xF, false);
}
template <int CTRL, int ROWS = 0xF>
__device__ __forceinline__ float dpp_f(float old, float v) {
  return __int_as_float(dpp_i<CTRL, ROWS>(__float_as_int(old), __float_as_int(v)));
}
template <int CTRL, int ROWS = 0xF>
__device__ __forceinline__ double dpp_d(double old, double v) {
  const long long o = __double_as_longlong(old), x = __double_as_longlong(v);
  const int lo = dpp_i<CTRL, ROWS>((int)o, (int)x);
  const int hi = dpp_i<CTRL, ROWS>((int)(o >> 32), (int)(x >> 32));
  return __longlong_as_double(((long long)hi << 32) | (unsigned)lo);
}
__device__ __forceinline__ float lane63(float v) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}
__device__ __forceinline__ double lane63(double v) {
  const long long b = __double_as_longlong(v);
  const int lo = __builtin_amdgcn_readlane((int)b, 63);
  const int hi = __builtin_amdgcn_readlane((int)(b >> 32), 63);
  return __longlong_as_double(((long long)hi << 32) | (unsigned)lo);
}
// v of lane ln (wave-uniform ln) in every lane.
__device__ __forceinline__ double bcast_lane(double v, int ln) {
  const long long b = __double_as_longlong(v);
  const int lo = __builtin_amdgcn_readlane((int)b, ln);
  const int hi = __builtin_amdgcn_readlane((int)(b >> 32), ln);
  return __longlong_as_double(((long long)hi << 32) | (unsigned)lo);
}

__device__ __forceinline__ float wave_sum(float v) {
  v += dpp_f<kDppXor1>(0.f, v);
  v += dpp_f<kDppXor2>(0.f, v);
  v += dpp_f<kDppHalfMirror>(0.f, v);
  v += dpp_f<kDppMirror>(0.f, v);
  v += dpp_f<kDppBcast15, 0xA>(0.f, v);
  v += dpp_f<kDppBcast31, 0xC>(0.f, v);
  return lane63(v);
}

__device__ __forceinline__ double wave_sum(double v) {
  v += dpp_d<kDppXor1>(0.0, v);
  v += dpp_d<kDppXor2>(0.0, v);
  v += dpp_d<kDppHalfMirror>(0.0, v);
  v += dpp_d<kDppMirror>(0.0, v);
  v += dpp_d<kDppBcast15, 0xA>(0.0, v);
  v += dpp_d<kDppBcast31, 0xC>(0.0, v);
  return lane63(v);
}

__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp_f<kDppXor1>(v, v));
  v = fmaxf(v, dpp_f<kDppXor2>(v, v));
  v = fmaxf(v, dpp_f<kDppHalfMirror>(v, v));
  v = fmaxf(v, dpp_f<kDppMirror>(v, v));
  v = fmaxf(v, dpp_f<kDppBcast15, 0xA>(v, v));
  v = fmaxf(v, dpp_f<kDppBcast31, 0xC>(v, v));
  return lane63(v);
}

// (score, index) pair ordered by score descending, index ascending.  Returns
// the best pair over the wave in every lane.  Index -1 marks "no candidate".
template <int CTRL, int ROWS>
__device__ __forceinline__ void argmax_step(float& s, int& idx) {
  const float so = dpp_f<CTRL, ROWS>(0.f, s);
  const int io = dpp_i<CTRL, ROWS>(-1, idx);
  const bool take = (io >= 0) && (idx < 0 || so > s || (so == s && io < idx));
  s = take ? so : s;
  idx = take ? io : idx;
}
__device__ __forceinline__ void wave_argmax(float& s, int& idx) {
  argmax_step<kDppXor1, 0xF>(s, idx);
  argmax_step<kDppXor2, 0xF>(s, idx);
  argmax_step<kDppHalfMirror, 0xF>(s, idx);
  argmax_step<kDppMirror, 0xF>(s, idx);
  argmax_step<kDppBcast15, 0xA>(s, idx);
  argmax_step<kDppBcast31, 0xC>(s, idx);
  s = lane63(s);
  idx = __builtin_amdgcn_readlane(idx, 63);
}

// ------------------------------------------- direct global->LDS streaming ---

// LDS rows hold 32 bf16 (64 bytes = four 16-byte chunks).  Chunk c of row r
// lives at c ^ swz4(r): consecutive rows reading the same logical chunk then
// hit distinct bank groups for 8- and for 16-lane LDS phases.  The pattern
// depends on row bits 1-3 only, so rows 16 or 32 apart share it.
__device__ __forceinline__ int swz4(int r) { return ((r >> 1) ^ (r >> 2)) & 3; }
// The same for rows of eight 16-byte chunks (128 bytes): for each row parity,
// the eight rows of a 16-row group map one logical chunk to eight distinct
// physical chunks.
__device__ __forceinline__ int swz8(int r) { return (r ^ (r >> 3)) & 7; }

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// s_waitcnt vmcnt(N), other counters untouched (gfx9 encoding: vmcnt[3:0] in
// bits 3:0 and vmcnt[5:4] in bits 15:14; expcnt 7 and lgkmcnt 15 mean "no wait").
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | (((N >> 4) & 3) << 14));
}

// s_waitcnt lgkmcnt(0): this wave's LDS reads (and scalar loads) have
// returned; vmcnt 63 and expcnt 7 mean "no wait".
__device__ __forceinline__ void wait_lgkmcnt0() { __builtin_amdgcn_s_waitcnt(0xC07F); }

// Wait until at most `later` groups of PER loads each are still in flight
// (later <= 7; the ring's static checks keep 7 * PER below the 6-bit limit
// where it is reached, the clamp only keeps the unused cases compiling).
template <int PER>
__device__ __forceinline__ void wait_stages(int later) {
#define MOE_WS(n) wait_vmcnt<((n) * PER < 63 ? (n) * PER : 63)>()
  switch (later) {
    case 0: MOE_WS(0); break;
    case 1: MOE_WS(1); break;
    case 2: MOE_WS(2); break;
    case 3: MOE_WS(3); break;
    case 4: MOE_WS(4); break;
    case 5: MOE_WS(5); break;
    case 6: MOE_WS(6); break;
    default: MOE_WS(7); break;
  }
#undef MOE_WS
}

// Buffer resource over `bytes` bytes from `base` (gfx9 descriptor: stride 0,
// so offsets are raw bytes; word 3 = 32-bit data format, which raw dword
// loads need to be non-zero).  Loads at or past `bytes` return zero.  base
// must be wave-uniform: the resource lives in scalar registers.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                          0x00020000);
}

// 16 bytes per lane from resource r at byte offset voff (per lane) + soff
// (uniform) straight into LDS at dst + 16 * lane (dst uniform): one 1-KB
// buffer_load_dwordx4 ... lds per wave.  CPOL: cache-policy bits.
template <int CPOL>
__device__ __forceinline__ void buffer_load_lds16(__amdgpu_buffer_rsrc_t r, char* dst, uint32_t voff,
                                                  uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)dst, 16, voff, soff, 0, CPOL);
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

}  // namespace moe
