// Device helpers shared by the verify kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sv {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;          // vocabulary pass: 4 waves of 64
constexpr int kWaves = kThreads / 64;
constexpr int kChunk = 8192;           // vocabulary elements per chunk
constexpr int kSubSpan = 2048;         // elements per sub-segment of the vocabulary pass
constexpr int kSubs = kChunk / kSubSpan;       // sub-segments per chunk
constexpr int kPerLane = kSubSpan / 64;        // 32 elements per lane and sub-segment
constexpr int kPartsPerChunk = 1;              // one Partial per (row, chunk)
constexpr int kFinThreads = 1024;      // finish passes: 16 waves of 64
constexpr int kFinWaves = kFinThreads / 64;
constexpr int kPerThread = kChunk / kFinThreads;  // 8 contiguous elements per thread
constexpr int kMaxChunks = 64;         // => V <= 524288
constexpr int kMaxGamma = 64;
constexpr int kMaxNodes = 64;
constexpr int kMaxDevices = 64;      // per-device caches of launch shapes

// Row status bits (mirrors the public header).
constexpr int kRowBadToken = 1;
constexpr int kRowBadShape = 2;
constexpr int kRowNonFinite = 4;
constexpr int kRowBadTemp = 8;
constexpr int kRowErrorMask = 0xFF;
constexpr int kRowWarnQZero = 256;
constexpr int kRowWarnRZero = 512;

constexpr double kLog2e = 1.4426950408889634074;

// One chunk's reduction of one logit row.  For a sampled row (T > 0):
// c = an integer offset in log2 units and s = sum_v exp2(x_v * k - c) with
// k = log2(e) / T; the pair stands for sum_v exp2(x_v * k) = s * 2^c.
// For a greedy row (T = 0): c = the maximum logit and amax its first index.
struct Partial {
  float c;
  int amax;
  double s;
};

// log2(e) / T rounded once to float; every kernel derives it the same way.
__device__ __forceinline__ float log2e_over_t(float T) {
  return (float)(kLog2e / (double)T);
}

__device__ __forceinline__ bool temp_ok(float T) {
  return T >= 0.0f && T < __builtin_huge_valf();
}

// Raw hardware 2^x (v_exp_f32).
__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

// s * 2^d for an integer-valued d <= 0 (exact; -inf and huge |d| give 0).
__device__ __forceinline__ double scale_pow2(double s, float d) {
  return __builtin_ldexp(s, (int)fmaxf(d, -4096.0f));
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __uint_as_float(((uint32_t)h) << 16);
}

// One logit, element type chosen at compile time (0 = fp32, 1 = bf16).
template <int DT>
__device__ __forceinline__ float load_logit(const void* base, long long idx) {
  if (DT == 1) return bf16_to_f32(((const uint16_t*)base)[idx]);
  return ((const float*)base)[idx];
}

// Philox-4x32-10 (Salmon, Moraes, Dror, Shaw, SC'11): each round multiplies
// counter words 0 and 2 by the two round constants, keeps both halves of the
// 64-bit products, and mixes them with words 1 and 3 and the round key; the
// key is advanced by the two Weyl constants after every round.
__device__ __forceinline__ uint4 philox4x32_10(uint4 ctr, uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint32_t a = ctr.x, c = ctr.z;
    const uint32_t hi0 = __umulhi(0xD2511F53u, a);
    const uint32_t lo0 = 0xD2511F53u * a;
    const uint32_t hi1 = __umulhi(0xCD9E8D57u, c);
    const uint32_t lo1 = 0xCD9E8D57u * c;
    ctr = make_uint4(hi1 ^ ctr.y ^ k0, lo1, hi0 ^ ctr.w ^ k1, lo0);
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
  return ctr;
}

// Counter (slot, row id, step low, step high) under key (seed low, seed high).
__device__ __forceinline__ uint4 verify_words(uint64_t seed, uint64_t step, uint32_t row_id,
                                              uint32_t slot) {
  return philox4x32_10(make_uint4(slot, row_id, (uint32_t)step, (uint32_t)(step >> 32)),
                       (uint32_t)seed, (uint32_t)(seed >> 32));
}

__device__ __forceinline__ double word_to_uniform(uint32_t w) {
  return (double)(w >> 8) * (1.0 / 16777216.0);
}

// ---- wave- and block-wide reductions ----------------------------------------
//
// Within each row of 16 lanes the wave combines values with DPP lane moves
// (a butterfly for reductions, shifts for prefix sums); the four row results
// are then combined through readlane.  All 64 lanes must be active.

// DPP move of a 32-bit value; lanes whose source is outside the row read 0.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xf, 0xf, true);
}
template <int CTRL>
__device__ __forceinline__ double dpp_f64(double v) {
  const uint64_t b = (uint64_t)__double_as_longlong(v);
  const uint64_t lo = dpp_u32<CTRL>((uint32_t)b), hi = dpp_u32<CTRL>((uint32_t)(b >> 32));
  return __longlong_as_double((long long)((hi << 32) | lo));
}
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __uint_as_float(dpp_u32<CTRL>(__float_as_uint(v)));
}
template <int CTRL>
__device__ __forceinline__ uint64_t dpp_u64(uint64_t v) {
  return ((uint64_t)dpp_u32<CTRL>((uint32_t)(v >> 32)) << 32) | dpp_u32<CTRL>((uint32_t)v);
}
__device__ __forceinline__ double readlane_f64(double v, int lane) {
  const uint64_t b = (uint64_t)__double_as_longlong(v);
  const uint64_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)b, lane);
  const uint64_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(b >> 32), lane);
  return __longlong_as_double((long long)((hi << 32) | lo));
}
__device__ __forceinline__ uint64_t readlane_u64(uint64_t v, int lane) {
  const uint64_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, lane);
  const uint64_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), lane);
  return (hi << 32) | lo;
}

constexpr int kDppXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141; // lane i of 8 <- 7 - i
constexpr int kDppMirror = 0x140;     // lane i of 16 <- 15 - i
constexpr int kDppShr1 = 0x111, kDppShr2 = 0x112, kDppShr4 = 0x114, kDppShr8 = 0x118;
constexpr int kDppWaveShr1 = 0x138;   // lane i <- lane i - 1 across the wave
constexpr int kDppWaveShl1 = 0x130;   // lane i <- lane i + 1 across the wave

// Sum over the wave; every lane gets the same result.
__device__ __forceinline__ double wave_sum(double v) {
  v += dpp_f64<kDppXor1>(v);
  v += dpp_f64<kDppXor2>(v);
  v += dpp_f64<kDppHalfMirror>(v);
  v += dpp_f64<kDppMirror>(v);
  return (readlane_f64(v, 0) + readlane_f64(v, 16)) + (readlane_f64(v, 32) + readlane_f64(v, 48));
}

__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp_f32<kDppXor1>(v));
  v = fmaxf(v, dpp_f32<kDppXor2>(v));
  v = fmaxf(v, dpp_f32<kDppHalfMirror>(v));
  v = fmaxf(v, dpp_f32<kDppMirror>(v));
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
}

__device__ __forceinline__ unsigned long long wave_or_u64(unsigned long long v) {
  v |= dpp_u64<kDppXor1>(v);
  v |= dpp_u64<kDppXor2>(v);
  v |= dpp_u64<kDppHalfMirror>(v);
  v |= dpp_u64<kDppMirror>(v);
  return readlane_u64(v, 0) | readlane_u64(v, 16) | readlane_u64(v, 32) | readlane_u64(v, 48);
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, dpp_u32<kDppXor1>(v));
  v = max(v, dpp_u32<kDppXor2>(v));
  v = max(v, dpp_u32<kDppHalfMirror>(v));
  v = max(v, dpp_u32<kDppMirror>(v));
  const uint32_t r0 = (uint32_t)__builtin_amdgcn_readlane((int)v, 0);
  const uint32_t r1 = (uint32_t)__builtin_amdgcn_readlane((int)v, 16);
  const uint32_t r2 = (uint32_t)__builtin_amdgcn_readlane((int)v, 32);
  const uint32_t r3 = (uint32_t)__builtin_amdgcn_readlane((int)v, 48);
  return max(max(r0, r1), max(r2, r3));
}

__device__ __forceinline__ unsigned long long wave_max_u64(unsigned long long v) {
  uint64_t w = dpp_u64<kDppXor1>(v);
  v = w > v ? w : v;
  w = dpp_u64<kDppXor2>(v);
  v = w > v ? w : v;
  w = dpp_u64<kDppHalfMirror>(v);
  v = w > v ? w : v;
  w = dpp_u64<kDppMirror>(v);
  v = w > v ? w : v;
  uint64_t r = readlane_u64(v, 0);
  w = readlane_u64(v, 16);
  r = w > r ? w : r;
  w = readlane_u64(v, 32);
  r = w > r ? w : r;
  w = readlane_u64(v, 48);
  return w > r ? w : r;
}

// Inclusive prefix sum over the 64 lanes of a wave, in lane order.
__device__ __forceinline__ double wave_inclusive_scan(double v) {
  v += dpp_f64<kDppShr1>(v);
  v += dpp_f64<kDppShr2>(v);
  v += dpp_f64<kDppShr4>(v);
  v += dpp_f64<kDppShr8>(v);
  const int row = (threadIdx.x & 63) >> 4;
  const double t0 = readlane_f64(v, 15), t1 = readlane_f64(v, 31), t2 = readlane_f64(v, 47);
  const double add = row == 0 ? 0.0 : (row == 1 ? t0 : (row == 2 ? t0 + t1 : (t0 + t1) + t2));
  return v + add;
}

// The inclusive value of the previous lane (0 for lane 0).
__device__ __forceinline__ double wave_shift_up1(double v) { return dpp_f64<kDppWaveShr1>(v); }

// Exclusive prefix sum over a block of NW waves in thread order, plus the
// block total.  The total is formed the same way on every call, so two
// passes over the same per-thread values agree bit for bit.  All threads
// must call it; `scratch` is __shared__ with NW slots.
template <int NW>
__device__ __forceinline__ double block_exclusive_scan(double v, double* scratch, double* total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const double incl = wave_inclusive_scan(v);
  const double excl_lane = wave_shift_up1(incl);
  __syncthreads();
  if (lane == 63) scratch[w] = incl;
  __syncthreads();
  double base = 0.0;
  for (int i = 0; i < w; ++i) base += scratch[i];
  double t = scratch[0];
#pragma unroll
  for (int i = 1; i < NW; ++i) t += scratch[i];
  *total = t;
  return base + excl_lane;
}

// A value that is the same in every lane, kept in scalar registers.
// A 32-bit input word that every thread of the work item reads at the same
// address, read as a scalar load (constant address space): its wait does not
// also wait for the vector loads issued before it.  Only for inputs that no
// kernel of the launch writes.
__device__ __forceinline__ uint32_t load_uniform_u32(const void* p) {
  return *(const __attribute__((address_space(4))) uint32_t*)p;
}
__device__ __forceinline__ int load_uniform_i32(const int* p) {
  return (int)load_uniform_u32(p);
}
__device__ __forceinline__ float load_uniform_f32(const float* p) {
  return __uint_as_float(load_uniform_u32(p));
}

__device__ __forceinline__ int uni(int v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ float uni(float v) {
  return __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(v)));
}
__device__ __forceinline__ double uni(double v) {
  const unsigned long long u = (unsigned long long)__double_as_longlong(v);
  const unsigned long long lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)u);
  const unsigned long long hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(u >> 32));
  return __longlong_as_double((long long)((hi << 32) | lo));
}

// Order-preserving map of a float to uint32 (for max-with-lowest-index keys).
__device__ __forceinline__ uint32_t float_order_key(float f) {
  uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float float_from_order_key(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

}  // namespace sv
