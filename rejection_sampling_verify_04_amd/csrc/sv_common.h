// Device helpers shared by the verify kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sv {

constexpr int kThreads = 256;          // vocabulary pass: 4 waves of 64
constexpr int kWaves = kThreads / 64;
constexpr int kChunk = 8192;           // vocabulary elements per chunk
constexpr int kWaveSpan = kChunk / kWaves;     // 2048 elements reduced by one wave
constexpr int kPerLane = kWaveSpan / 64;       // 32 elements per lane in the vocabulary pass
constexpr int kPartsPerChunk = kWaves;         // one partial per wave
constexpr int kFinThreads = 1024;      // finish passes: 16 waves of 64
constexpr int kFinWaves = kFinThreads / 64;
constexpr int kPerThread = kChunk / kFinThreads;  // 8 contiguous elements per thread
constexpr int kMaxChunks = 64;         // => V <= 524288
constexpr int kMaxGamma = 64;
constexpr int kMaxNodes = 64;

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
// c = an offset in log2 units and s = sum_v exp2(x_v * k - c) with
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

__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

__device__ __forceinline__ unsigned long long wave_max_u64(unsigned long long v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    unsigned long long w = __shfl_xor(v, o, 64);
    v = w > v ? w : v;
  }
  return v;
}

// Inclusive prefix sum over the 64 lanes of a wave, in lane order.
__device__ __forceinline__ double wave_inclusive_scan(double v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const double y = __shfl_up(v, o, 64);
    if (lane >= o) v += y;
  }
  return v;
}

// Exclusive prefix sum over a block of NW waves in thread order, plus the
// block total.  The total is formed the same way on every call, so two
// passes over the same per-thread values agree bit for bit.  All threads
// must call it; `scratch` is __shared__ with NW slots.
template <int NW>
__device__ __forceinline__ double block_exclusive_scan(double v, double* scratch, double* total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const double incl = wave_inclusive_scan(v);
  double excl_lane = __shfl_up(incl, 1, 64);
  if (lane == 0) excl_lane = 0.0;
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

// Order-preserving map of a float to uint32 (for max-with-lowest-index keys).
__device__ __forceinline__ uint32_t float_order_key(float f) {
  uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float float_from_order_key(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

}  // namespace sv
