// Device pieces shared by the finish passes (linear and tree): merging a
// row's chunk partials, token probabilities, stop-distribution weights,
// chunk masses and the in-chunk inverse-CDF search.
//
// Every pass forms weights and their sums with the same code in the same
// order, so chunk totals and in-chunk cumulative sums agree bit for bit.
#pragma once

#include "sv_common.h"
#include "sv_internal.h"

namespace sv {

struct RowStats {
  float c;     // log2 offset (sampled) or max logit (greedy)
  int amax;    // first argmax (greedy)
  double s;    // sum of 2^(x k - c) (sampled)
  double inv_s;  // 1 / s
};

static_assert(kMaxChunks * kPartsPerChunk <= 64, "one partial per lane");

// This lane's partial of a row (lane j holds partial j), or an empty one.
// Every lane loads (from a clamped index), so that no load sits behind a
// branch: a load whose value crosses a branch join is waited for there.
// Lanes >= n_parts read partial 0; the merge ignores them.
__device__ __forceinline__ Partial lane_partial(const Partial* __restrict__ p, int n_parts) {
  const int lane = threadIdx.x & 63;
  return p[lane < n_parts ? lane : 0];
}

// Merge one row's partials, loaded one per lane (lanes >= n_parts ignored),
// with one wave; returns false when the row has no finite maximum.  Both the
// greedy and the sampled merge are formed and one is selected, so that every
// field of the loaded partial is used on one path and its load stays whole
// and ahead of any branch.
__device__ bool merge_parts_wave(const Partial& q_in, int n_parts, bool greedy, RowStats* out) {
  const int lane = threadIdx.x & 63;
  const bool valid = lane < n_parts;
  const float qc = valid ? q_in.c : -__builtin_huge_valf();
  const double qs = valid ? q_in.s : 0.0;
  // greedy: largest value, lowest index on ties
  const unsigned long long key =
      valid ? ((unsigned long long)float_order_key(q_in.c) << 32) | (0xffffffffu - (uint32_t)q_in.amax)
            : 0ull;
  const unsigned long long best = wave_max_u64(key);
  const float gm = float_from_order_key((uint32_t)(best >> 32));
  // sampled: common integer offset, exact rescale of each chunk sum
  const float C = wave_max(qc);
  const double S = wave_sum(qs > 0.0 ? scale_pow2(qs, qc - C) : 0.0);
  if (greedy) {
    out->c = gm;
    out->amax = (int)(0xffffffffu - (uint32_t)best);
    out->s = 0.0;
    out->inv_s = 0.0;
    return gm > -__builtin_huge_valf() && gm < __builtin_huge_valf();
  }
  out->c = C;
  out->amax = 0;
  out->s = S;
  out->inv_s = 1.0 / S;
  const bool finite_c = C > -__builtin_huge_valf() && C < __builtin_huge_valf();
  return finite_c && S > 0.0 && S < __builtin_huge_val();
}

// Segmented forms of the merge: lanes in groups of P (a power of two, 1..64,
// uniform over the wave) each hold one partial of the group's row, so a wave
// merges 64 / P rows at once.  Within 16 lanes the groups combine through
// DPP butterflies; wider groups through lane permutes.  Every lane of a group
// gets the same result.
__device__ __forceinline__ uint32_t lane_xor_u32(uint32_t v, int m) {
  const int src = ((int)(threadIdx.x & 63) ^ m) << 2;
  return (uint32_t)__builtin_amdgcn_ds_bpermute(src, (int)v);
}
__device__ __forceinline__ float seg_max_f32(float v, int P) {
  if (P >= 2) v = fmaxf(v, dpp_f32<kDppXor1>(v));
  if (P >= 4) v = fmaxf(v, dpp_f32<kDppXor2>(v));
  if (P >= 8) v = fmaxf(v, dpp_f32<kDppHalfMirror>(v));
  if (P >= 16) v = fmaxf(v, dpp_f32<kDppMirror>(v));
  if (P >= 32) v = fmaxf(v, __uint_as_float(lane_xor_u32(__float_as_uint(v), 16)));
  if (P >= 64) v = fmaxf(v, __uint_as_float(lane_xor_u32(__float_as_uint(v), 32)));
  return v;
}
__device__ __forceinline__ double lane_xor_f64(double v, int m) {
  const uint64_t b = (uint64_t)__double_as_longlong(v);
  const uint64_t lo = lane_xor_u32((uint32_t)b, m), hi = lane_xor_u32((uint32_t)(b >> 32), m);
  return __longlong_as_double((long long)((hi << 32) | lo));
}
__device__ __forceinline__ double seg_sum_f64(double v, int P) {
  if (P >= 2) v += dpp_f64<kDppXor1>(v);
  if (P >= 4) v += dpp_f64<kDppXor2>(v);
  if (P >= 8) v += dpp_f64<kDppHalfMirror>(v);
  if (P >= 16) v += dpp_f64<kDppMirror>(v);
  if (P >= 32) v += lane_xor_f64(v, 16);
  if (P >= 64) v += lane_xor_f64(v, 32);
  return v;
}
__device__ __forceinline__ uint64_t seg_max_u64(uint64_t v, int P) {
  uint64_t w;
  if (P >= 2) { w = dpp_u64<kDppXor1>(v); v = w > v ? w : v; }
  if (P >= 4) { w = dpp_u64<kDppXor2>(v); v = w > v ? w : v; }
  if (P >= 8) { w = dpp_u64<kDppHalfMirror>(v); v = w > v ? w : v; }
  if (P >= 16) { w = dpp_u64<kDppMirror>(v); v = w > v ? w : v; }
  if (P >= 32) {
    w = ((uint64_t)lane_xor_u32((uint32_t)(v >> 32), 16) << 32) | lane_xor_u32((uint32_t)v, 16);
    v = w > v ? w : v;
  }
  if (P >= 64) {
    w = ((uint64_t)lane_xor_u32((uint32_t)(v >> 32), 32) << 32) | lane_xor_u32((uint32_t)v, 32);
    v = w > v ? w : v;
  }
  return v;
}

// The group merge of one row (`valid`: this lane holds one of its partials);
// returns false when the row has no finite maximum.  Same results as
// merge_parts_wave up to the order of the float64 additions.
__device__ __forceinline__ bool merge_parts_seg(const Partial& q_in, bool valid, int P,
                                                bool greedy, RowStats* out) {
  const float qc = valid ? q_in.c : -__builtin_huge_valf();
  const double qs = valid ? q_in.s : 0.0;
  const unsigned long long key =
      valid ? ((unsigned long long)float_order_key(q_in.c) << 32) | (0xffffffffu - (uint32_t)q_in.amax)
            : 0ull;
  const unsigned long long best = seg_max_u64(key, P);
  const float gm = float_from_order_key((uint32_t)(best >> 32));
  const float C = seg_max_f32(qc, P);
  const double S = seg_sum_f64(qs > 0.0 ? scale_pow2(qs, qc - C) : 0.0, P);
  if (greedy) {
    out->c = gm;
    out->amax = (int)(0xffffffffu - (uint32_t)best);
    out->s = 0.0;
    out->inv_s = 0.0;
    return gm > -__builtin_huge_valf() && gm < __builtin_huge_valf();
  }
  out->c = C;
  out->amax = 0;
  out->s = S;
  out->inv_s = 1.0 / S;
  const bool finite_c = C > -__builtin_huge_valf() && C < __builtin_huge_valf();
  return finite_c && S > 0.0 && S < __builtin_huge_val();
}

// Lanes per row of a segmented merge: n_parts rounded up to a power of two.
__host__ __device__ inline int seg_width(int n_parts) {
  int P = 1;
  while (P < n_parts) P <<= 1;
  return P;
}

__device__ __forceinline__ bool merge_row_wave(const Partial* __restrict__ p, int n_parts,
                                               bool greedy, RowStats* out) {
  return merge_parts_wave(lane_partial(p, n_parts), n_parts, greedy, out);
}

// 2^e for a float64 e: the integer part exactly (ldexp), the fraction in
// [-1/2, 1/2] through the hardware 2^x (about 1e-7 relative).
__device__ __forceinline__ double exp2_split(double e) {
  const double n = __builtin_rint(e);
  const float f = (float)(e - n);
  return __builtin_ldexp((double)exp2_hw(f), (int)fmax(fmin(n, 2000.0), -2000.0));
}

// Probability of token `tok` under a merged row (exponent formed exactly in
// float64: x k is exact there and the offset is an integer).
__device__ __forceinline__ double row_prob(const RowStats& r, bool greedy, float k2, float x,
                                           int tok) {
  if (greedy) return tok == r.amax ? 1.0 : 0.0;
  return exp2_split((double)x * (double)k2 - (double)r.c) * r.inv_s;
}

// The stop distribution's unnormalised weights for one row.
struct StopDist {
  const void* prow;       // target row at the stop position / node
  const void* qrow;       // draft row (residual only)
  int residual;           // 1: max(0, p - q); 0: p
  int q_greedy, q_amax;
  float p_k, p_c, p_inv_s;
  float q_k, q_c, q_inv_s;
};

// A thread's total of its 8 weights: pairwise in float32, once to float64.
// Every pass forms thread totals through this code.
__device__ __forceinline__ double thread_total(const float w[kPerThread]) {
  static_assert((kPerThread & (kPerThread - 1)) == 0, "pairwise tree");
  float t[kPerThread];
#pragma unroll
  for (int e = 0; e < kPerThread; ++e) t[e] = w[e];
#pragma unroll
  for (int h = kPerThread / 2; h >= 1; h >>= 1) {
#pragma unroll
    for (int e = 0; e < h; ++e) t[e] = t[2 * e] + t[2 * e + 1];
  }
  return (double)t[0];
}

// This thread's 8 contiguous elements of one chunk of the stop row(s), as
// loaded (vector path).
template <int DT>
struct StopVec {
  static constexpr int ES = DT ? 2 : 4;
  static constexpr int EPV = 16 / ES;
  static constexpr int NV = kPerThread / EPV;
  uint4 p[NV], q[NV];
};

// Issue this thread's loads of chunk `chunk` (vector path: V a multiple of
// the vector width, so each vector lies wholly inside or wholly past the
// row).  Vectors past V, and the draft row when it is not needed, load from
// a valid address whose values are never used; nothing sits behind a branch.
template <int DT>
__device__ __forceinline__ void stop_load(const StopDist& d, int V, int chunk, StopVec<DT>& r,
                                          int tix = threadIdx.x) {
  constexpr int ES = StopVec<DT>::ES, EPV = StopVec<DT>::EPV;
  const int e0 = chunk * kChunk + tix * kPerThread;
  const bool need_q = d.residual && !d.q_greedy;
  const char* prow = (const char*)d.prow;
  const char* qrow = need_q ? (const char*)d.qrow : prow;
#pragma unroll
  for (int j = 0; j < StopVec<DT>::NV; ++j) {
    const int ej = e0 + j * EPV;
    const long long off = ej < V ? (long long)ej * ES : 0;
    // read once per pass: non-temporal loads
    const u32x4_t pv = __builtin_nontemporal_load((const u32x4_t*)(prow + off));
    const u32x4_t qv = __builtin_nontemporal_load((const u32x4_t*)(qrow + off));
    r.p[j] = make_uint4(pv.x, pv.y, pv.z, pv.w);
    r.q[j] = make_uint4(qv.x, qv.y, qv.z, qv.w);
  }
}

// The 8 contiguous weights of thread `tix` (of 1024) in chunk `chunk` (zero
// past V and for the bits set in `mask`).  Every pass derives weights
// through this code.
template <int DT>
__device__ __forceinline__ void stop_weights_from(const StopDist& d, int V, int chunk, int vec_ok,
                                                  uint32_t mask, const StopVec<DT>& r,
                                                  float w[kPerThread], int tix = threadIdx.x) {
#pragma clang fp contract(off)
  constexpr int EPV = StopVec<DT>::EPV;
  const int e0 = chunk * kChunk + tix * kPerThread;
  float xp[kPerThread], xq[kPerThread];
  const bool need_q = d.residual && !d.q_greedy;
  if (vec_ok) {
#pragma unroll
    for (int j = 0; j < StopVec<DT>::NV; ++j) {
      const uint32_t rw[4] = {r.p[j].x, r.p[j].y, r.p[j].z, r.p[j].w};
      const uint32_t sw[4] = {r.q[j].x, r.q[j].y, r.q[j].z, r.q[j].w};
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        if (DT == 1) {
          xp[j * 8 + 2 * h] = bf16_lo(rw[h]);
          xp[j * 8 + 2 * h + 1] = bf16_hi(rw[h]);
          xq[j * 8 + 2 * h] = bf16_lo(sw[h]);
          xq[j * 8 + 2 * h + 1] = bf16_hi(sw[h]);
        } else {
          xp[j * EPV + h] = __uint_as_float(rw[h]);
          xq[j * EPV + h] = __uint_as_float(sw[h]);
        }
      }
    }
  } else {
#pragma unroll
    for (int e = 0; e < kPerThread; ++e) {
      const int idx = e0 + e;
      xp[e] = idx < V ? load_logit<DT>(d.prow, idx) : 0.0f;
      xq[e] = (need_q && idx < V) ? load_logit<DT>(d.qrow, idx) : 0.0f;
    }
  }
  // One straight-line loop per case (the cases are uniform over the block),
  // then the range and mask tests, behind a test of the whole wave, only
  // where they can matter.  No product is fused into the difference, so
  // every pass forms the same weights.
  if (!d.residual) {
#pragma unroll
    for (int e = 0; e < kPerThread; ++e) w[e] = exp2_hw(fmaf(xp[e], d.p_k, -d.p_c)) * d.p_inv_s;
  } else if (!d.q_greedy) {
#pragma unroll
    for (int e = 0; e < kPerThread; ++e) {
      const float p = exp2_hw(fmaf(xp[e], d.p_k, -d.p_c)) * d.p_inv_s;
      const float q = exp2_hw(fmaf(xq[e], d.q_k, -d.q_c)) * d.q_inv_s;
      w[e] = fmaxf(p - q, 0.0f);
    }
  } else {
#pragma unroll
    for (int e = 0; e < kPerThread; ++e) {
      const float p = exp2_hw(fmaf(xp[e], d.p_k, -d.p_c)) * d.p_inv_s;
      w[e] = fmaxf(p - (e0 + e == d.q_amax ? 1.0f : 0.0f), 0.0f);
    }
  }
  const bool plain = mask == 0u && e0 + kPerThread <= V;
  if (__ballot(!plain) != 0ull) {
#pragma unroll
    for (int e = 0; e < kPerThread; ++e)
      if (!plain && (e0 + e >= V || ((mask >> e) & 1u))) w[e] = 0.0f;
  }
}

template <int DT>
__device__ __forceinline__ void stop_weights(const StopDist& d, int V, int chunk, int vec_ok,
                                             uint32_t mask, float w[kPerThread]) {
  StopVec<DT> r;
  if (vec_ok) stop_load<DT>(d, V, chunk, r);
  stop_weights_from<DT>(d, V, chunk, vec_ok, mask, r, w);
}

template <int DT>
__device__ double chunk_mass(const StopDist& d, int V, int chunk, int vec_ok, uint32_t mask,
                             double* s_scan) {
  float w[kPerThread];
  stop_weights<DT>(d, V, chunk, vec_ok, mask, w);
  const double acc = thread_total(w);
  double total;
  block_exclusive_scan<kFinWaves>(acc, s_scan, &total);
  return total;
}

// Lowest index over the block of the per-thread candidates `found` (or
// 0x7fffffff), and the highest of `lastp` (or -1): a ballot per wave, then
// one shared slot per wave (waves cover increasing index ranges).
__device__ __forceinline__ void block_first_last(int found, int lastp, int* s_found, int* s_last,
                                                 int* first_out, int* last_out) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const unsigned long long fm = __ballot(found != 0x7fffffff);
  const unsigned long long lm = __ballot(lastp >= 0);
  const int wf = fm ? __builtin_amdgcn_readlane(found, __ffsll((long long)fm) - 1) : 0x7fffffff;
  const int wl = lm ? __builtin_amdgcn_readlane(lastp, 63 - __clzll((long long)lm)) : -1;
  if (lane == 0) {
    s_found[wave] = wf;
    s_last[wave] = wl;
  }
  __syncthreads();
  int f = 0x7fffffff, l = -1;
  for (int w = 0; w < kFinWaves; ++w) {
    if (f == 0x7fffffff) f = s_found[w];
    l = s_last[w] >= 0 ? s_last[w] : l;
  }
  *first_out = f;
  *last_out = l;
  __syncthreads();
}

// Given this thread's weights of one chunk and the block-exclusive prefix of
// the thread totals, the first index whose cumulative mass (from `base`)
// exceeds `target`; if rounding leaves it uncrossed, the last index with
// positive weight; if the chunk has none, its first index.
__device__ int find_in_chunk(const float w[kPerThread], int chunk, double base, double excl,
                             double target, int* s_found, int* s_last) {
  const int e0 = chunk * kChunk + threadIdx.x * kPerThread;
  int found = 0x7fffffff, lastp = -1;
  double run = base + excl;
#pragma unroll
  for (int e = 0; e < kPerThread; ++e) {
    run += (double)w[e];
    if (found == 0x7fffffff && run > target && w[e] > 0.0f) found = e0 + e;
    if (w[e] > 0.0f) lastp = e0 + e;
  }
  int f, l;
  block_first_last(found, lastp, s_found, s_last, &f, &l);
  if (f != 0x7fffffff) return f;
  return l >= 0 ? l : chunk * kChunk;
}

template <int DT>
__device__ int chunk_select(const StopDist& d, int V, int chunk, int vec_ok, uint32_t mask,
                            double base, double target, double* s_scan, int* s_found,
                            int* s_last) {
  float w[kPerThread];
  stop_weights<DT>(d, V, chunk, vec_ok, mask, w);
  const double acc = thread_total(w);
  double total;
  const double excl = block_exclusive_scan<kFinWaves>(acc, s_scan, &total);
  return find_in_chunk(w, chunk, base, excl, target, s_found, s_last);
}

// Wave 0 finds the chunk holding u * R (R = the lane-ordered sum of the
// chunk masses) and the mass before it; results land in shared memory.
__device__ void choose_chunk(const double* s_mass, int n_chunks, double u, int* s_jc,
                             double* s_base, double* s_t) {
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    const double m = lane < n_chunks ? s_mass[lane] : 0.0;
    const double incl = wave_inclusive_scan(m);
    const double R = readlane_f64(incl, 63);
    const double t = u * R;
    const double excl = wave_shift_up1(incl);
    const unsigned long long hit = __ballot(lane < n_chunks && m > 0.0 && incl > t);
    const unsigned long long pos = __ballot(lane < n_chunks && m > 0.0);
    // rounding left u * R uncrossed: the last chunk with mass
    const int jc = hit ? __ffsll((long long)hit) - 1 : (pos ? 63 - __clzll((long long)pos) : 0);
    const double base = readlane_f64(excl, jc);
    if (lane == 0) {
      *s_jc = jc;
      *s_base = base;
      *s_t = t;
    }
  }
  __syncthreads();
}

}  // namespace sv
