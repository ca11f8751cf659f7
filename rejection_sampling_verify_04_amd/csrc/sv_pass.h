// The vocabulary pass's reduction of one chunk of one logit row by one wave,
// shared by pass 1 and by the tree walks, which form a stop leaf's chunk
// statistics with the same arithmetic when pass 1 did not read its row.
//
// One wave reduces one chunk (8192 elements) as four sub-segments of 2048
// elements; each of the wave's load instructions reads 1 KB of consecutive
// bytes.  Each lane keeps a running offset and sum over its 128 elements of
// the chunk, and the lanes are combined once per chunk.  Offsets of sampled
// rows are integers (ceil of the scaled maximum), so every rescale of a sum
// is an exact power of two.
//
// Sources: the softmax statistics that the acceptance ratio and the draws
// need (kwkr.cn/news/620872 §2.3, §4.1; blog.lonae.com/posts/
// 2026-draft-model-kv-jDwzYp, formal-definition paragraph).
#pragma once

#include "sv_common.h"
#include "sv_internal.h"

namespace sv {

// One wave's 2048-element segment: lane l's vector j covers elements
// seg0 + (j * 64 + l) * EPV + [0, EPV), so each load instruction of the wave
// reads 1 KB of consecutive bytes.
template <int DT>
struct SegLoad {
  static constexpr int ES = DT ? 2 : 4;          // bytes per element
  static constexpr int EPV = 16 / ES;            // elements per 16-byte load
  static constexpr int NV = kPerLane / EPV;      // loads per lane per segment
  uint4 raw[NV];

  // Vectors past V read as -inf.  Rows are read once here, so the loads carry
  // the non-temporal hint.  With vectors valid (V a multiple of EPV) a vector
  // is either wholly inside the row or wholly past it.
  __device__ __forceinline__ void issue(const char* rowp, int V, int seg0) {
    const int lane = threadIdx.x & 63;
    constexpr uint32_t kNegInf = DT ? 0xff80ff80u : 0xff800000u;
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      const int e0 = seg0 + (j * 64 + lane) * EPV;
      if (e0 < V) {
        const u32x4_t w =
            __builtin_nontemporal_load((const u32x4_t*)(rowp + (long long)e0 * ES));
        raw[j] = make_uint4(w.x, w.y, w.z, w.w);
      } else {
        raw[j] = make_uint4(kNegInf, kNegInf, kNegInf, kNegInf);
      }
    }
  }

  __device__ __forceinline__ void unpack(float v[kPerLane]) const {
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      if (DT == 1) {
        const uint32_t w[4] = {raw[j].x, raw[j].y, raw[j].z, raw[j].w};
#pragma unroll
        for (int h = 0; h < 4; ++h) {
          v[j * 8 + 2 * h] = bf16_lo(w[h]);
          v[j * 8 + 2 * h + 1] = bf16_hi(w[h]);
        }
      } else {
        v[j * 4 + 0] = __uint_as_float(raw[j].x);
        v[j * 4 + 1] = __uint_as_float(raw[j].y);
        v[j * 4 + 2] = __uint_as_float(raw[j].z);
        v[j * 4 + 3] = __uint_as_float(raw[j].w);
      }
    }
  }
};

template <int DT>
__device__ __forceinline__ void seg_load_scalar(const char* rowp, int V, int seg0,
                                                float v[kPerLane]) {
  constexpr int EPV = SegLoad<DT>::EPV;
  constexpr int NV = SegLoad<DT>::NV;
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int j = 0; j < NV; ++j) {
#pragma unroll
    for (int k = 0; k < EPV; ++k) {
      const int e = seg0 + (j * 64 + lane) * EPV + k;
      v[j * EPV + k] = e < V ? load_logit<DT>(rowp, e) : -__builtin_huge_valf();
    }
  }
}

// A lane's running statistics over its elements of one chunk.
struct LaneStats {
  float c;     // sampled: integer log2 offset; greedy: largest value so far
  int idx;     // greedy: first index of that value
  double s;    // sampled: sum of 2^(x k - c)
};

// Fold one sub-segment (this lane's 32 values, in increasing index order:
// element e of vector j sits at seg0 + (j * 64 + lane) * EPV + e).
template <int DT>
__device__ __forceinline__ void lane_fold(float v[kPerLane], int seg0, bool greedy, float k2,
                                          LaneStats& st) {
  constexpr int EPV = SegLoad<DT>::EPV;
  constexpr int NV = SegLoad<DT>::NV;
  const int lane = threadIdx.x & 63;
  if (greedy) {
#pragma unroll
    for (int j = 0; j < NV; ++j) {
#pragma unroll
      for (int e = 0; e < EPV; ++e) {
        const float x = v[j * EPV + e];
        const bool gt = x > st.c;
        st.c = gt ? x : st.c;
        st.idx = gt ? seg0 + (j * 64 + lane) * EPV + e : st.idx;
      }
    }
    return;
  }
  float m = -__builtin_huge_valf();
#pragma unroll
  for (int e = 0; e < kPerLane; ++e) m = fmaxf(m, v[e]);
  const float mk = ceilf(m * k2);
  if (mk > st.c) {
    st.s = scale_pow2(st.s, st.c - mk);
    st.c = mk;
  }
  const float cu = st.c > -__builtin_huge_valf() ? st.c : 0.0f;  // all -inf so far: terms are 0
#pragma unroll
  for (int e = 0; e < kPerLane; ++e) v[e] = exp2_hw(fmaf(v[e], k2, -cu));
#pragma unroll
  for (int w = kPerLane / 2; w >= 1; w >>= 1) {
#pragma unroll
    for (int e = 0; e < w; ++e) v[e] += v[e + w];
  }
  st.s += (double)v[0];
}

// Combine the wave's lanes into the chunk's Partial.
__device__ __forceinline__ Partial wave_combine(const LaneStats& st, bool greedy) {
  if (greedy) {
    const unsigned long long key =
        ((unsigned long long)float_order_key(st.c) << 32) | (0xffffffffu - (uint32_t)st.idx);
    const unsigned long long best = wave_max_u64(key);
    return Partial{float_from_order_key((uint32_t)(best >> 32)),
                   (int)(0xffffffffu - (uint32_t)best), 0.0};
  }
  const float C = wave_max(st.c);
  if (!(C > -__builtin_huge_valf())) return Partial{-__builtin_huge_valf(), 0, 0.0};
  const double t = st.s != 0.0 ? scale_pow2(st.s, st.c - C) : 0.0;
  return Partial{C, 0, wave_sum(t)};
}

// A chunk's Partial formed by the calling wave alone, with the pass's own
// arithmetic (the same values, folded in the same order).  One sub-segment's
// loads are in flight while the one before is folded (vector path), so that
// the caller's registers are spared; or plain loads.
template <int DT>
__device__ __forceinline__ Partial wave_chunk_partial(const char* rowp, int V, int ch, int vec_ok,
                                                      bool greedy, float k2) {
  const int lane = threadIdx.x & 63;
  LaneStats st{-__builtin_huge_valf(), ch * kChunk + lane * SegLoad<DT>::EPV, 0.0};
  if (vec_ok) {
    SegLoad<DT> seg;
    seg.issue(rowp, V, ch * kChunk);
    for (int k = 0; k < kSubs; ++k) {
      float v[kPerLane];
      seg.unpack(v);
      if (k + 1 < kSubs) seg.issue(rowp, V, ch * kChunk + (k + 1) * kSubSpan);
      lane_fold<DT>(v, ch * kChunk + k * kSubSpan, greedy, k2, st);
    }
  } else {
    for (int k = 0; k < kSubs; ++k) {
      float v[kPerLane];
      const int seg0 = ch * kChunk + k * kSubSpan;
      seg_load_scalar<DT>(rowp, V, seg0, v);
      lane_fold<DT>(v, seg0, greedy, k2, st);
    }
  }
  return wave_combine(st, greedy);
}

}  // namespace sv
