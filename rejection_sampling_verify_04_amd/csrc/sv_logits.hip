// Vocabulary-wide verify kernels (linear and tree), gfx950.
//
// Pass 1, stats_kernel: a resident grid in which each wave reduces whole
// 8192-logit chunks of the logit rows (one HBM read of every logit, with
// non-temporal 16-byte loads in flight ahead of the reduction) into one
// Partial per (row, chunk): an integer log2 offset and a float64 sum of
// exponentials for a sampled row, the maximum and its first index for a
// greedy row.  Its first work items gather the logits at the draft tokens.
//
// Linear finish:
//   V of one chunk    linear_row_kernel: one work item per batch row takes
//                     the decision, forms the stop weights, scans and draws.
//   V of 2..4 chunks  linear_decide_mass_kernel (one work item per (row,
//                     chunk): decision, then the chunk's stop mass as 16 wave
//                     totals), then linear_select_kernel.
//   larger V          linear_decide_kernel (per row), linear_mass_kernel (a
//                     resident, pipelined grid over (row, chunk)), then
//                     linear_select_kernel (one wave per row: chunk from the
//                     masses, wave from the wave totals, element from that
//                     wave's 512 weights).
// Tree finish, tree_kernel: one work item per tree walks it with one lane per
// node and draws in one chunk of the stop row.
//
// Work items never wait for one another: a kernel boundary is the only
// synchronisation, because device-scope fences and atomics are costly here.
// Every pass forms weights and their sums with the same code in the same
// order, so chunk totals and in-chunk cumulative sums agree bit for bit.
//
// Sources: acceptance rule and first-reject stop (kwkr.cn/news/620872 §2.3,
// §4.1, §4.3; cf-1.com/news/5632551 §2.2); residual and bonus draws
// (blog.lonae.com/posts/2026-draft-model-kv-jDwzYp, formal-definition
// paragraph); greedy exact match (kwkr §4.3); tree walk over top-k siblings
// (kwkr §5.3; lonae tree-attention paragraphs).
#include <hip/hip_ext.h>

#include <algorithm>
#include <atomic>

#include "sv_common.h"
#include "sv_internal.h"

namespace sv {

// Largest j in [0, B) whose key off[j] + add * j is <= x.  All threads of the
// block take part; one round covers 256 keys, so B <= 256 needs one round.
__device__ int find_batch_row(const int* __restrict__ off, int B, long long x, int add,
                              int* s_best) {
  int lo = 0, len = B;
  while (len > 1) {
    const int step = (len + kThreads - 1) / kThreads;
    const int t = threadIdx.x;
    bool pred = false;
    if ((long long)t * step < len) {
      const int j = lo + t * step;
      pred = (long long)off[j] + (long long)add * j <= x;
    }
    if (t == 0) *s_best = 0;
    __syncthreads();
    if (pred) atomicMax(s_best, t);
    __syncthreads();
    const int best = *s_best;
    __syncthreads();
    lo += best * step;
    len = min(step, len - best * step);
  }
  return lo;
}

// ---------------------------------------------------------------------------
// Pass 1: statistics of every logit chunk.
//
// One wave reduces one chunk (8192 elements) of one row at a time, as four
// sub-segments of 2048 elements; each of the wave's load instructions reads
// 1 KB of consecutive bytes.  Each lane keeps a running offset and sum over
// its 128 elements of the chunk, and the lanes are combined once per chunk.
// The grid is sized to stay resident: wave g of G takes chunks g, g + G,
// g + 2G, ... of the concatenated rows, so at any moment the grid sweeps one
// contiguous window of the logits, and each wave's sub-segment loads run
// RING sub-segments ahead of the one it reduces, across chunk boundaries.
//
// Offsets of sampled rows are integers (ceil of the scaled maximum), so every
// rescale of a sum is an exact power of two.

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

constexpr int kStatsCache = 1024;  // batch rows whose offsets/temperatures go to LDS

// Largest j in [0, B) whose key off[j] + add * j is <= x, found by one wave
// with 64 probes per round (B <= 64: one round; B <= 4096: two).
__device__ __forceinline__ int wave_find_batch_row(const int* off, int B, long long x, int add) {
  const int lane = threadIdx.x & 63;
  int lo = 0, len = B;
  while (len > 1) {
    const int step = (len + 63) >> 6;
    bool pred = false;
    if (lane * step < len) {
      const int j = lo + lane * step;
      pred = (long long)off[j] + (long long)add * j <= x;
    }
    const unsigned long long m = __ballot(pred);
    const int best = m ? 63 - __builtin_clzll(m) : 0;
    lo += best * step;
    len = min(step, len - best * step);
  }
  return lo;
}

// Largest b in [0, B) with off[b] <= i, each lane for its own i (fixed
// number of steps: ceil(log2(B))).
__device__ __forceinline__ int lane_batch_row(const int* off, int B, long long i) {
  int lo = 0;
  for (int step = 1 << (31 - __builtin_clz(max(B, 1))); step > 0; step >>= 1)
    if (lo + step < B && (long long)off[lo + step] <= i) lo += step;
  return lo;
}

// s * 2^d for an integer-valued d <= 0 (exact; -inf and huge |d| give 0).
__device__ __forceinline__ double scale_pow2(double s, float d) {
  return __builtin_ldexp(s, (int)fmaxf(d, -4096.0f));
}

// Work items of the stats launch that gather logits at draft tokens (one
// item per thread): linear, total_draft items; tree, B * N.
__host__ __device__ inline long long gather_items(const StatsArgs& a) {
  return a.tree ? (long long)a.B * a.N : (long long)a.total_draft;
}
__host__ __device__ inline int gather_blocks(const StatsArgs& a) {
  return (int)((gather_items(a) + kThreads - 1) / kThreads);
}

// gath[i] = logit of item i's token: linear, x_i[d_i] at [i] and y_i[d_i]
// at [total_draft + i] (target row i + b for position i of batch row b,
// draft row i); tree, node j's token under its parent row at [j].  Tokens
// and parents outside their range read index 0 (the finish pass flags them).
template <int DT>
__device__ void gather_logits(const StatsArgs& a, int* s_off) {
  const long long n = gather_items(a);
  const long long it = (long long)blockIdx.x * kThreads + threadIdx.x;
  const int V = a.V;
  const bool cache = !a.tree && a.B <= kStatsCache;
  if (cache) {
    for (int i = threadIdx.x; i <= a.B; i += kThreads) s_off[i] = a.offsets[i];
    __syncthreads();
  }
  if (it >= n) return;
  const int tok = a.tokens[it];
  const int tc = (tok >= 0 && tok < V) ? tok : 0;
  if (a.tree) {
    const int par = a.parents[it];
    const long long xr = it - it % a.N + ((par >= 0 && par < a.N) ? par : 0);
    a.gath[it] = load_logit<DT>(a.rows_a, xr * V + tc);
  } else {
    const int b = cache ? lane_batch_row(s_off, a.B, it) : lane_batch_row(a.offsets, a.B, it);
    a.gath[it] = load_logit<DT>(a.rows_a, (it + b) * V + tc);
    a.gath[n + it] = load_logit<DT>(a.rows_b, it * V + tc);
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

// RING = sub-segments in flight per wave: 2 for streaming many chunks per
// wave, 4 (a whole chunk) when every wave has about one chunk.
template <int DT, int RING>
__global__ __launch_bounds__(kThreads) void stats_kernel(StatsArgs a) {
  __shared__ int s_i[kStatsCache + 1];
  __shared__ float s_f0[kStatsCache], s_f1[kStatsCache];

  const int V = a.V;
  // The first work items gather the logits at the draft tokens; being
  // dispatched first, they finish while the rest stream the vocabulary.
  const int n_gblk = gather_blocks(a);
  if ((int)blockIdx.x < n_gblk) {
    gather_logits<DT>(a, s_i);
    return;
  }
  const int blk = blockIdx.x - n_gblk;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint32_t nc = (uint32_t)a.n_chunks;
  const uint32_t total = (uint32_t)a.n_rows * nc;   // < 2^31 (checked by the host)
  const uint32_t G = (gridDim.x - n_gblk) * kWaves;
  const uint32_t Gq = G / nc, Gr = G - Gq * nc;
  const long long rowbytes = (long long)V * SegLoad<DT>::ES;
  auto row_ptr = [&](uint32_t r) -> const char* {
    return r < a.n_a ? (const char*)a.rows_a + (long long)r * rowbytes
                     : (const char*)a.rows_b + ((long long)r - a.n_a) * rowbytes;
  };

  uint32_t u = blk * kWaves + wave;
  uint32_t row = u / nc, ch = u - row * nc;

  SegLoad<DT> ring[RING];
  // The first chunk's loads go out before anything else; an unused tree
  // row is still allocated, so reading it is harmless.
  if (a.vec_ok && u < total) {
#pragma unroll
    for (int r = 0; r < RING; ++r) ring[r].issue(row_ptr(row), V, (int)ch * kChunk + r * kSubSpan);
  }

  const bool cache = a.B <= kStatsCache;
  if (cache) {
    for (int i = threadIdx.x; i <= a.B; i += kThreads) {
      if (a.tree) {
        if (i < a.B) {
          s_i[i] = a.n_nodes ? a.n_nodes[i] : a.N;
          s_f0[i] = a.temp_a[i];
        }
      } else {
        s_i[i] = a.offsets[i];
        if (i < a.B) {
          s_f0[i] = a.temp_a[i];
          s_f1[i] = a.temp_b[i];
        }
      }
    }
    __syncthreads();
  }
  if (u >= total) return;

  // Whether a row's partials are needed (tree rows past n_nodes are not).
  auto row_used = [&](uint32_t r) -> bool {
    if (!a.tree) return true;
    const uint32_t b = r / (uint32_t)a.N;
    const int node = (int)(r - b * (uint32_t)a.N);
    const int nn = cache ? s_i[b] : (a.n_nodes ? a.n_nodes[b] : a.N);
    return node < nn;
  };
  auto row_temp = [&](uint32_t r) -> float {
    if (a.tree) {
      const uint32_t b = r / (uint32_t)a.N;
      return cache ? s_f0[b] : a.temp_a[b];
    }
    if (r < a.n_a) {
      if (cache) return s_f0[wave_find_batch_row(s_i, a.B, r, 1)];
      return a.temp_a[wave_find_batch_row(a.offsets, a.B, r, 1)];
    }
    const long long x = (long long)r - a.n_a;
    if (cache) return s_f1[wave_find_batch_row(s_i, a.B, x, 0)];
    return a.temp_b[wave_find_batch_row(a.offsets, a.B, x, 0)];
  };
  auto advance = [&](uint32_t& r, uint32_t& c) {
    c += Gr;
    r += Gq;
    if (c >= nc) {
      c -= nc;
      ++r;
    }
  };
  auto chunk_begin = [&](uint32_t c, float T, bool& greedy, float& k2) {
    greedy = T == 0.0f;
    k2 = greedy ? 0.0f : log2e_over_t(T);
    return LaneStats{-__builtin_huge_valf(), (int)c * kChunk + lane * SegLoad<DT>::EPV, 0.0};
  };
  auto chunk_end = [&](uint32_t r, uint32_t c, bool ok, bool greedy, const LaneStats& st) {
    // a bad temperature is reported by the finish pass
    const Partial p = ok ? wave_combine(st, greedy) : Partial{0.0f, 0, 0.0};
    if (lane == 0) a.part[(long long)r * nc + c] = p;
  };

  if (!a.vec_ok) {                        // unaligned rows: plain loads, no prefetch
    for (; u < total; u += G, advance(row, ch)) {
      if (!row_used(row)) continue;
      const float T = row_temp(row);
      const bool ok = temp_ok(T);
      bool greedy;
      float k2;
      LaneStats st = chunk_begin(ch, T, greedy, k2);
      if (ok) {
        for (int k = 0; k < kSubs; ++k) {
          float v[kPerLane];
          const int seg0 = (int)ch * kChunk + k * kSubSpan;
          seg_load_scalar<DT>(row_ptr(row), V, seg0, v);
          lane_fold<DT>(v, seg0, greedy, k2, st);
        }
      }
      chunk_end(row, ch, ok, greedy, st);
    }
    return;
  }

  bool used = row_used(row);
  float T = used ? row_temp(row) : 0.0f;
  for (;;) {
    uint32_t row1 = row, ch1 = ch;
    advance(row1, ch1);
    const bool has1 = u + G < total;
    const bool used1 = has1 && row_used(row1);
    const float T1 = used1 ? row_temp(row1) : 0.0f;
    const char* p0 = row_ptr(row);
    const char* p1 = row_ptr(row1);
    const bool ok = used && temp_ok(T);
    bool greedy;
    float k2;
    LaneStats st = chunk_begin(ch, T, greedy, k2);
#pragma unroll
    for (int k = 0; k < kSubs; ++k) {
      SegLoad<DT>& cur = ring[k % RING];
      const int seg0 = (int)ch * kChunk + k * kSubSpan;
      if (ok) {
        float v[kPerLane];
        cur.unpack(v);
        lane_fold<DT>(v, seg0, greedy, k2, st);
      }
      // refill this slot with the sub-segment RING ahead
      const int kn = k + RING;
      if (kn < kSubs) {
        if (used) cur.issue(p0, V, (int)ch * kChunk + kn * kSubSpan);
      } else if (used1) {
        cur.issue(p1, V, (int)ch1 * kChunk + (kn - kSubs) * kSubSpan);
      }
    }
    if (used) chunk_end(row, ch, ok, greedy, st);
    if (!has1) break;
    u += G;
    row = row1;
    ch = ch1;
    used = used1;
    T = T1;
  }
}

// ---------------------------------------------------------------------------
// Shared pieces of the finish passes.

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
    r.p[j] = *(const uint4*)(prow + off);
    r.q[j] = *(const uint4*)(qrow + off);
  }
}

// The 8 contiguous weights of thread `tix` (of 1024) in chunk `chunk` (zero
// past V and for the bits set in `mask`).  Every pass derives weights
// through this code.
template <int DT>
__device__ __forceinline__ void stop_weights_from(const StopDist& d, int V, int chunk, int vec_ok,
                                                  uint32_t mask, const StopVec<DT>& r,
                                                  float w[kPerThread], int tix = threadIdx.x) {
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
  // per-element range and mask tests only where they can matter
  const bool plain = mask == 0u && e0 + kPerThread <= V;
#pragma unroll
  for (int e = 0; e < kPerThread; ++e) {
    const int idx = e0 + e;
    float p = exp2_hw(fmaf(xp[e], d.p_k, -d.p_c)) * d.p_inv_s;
    if (d.residual) {
      const float q = d.q_greedy ? (idx == d.q_amax ? 1.0f : 0.0f)
                                 : exp2_hw(fmaf(xq[e], d.q_k, -d.q_c)) * d.q_inv_s;
      p = fmaxf(p - q, 0.0f);
    }
    if (!plain && (idx >= V || ((mask >> e) & 1u))) p = 0.0f;
    w[e] = p;
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

// ---------------------------------------------------------------------------
// Linear verify: the per-row decision (shared by the fused and split paths).

constexpr int kKindReject = 0, kKindBonus = 1, kKindGreedy = 2, kKindError = 3,
              kKindBadShape = 4;

constexpr int kDecideRowsPerWave = 2;   // logit rows each wave merges up front (2 g + 1 <= 32)

struct LinShared {
  RowStats rows[2 * kMaxGamma + 1];
  double p[kMaxGamma], q[kMaxGamma];
  int tok[kMaxGamma];
  int rowok[2 * kMaxGamma + 1];
  int flags, nacc;
  float usmp;
};

// Merge row b's partials (one wave per logit row), test its drafts and fill a
// record.  Writes every output token but the drawn one (all of them for
// greedy and error rows) and p/q at the drafts.  All threads take part.
template <int DT>
__device__ LinRecord linear_decide(const LinearArgs& a, int b, bool write_outputs,
                                   LinShared& sh) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n_parts = a.n_chunks * kPartsPerChunk;
  const int V = a.V;
  LinRecord r{};
  const int o0 = a.off[b], o1 = a.off[b + 1];
  const int g = o1 - o0;
  const float Tt = a.temp_t[b], Td = a.temp_d[b];
  r.o0 = o0;
  r.g = g;
  int err = 0;
  if (o0 < 0 || o1 < o0 || o1 > a.total_draft || g > kMaxGamma) err = kRowBadShape;
  else if (!temp_ok(Tt) || !temp_ok(Td)) err = kRowBadTemp;
  const long long tr0 = (long long)o0 + b;  // first target row of b
  if (err) {
    if (write_outputs && err != kRowBadShape)
      for (int i = tid; i <= g; i += kFinThreads) a.out_tokens[tr0 + i] = -1;
    r.kind = err == kRowBadShape ? kKindBadShape : kKindError;
    r.flags = err;
    return r;
  }
  const bool gt = Tt == 0.0f, gd = Td == 0.0f;
  const float kt = gt ? 0.0f : log2e_over_t(Tt);
  const float kd = gd ? 0.0f : log2e_over_t(Td);

  // Every wave loads the partials of its logit rows (target rows 0..g, then
  // draft rows 0..g-1) first, then the draft token of its lane's position
  // and the two logits at it; only wave 0's lanes < g keep the latter.  All
  // addresses are clamped to valid ones, so every lane loads unconditionally.
  const int nr = 2 * g + 1;
  auto row_of = [&](int rr) -> long long {
    return rr <= g ? tr0 + rr : a.n_target_rows + o0 + (rr - g - 1);
  };
  // rows wave + 4 k (k < kDecideRowsPerWave), clamped into [0, nr): loaded
  // and merged unconditionally
  Partial q[kDecideRowsPerWave];
#pragma unroll
  for (int k = 0; k < kDecideRowsPerWave; ++k)
    q[k] = lane_partial(a.part + row_of(min(wave + k * kFinWaves, nr - 1)) * n_parts, n_parts);
  // lane l's Philox block of slot l, formed while the loads are in flight
  // (wave 0 uses it: word 0 tests d_{l-1}, word 1 is the draw at stop l)
  const uint32_t rid = a.row_ids ? a.row_ids[b] : (uint32_t)b;
  const uint4 wl = verify_words(a.seed, a.step, rid, (uint32_t)lane);
  // the draft tokens and the logits at them (gathered by the vocabulary pass)
  const int li = min(lane, g > 0 ? g - 1 : 0);
  const int tok = *(g > 0 ? a.tokens + o0 + li : a.off);
  const float x = g > 0 ? a.gath[o0 + li] : 0.0f;
  const float y = g > 0 ? a.gath[a.total_draft + o0 + li] : 0.0f;
#pragma unroll
  for (int k = 0; k < kDecideRowsPerWave; ++k) {
    const int rr = min(wave + k * kFinWaves, nr - 1);
    RowStats rs;
    const bool ok = merge_parts_wave(q[k], n_parts, rr <= g ? gt : gd, &rs);
    if (lane == 0 && wave + k * kFinWaves < nr) {
      sh.rows[rr] = rs;
      sh.rowok[rr] = ok;
    }
  }
  // long draft runs (2g + 1 > 32 rows): the rest, one row per round
  for (int rr = wave + kDecideRowsPerWave * kFinWaves; rr < nr; rr += kFinWaves) {
    RowStats rs;
    const bool ok = merge_row_wave(a.part + row_of(rr) * n_parts, n_parts, rr <= g ? gt : gd, &rs);
    if (lane == 0) {
      sh.rows[rr] = rs;
      sh.rowok[rr] = ok;
    }
  }
  __syncthreads();

  if (tid < 64) {
    const int i = tid;
    bool reject = false, badtok = false, qzero = false, bad_row = false;
    for (int rr = i; rr < nr; rr += 64) bad_row |= !sh.rowok[rr];
    // slot 64 (g = 64 only) separately
    uint32_t acc_word = dpp_u32<kDppWaveShl1>(wl.x);   // lane i <- lane i + 1
    if (g == kMaxGamma && i == 63) acc_word = verify_words(a.seed, a.step, rid, 64u).x;
    if (i < g) {
      sh.tok[i] = tok;
      badtok = tok < 0 || tok >= V;
      const int tk = badtok ? 0 : tok;
      const double p = row_prob(sh.rows[i], gt, kt, x, tk);
      const double q = row_prob(sh.rows[g + 1 + i], gd, kd, y, tk);
      qzero = !(q > 0.0);
      // u < min(1, p / q), written without the division (u < 1; q = 0
      // accepts iff p > 0; p = 0 always rejects)
      const double u = word_to_uniform(acc_word);
      reject = !(u * q < p);
      sh.p[i] = p;
      sh.q[i] = q;
    }
    const unsigned long long rej = __ballot(reject);
    const int flags = (__ballot(bad_row) ? kRowNonFinite : 0) | (__ballot(badtok) ? kRowBadToken : 0) |
                      (__ballot(qzero) ? kRowWarnQZero : 0);
    const int nacc = rej ? (__ffsll((long long)rej) - 1) : g;
    const uint32_t smp_word = nacc < 64 ? (uint32_t)__builtin_amdgcn_readlane((int)wl.y, nacc)
                                        : verify_words(a.seed, a.step, rid, 64u).y;
    if (tid == 0) {
      sh.nacc = nacc;
      sh.flags = flags;
      sh.usmp = (float)word_to_uniform(smp_word);
    }
  }
  __syncthreads();
  const int flags = sh.flags;
  const int n_acc = sh.nacc;
  r.flags = flags;
  if (flags & kRowErrorMask) {
    if (write_outputs)
      for (int i = tid; i <= g; i += kFinThreads) a.out_tokens[tr0 + i] = -1;
    r.kind = kKindError;
    r.flags = flags & kRowErrorMask;
    return r;
  }
  r.n_acc = n_acc;
  if (write_outputs) {
    for (int i = tid; i <= g; i += kFinThreads) {
      if (i < n_acc) a.out_tokens[tr0 + i] = sh.tok[i];
      else if (i > n_acc) a.out_tokens[tr0 + i] = -1;
      else if (gt) a.out_tokens[tr0 + i] = sh.rows[n_acc].amax;
    }
    if (a.p_at) for (int i = tid; i < g; i += kFinThreads) a.p_at[o0 + i] = (float)sh.p[i];
    if (a.q_at) for (int i = tid; i < g; i += kFinThreads) a.q_at[o0 + i] = (float)sh.q[i];
  }
  if (gt) {  // greedy target: the draw is the argmax of target row n_acc (no randoms)
    r.kind = kKindGreedy;
    r.token = sh.rows[n_acc].amax;
    return r;
  }
  r.u_smp = sh.usmp;
  const bool residual = n_acc < g;
  r.kind = residual ? kKindReject : kKindBonus;
  r.p_k = kt;
  r.p_c = sh.rows[n_acc].c;
  r.p_inv_s = (float)sh.rows[n_acc].inv_s;
  if (residual) {
    const RowStats& qs = sh.rows[g + 1 + n_acc];
    r.q_greedy = gd;
    r.q_amax = qs.amax;
    r.q_k = kd;
    r.q_c = qs.c;
    r.q_inv_s = gd ? 0.0f : (float)qs.inv_s;
  }
  return r;
}

// The stop distribution a non-greedy record describes.
template <int DT>
__device__ __forceinline__ StopDist record_dist(const LinearArgs& a, int b, const LinRecord& r) {
  StopDist d;
  const long long tr0 = (long long)r.o0 + b;
  const long long es = DT ? 2 : 4;
  d.prow = (const char*)a.target + (tr0 + r.n_acc) * (long long)a.V * es;
  d.residual = r.kind == kKindReject;
  d.qrow = d.residual ? (const char*)a.draft + ((long long)r.o0 + r.n_acc) * a.V * es : d.prow;
  d.p_k = r.p_k;
  d.p_c = r.p_c;
  d.p_inv_s = r.p_inv_s;
  d.q_greedy = d.residual ? r.q_greedy : 0;
  d.q_amax = r.q_amax;
  d.q_k = d.residual ? r.q_k : 0.0f;
  d.q_c = r.q_c;
  d.q_inv_s = r.q_inv_s;
  return d;
}

__device__ __forceinline__ void write_row_status(const LinearArgs& a, int b, const LinRecord& r,
                                                 int warn) {
  if (r.kind == kKindBadShape || r.kind == kKindError) {
    a.num_accepted[b] = -1;
    if (a.row_status) a.row_status[b] = r.flags;
  } else {
    a.num_accepted[b] = r.n_acc;
    if (a.row_status) a.row_status[b] = (r.flags | warn) & ~kRowErrorMask;
  }
}

// ---------------------------------------------------------------------------
// Linear verify, V of one chunk: one work item per batch row does everything.

template <int DT>
__global__ __launch_bounds__(kFinThreads) void linear_row_kernel(LinearArgs a) {
  __shared__ LinShared sh;
  __shared__ double s_scan[kFinWaves];
  __shared__ int s_found[kFinWaves], s_last[kFinWaves];

  const int b = blockIdx.x;
  const LinRecord r = linear_decide<DT>(a, b, true, sh);
  int warn = 0;
  if (r.kind == kKindReject || r.kind == kKindBonus) {
    StopDist d = record_dist<DT>(a, b, r);
    float w[kPerThread];
    double R, excl;
    for (int pass = 0; pass < 2; ++pass) {
      stop_weights<DT>(d, a.V, 0, a.vec_ok, 0u, w);
      const double acc = thread_total(w);
      excl = block_exclusive_scan<kFinWaves>(acc, s_scan, &R);
      if (R > 0.0 || !d.residual) break;
      // zero residual mass (rounding only): draw from p at this position
      warn |= kRowWarnRZero;
      d.residual = 0;
    }
    const int token = find_in_chunk(w, 0, 0.0, excl, (double)r.u_smp * R, s_found, s_last);
    if (threadIdx.x == 0) a.out_tokens[(long long)r.o0 + b + r.n_acc] = token;
  }
  if (threadIdx.x == 0) write_row_status(a, b, r, warn);
}

// ---------------------------------------------------------------------------
// Linear verify, larger V: decide per row, mass per (row, chunk), select per row.

template <int DT>
__global__ __launch_bounds__(kFinThreads) void linear_decide_kernel(LinearArgs a) {
  __shared__ LinShared sh;
  const int b = blockIdx.x;
  const LinRecord r = linear_decide<DT>(a, b, true, sh);
  if (threadIdx.x == 0) a.rec[b] = r;
}

constexpr int kMassRecCache = 512;   // batch-row decisions staged in LDS by the mass pass

// Mass of the stop distribution per (row, chunk), kept as the chunk's 16 wave
// totals (the block scan's partial sums; the chunk mass is their sum in wave
// order).  The grid stays resident; work item g takes units g, g + G, ...
// (unit = row-major (row, chunk)), with the next unit's loads in flight
// while the current one is reduced.
// With CACHE the decisions are read from LDS only (B <= kMassRecCache), so
// that waiting for one never waits for the data loads in flight.
template <int DT, bool CACHE>
__global__ __launch_bounds__(kFinThreads) void linear_mass_kernel(LinearArgs a) {
  __shared__ LinRecord s_rec[CACHE ? kMassRecCache : 1];
  __shared__ double s_scan[kFinWaves];
  const int nc = a.n_chunks, V = a.V;
  const long long total = (long long)a.B * nc;
  if (CACHE) {
    for (int i = threadIdx.x; i < a.B; i += kFinThreads) s_rec[i] = a.rec[i];
    __syncthreads();
  }
  const long long G = gridDim.x;
  long long u = blockIdx.x;
  if (u >= total) return;
  // The unit's stop distribution; a unit with nothing to draw loads row 0.
  auto unit = [&](long long uu, int& bb, int& cc, bool& live) -> StopDist {
    bb = (int)(uu / nc);
    cc = (int)(uu - (long long)bb * nc);
    const LinRecord r = CACHE ? s_rec[bb] : a.rec[bb];
    live = r.kind == kKindReject || r.kind == kKindBonus;
    StopDist d = record_dist<DT>(a, bb, r);
    if (!live) {
      d.prow = d.qrow = a.target;
      d.residual = 0;
    }
    return d;
  };
  int b, c;
  bool live;
  auto reduce = [&](const StopDist& dd, int bb, int cc, const StopVec<DT>& cur, int vec) {
    float w[kPerThread];
    stop_weights_from<DT>(dd, V, cc, vec, 0u, cur, w);
    const double acc = thread_total(w);
    double m;
    block_exclusive_scan<kFinWaves>(acc, s_scan, &m);
    if (threadIdx.x < kFinWaves) a.wsum[((long long)bb * nc + cc) * kFinWaves + threadIdx.x] = s_scan[threadIdx.x];
  };
  if (!a.vec_ok) {                        // unaligned rows: plain loads, no prefetch
    const StopVec<DT> none{};
    for (; u < total; u += G) {
      const StopDist dd = unit(u, b, c, live);
      if (live) reduce(dd, b, c, none, 0);
    }
    return;
  }
  StopDist d = unit(u, b, c, live);
  StopVec<DT> buf0, buf1;
  stop_load<DT>(d, V, c, buf0);
  // One step: issue the next unit's loads into `nxt`, reduce the current
  // unit from `cur`; false when the current unit was this item's last.
  auto step = [&](StopVec<DT>& cur, StopVec<DT>& nxt) -> bool {
    const long long u1 = u + G;
    const bool has1 = u1 < total;
    int b1, c1;
    bool live1;
    const StopDist d1 = unit(has1 ? u1 : u, b1, c1, live1);
    live1 = live1 && has1;
    stop_load<DT>(d1, V, c1, nxt);
    if (live) reduce(d, b, c, cur, 1);
    u = u1;
    b = b1;
    c = c1;
    live = live1;
    d = d1;
    return has1;
  };
  for (;;) {
    if (!step(buf0, buf1)) break;
    if (!step(buf1, buf0)) break;
  }
}

// V of 2..4 chunks: every (row, chunk) work item takes the row's decision
// itself (identical arithmetic, so identical results; the chunk-0 item
// stores it and the accepted tokens) and then its chunk's wave totals, so
// that the stop row is read, and its weights formed, by as many compute
// units as it has chunks.
template <int DT>
__global__ __launch_bounds__(kFinThreads) void linear_decide_mass_kernel(LinearArgs a) {
  __shared__ LinShared sh;
  __shared__ double s_scan[kFinWaves];
  const int n_chunks = a.n_chunks;
  const int b = blockIdx.x / n_chunks;
  const int c = blockIdx.x - b * n_chunks;
  const LinRecord r = linear_decide<DT>(a, b, c == 0, sh);
  if (c == 0 && threadIdx.x == 0) a.rec[b] = r;
  if (r.kind != kKindReject && r.kind != kKindBonus) return;
  const StopDist d = record_dist<DT>(a, b, r);
  chunk_mass<DT>(d, a.V, c, a.vec_ok, 0u, s_scan);
  if (threadIdx.x < kFinWaves)
    a.wsum[((long long)b * n_chunks + c) * kFinWaves + threadIdx.x] = s_scan[threadIdx.x];
}

// This wave's 64 lanes form the weights of threads 64 w + lane (of 1024) of
// chunk c and their exclusive prefix within the wave, as the block scan does.
template <int DT>
__device__ __forceinline__ double wave_chunk_part(const StopDist& d, int V, int c, int w,
                                                  int vec_ok, float wt[kPerThread], double* acc_out) {
  const int tix = w * 64 + (threadIdx.x & 63);
  StopVec<DT> sv;
  if (vec_ok) stop_load<DT>(d, V, c, sv, tix);
  stop_weights_from<DT>(d, V, c, vec_ok, 0u, sv, wt, tix);
  const double acc = thread_total(wt);
  *acc_out = acc;
  return wave_inclusive_scan(acc);
}

// Select, one wave per batch row: the chunk holding u * R from the chunk masses (each the wave-order sum of its
// 16 wave totals), the wave of that chunk holding it from the running wave
// totals, then the element from that wave's 512 weights -- the same sums,
// in the same order, as a block-wide search over the chunk.  With zero
// residual mass (rounding only) the draw falls back to p, whose wave totals
// this wave then forms itself.
template <int DT>
__global__ __launch_bounds__(64) void linear_select_kernel(LinearArgs a) {
  __shared__ double s_ws[kMaxChunks * kFinWaves];
  const int lane = threadIdx.x;
  const int b = blockIdx.x;
  const int nc = a.n_chunks;
  const int nws = nc * kFinWaves;
  const double* wsb = a.wsum + (long long)b * nws;
  constexpr int kPerLaneWs = kMaxChunks * kFinWaves / 64;
  double wv[kPerLaneWs];
#pragma unroll
  for (int k = 0; k < kPerLaneWs; ++k) {
    const int i = lane + 64 * k;
    wv[k] = wsb[i < nws ? i : 0];
  }
  const LinRecord r = a.rec[b];
  int warn = 0;
  if (r.kind == kKindReject || r.kind == kKindBonus) {
    StopDist d = record_dist<DT>(a, b, r);
#pragma unroll
    for (int k = 0; k < kPerLaneWs; ++k)
      if (lane + 64 * k < nws) s_ws[lane + 64 * k] = wv[k];
    __syncthreads();
    auto chunk_masses = [&]() -> double {
      double m = 0.0;
      if (lane < nc) {
        const double* w = s_ws + lane * kFinWaves;
        m = w[0];
#pragma unroll
        for (int i = 1; i < kFinWaves; ++i) m += w[i];
      }
      return m;
    };
    double m = chunk_masses();
    double incl = wave_inclusive_scan(m);
    double R = readlane_f64(incl, 63);
    if (!(R > 0.0) && d.residual) {
      // zero residual mass: form p's wave totals here, chunk by chunk
      warn |= kRowWarnRZero;
      d.residual = 0;
      for (int c = 0; c < nc; ++c) {
        for (int w = 0; w < kFinWaves; ++w) {
          float wt[kPerThread];
          double acc;
          const double inc = wave_chunk_part<DT>(d, a.V, c, w, a.vec_ok, wt, &acc);
          const double tot = readlane_f64(inc, 63);
          if (lane == 0) s_ws[c * kFinWaves + w] = tot;
        }
      }
      __syncthreads();
      m = chunk_masses();
      incl = wave_inclusive_scan(m);
      R = readlane_f64(incl, 63);
    }
    // chunk
    const double t = (double)r.u_smp * R;
    const double excl = wave_shift_up1(incl);
    const unsigned long long hit = __ballot(lane < nc && m > 0.0 && incl > t);
    const unsigned long long pos = __ballot(lane < nc && m > 0.0);
    const int jc = hit ? __ffsll((long long)hit) - 1 : (pos ? 63 - __clzll((long long)pos) : 0);
    const double base = readlane_f64(excl, jc);
    // wave of the chunk: running wave totals X_w, summed from 0 in wave order
    const double* wj = s_ws + jc * kFinWaves;
    int ws_hit = -1, ws_pos = -1;
    double X = 0.0, Xw = 0.0;
    for (int w = 0; w < kFinWaves; ++w) {
      const double next = X + wj[w];
      if (wj[w] > 0.0) {
        if (ws_hit < 0 && base + next > t) {
          ws_hit = w;
          Xw = X;
        }
        ws_pos = w;
      }
      X = next;
    }
    int wsel = ws_hit;
    if (wsel < 0) {
      wsel = ws_pos >= 0 ? ws_pos : 0;
      X = 0.0;
      for (int w = 0; w < wsel; ++w) X += wj[w];
      Xw = X;
    }
    // element, within wave wsel of chunk jc
    float wt[kPerThread];
    double acc;
    const double inc = wave_chunk_part<DT>(d, a.V, jc, wsel, a.vec_ok, wt, &acc);
    double run = base + (Xw + wave_shift_up1(inc));
    const int e0 = jc * kChunk + (wsel * 64 + lane) * kPerThread;
    int found = 0x7fffffff, lastp = -1;
#pragma unroll
    for (int e = 0; e < kPerThread; ++e) {
      run += (double)wt[e];
      if (found == 0x7fffffff && run > t && wt[e] > 0.0f) found = e0 + e;
      if (wt[e] > 0.0f) lastp = e0 + e;
    }
    const unsigned long long fm = __ballot(found != 0x7fffffff);
    const unsigned long long lm = __ballot(lastp >= 0);
    int token;
    if (fm) token = __builtin_amdgcn_readlane(found, __ffsll((long long)fm) - 1);
    else if (lm) token = __builtin_amdgcn_readlane(lastp, 63 - __clzll((long long)lm));
    else token = jc * kChunk;
    if (lane == 0) a.out_tokens[(long long)r.o0 + b + r.n_acc] = token;
  }
  if (lane == 0) write_row_status(a, b, r, warn);
}

// ---------------------------------------------------------------------------
// Tree verify (TOPK): one work item per tree.

template <int DT>
__global__ __launch_bounds__(kFinThreads) void tree_kernel(TreeArgs a) {
  constexpr int kNodesPerWave = kMaxNodes / kFinWaves;
  __shared__ RowStats s_rows[kMaxNodes];
  __shared__ int s_par[kMaxNodes], s_tok[kMaxNodes], s_path[kMaxNodes], s_rowok[kMaxNodes];
  __shared__ double s_pn[kMaxNodes];
  __shared__ double s_cm[kMaxNodes * kMaxChunks];  // p's mass per (node, chunk)
  __shared__ int s_flags, s_stop, s_depth;
  __shared__ unsigned long long s_removed;   // node bits of the rejected siblings
  __shared__ double s_scan[kFinWaves];
  __shared__ double s_mass[kMaxChunks];
  __shared__ int s_found[kFinWaves], s_last[kFinWaves];
  __shared__ int s_jc;
  __shared__ double s_base, s_t;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n_chunks = a.n_chunks;
  const int n_parts = n_chunks * kPartsPerChunk;
  const int b = blockIdx.x;
  const int V = a.V, N = a.N;
  const int nn = a.n_nodes ? a.n_nodes[b] : N;
  const float T = a.temp[b];
  const long long rb = (long long)b * N;
  const uint32_t rid = a.row_ids ? a.row_ids[b] : (uint32_t)b;

  int err0 = 0;
  if (nn < 1 || nn > N) err0 = kRowBadShape;
  else if (!temp_ok(T)) err0 = kRowBadTemp;
  const bool greedy = T == 0.0f;
  const float k2 = (greedy || err0) ? 0.0f : log2e_over_t(T);

  // Every wave loads its node rows' partials (rows clamped into the tree)
  // and one node per lane: its parent, its token and the logit of the token
  // under the parent (gathered by the vocabulary pass).  Only wave 0's lanes
  // 1..nn-1 keep the latter.  No load sits behind a branch.
  Partial q[kNodesPerWave];
#pragma unroll
  for (int k = 0; k < kNodesPerWave; ++k) {
    const int n = min(wave + k * kFinWaves, N - 1);
    q[k] = lane_partial(a.part + (rb + n) * n_parts, n_parts);
  }
  const int li = lane < N ? lane : 0;
  int par = a.parents[rb + li];
  int tok = a.tokens[rb + li];
  const float x = a.gath[rb + li];   // gathered by the vocabulary pass
  const bool mine = !err0 && tid > 0 && tid < nn;
  const bool badpar = mine && (par < 0 || par >= tid);
  const bool badtok = mine && (tok < 0 || tok >= V);
  if (!mine) {
    par = -1;
    tok = 0;
  }
  if (!err0) {
#pragma unroll
    for (int k = 0; k < kNodesPerWave; ++k) {
      const int n = wave + k * kFinWaves;
      if (n < nn) {
        RowStats rs;
        const bool ok = merge_parts_wave(q[k], n_parts, greedy, &rs);
        if (lane == 0) {
          s_rows[n] = rs;
          s_rowok[n] = ok;
        }
        if (!greedy && lane < n_chunks)
          s_cm[n * n_chunks + lane] =
              q[k].s > 0.0 ? scale_pow2(q[k].s, q[k].c - rs.c) / rs.s : 0.0;
      }
    }
  }
  if (tid < kMaxNodes) {
    s_par[tid] = par;
    s_tok[tid] = tok;
  }
  __syncthreads();
  if (tid < 64) {
    const int flags = (__ballot(badpar) ? kRowBadShape : 0) | (__ballot(badtok) ? kRowBadToken : 0) |
                      (__ballot(tid < nn && !err0 && !s_rowok[tid < kMaxNodes ? tid : 0])
                           ? kRowNonFinite : 0);
    if (tid == 0) s_flags = err0 | flags;
  }
  __syncthreads();
  const int err = s_flags & kRowErrorMask;
  if (err) {
    for (int i = tid; i < N; i += kFinThreads) {
      a.out_tokens[rb + i] = -1;
      if (i < N - 1) a.path_nodes[(long long)b * (N - 1) + i] = -1;
      if (a.p_at) a.p_at[rb + i] = 0.0f;
    }
    if (tid == 0) {
      a.num_accepted[b] = -1;
      if (a.row_status) a.row_status[b] = err;
    }
    return;
  }

  double u_acc = 0.0;
  if (tid > 0 && tid < nn) {
    s_pn[tid] = row_prob(s_rows[par], greedy, k2, x, tok);
    u_acc = word_to_uniform(verify_words(a.seed, a.step, rid, (uint32_t)tid).x);
  }
  __syncthreads();

  // Walk: one lane per node; at each level the current node's children are
  // tested in index order through a prefix sum of the removed mass.
  if (tid < 64) {
    const int i = tid;
    int node = 0, depth = 0;
    unsigned long long removed = 0ull;
    while (true) {
      const bool child = i > node && i < nn && s_par[i] == node;
      const unsigned long long kids = __ballot(child);
      if (!kids) break;   // leaf: bonus draw from p
      // a sibling repeating an earlier sibling's token has nothing left to accept
      bool dup = false;
      if (child) {
        unsigned long long before = kids & ((1ull << i) - 1ull);
        while (before) {
          const int j = __ffsll((long long)before) - 1;
          before &= before - 1ull;
          dup |= s_tok[j] == s_tok[i];
        }
      }
      const double mass = (child && !dup) ? s_pn[i] : 0.0;
      const double incl = wave_inclusive_scan(mass);
      const double excl = wave_shift_up1(incl);
      const double denom = 1.0 - excl;
      const double ratio = (child && !dup && denom > 0.0) ? s_pn[i] / denom : 0.0;
      const unsigned long long acc = __ballot(child && u_acc < ratio);
      if (acc) {
        const int first = __ffsll((long long)acc) - 1;
        if (i == 0) s_path[depth] = first;
        ++depth;
        node = first;
        continue;
      }
      removed = __ballot(child && !dup);
      break;
    }
    if (i == 0) {
      s_stop = node;
      s_depth = depth;
      s_removed = removed;
    }
  }
  __syncthreads();
  const int stop = s_stop, depth = s_depth;
  const unsigned long long removed = s_removed;

  int token;
  int warn = 0;
  if (greedy) {
    token = s_rows[stop].amax;
  } else {
    const RowStats st = s_rows[stop];
    // chunk masses of p at the stop node, minus the rejected siblings'
    // probabilities
    if (tid < n_chunks) {
      double m = s_cm[stop * n_chunks + tid];
      unsigned long long rm = removed;
      const int lo = tid * kChunk, hi = lo + kChunk;
      double cut = 0.0;
      while (rm) {
        const int j = __ffsll((long long)rm) - 1;
        rm &= rm - 1ull;
        if (s_tok[j] >= lo && s_tok[j] < hi) cut += s_pn[j];
      }
      m -= cut;
      s_mass[tid] = m > 0.0 ? m : 0.0;
    }
    __syncthreads();
    double R = 0.0;
    for (int j = 0; j < n_chunks; ++j) R += s_mass[j];
    bool masked = removed != 0ull;
    __syncthreads();
    if (!(R > 0.0)) {
      // every sibling's token took the whole mass (rounding only): draw from p
      warn |= kRowWarnRZero;
      masked = false;
      if (tid < n_chunks) s_mass[tid] = s_cm[stop * n_chunks + tid];
      __syncthreads();
    }
    StopDist d;
    d.prow = (const char*)a.target + (rb + stop) * (long long)V * (DT ? 2 : 4);
    d.qrow = d.prow;
    d.residual = 0;
    d.p_k = k2;
    d.p_c = st.c;
    d.p_inv_s = (float)st.inv_s;
    d.q_greedy = 0;
    d.q_amax = 0;
    d.q_k = d.q_c = d.q_inv_s = 0.0f;
    const double u = word_to_uniform(verify_words(a.seed, a.step, rid, (uint32_t)stop).y);
    choose_chunk(s_mass, n_chunks, u, &s_jc, &s_base, &s_t);
    const int jc = s_jc;
    // bits of this thread's 8 elements that belong to rejected siblings
    uint32_t mk = 0u;
    if (masked) {
      const int e0 = jc * kChunk + tid * kPerThread;
      unsigned long long rm = removed;
      while (rm) {
        const int j = __ffsll((long long)rm) - 1;
        rm &= rm - 1ull;
        const int off = s_tok[j] - e0;
        if (off >= 0 && off < kPerThread) mk |= 1u << off;
      }
    }
    token = chunk_select<DT>(d, V, jc, a.vec_ok, mk, s_base, s_t, s_scan, s_found, s_last);
  }

  for (int i = tid; i < N; i += kFinThreads) {
    a.out_tokens[rb + i] = i < depth ? s_tok[s_path[i]] : (i == depth ? token : -1);
    if (i < N - 1) a.path_nodes[(long long)b * (N - 1) + i] = i < depth ? s_path[i] : -1;
    if (a.p_at) a.p_at[rb + i] = (i > 0 && i < nn) ? (float)s_pn[i] : 0.0f;
  }
  if (tid == 0) {
    a.num_accepted[b] = depth;
    if (a.row_status) a.row_status[b] = warn;
  }
}

// ---------------------------------------------------------------------------
// Raw Philox words (diagnostic entry point).

__global__ __launch_bounds__(kThreads) void philox_words_kernel(uint64_t seed, uint64_t step,
                                                                const uint32_t* row_ids,
                                                                int n_rows, int n_slots,
                                                                uint32_t* out) {
  const long long i = (long long)blockIdx.x * kThreads + threadIdx.x;
  if (i >= (long long)n_rows * n_slots) return;
  const int r = (int)(i / n_slots), s = (int)(i - (long long)r * n_slots);
  const uint4 w = verify_words(seed, step, row_ids ? row_ids[r] : (uint32_t)r, (uint32_t)s);
  uint4* o = (uint4*)(out + i * 4);
  *o = w;
}

// ---------------------------------------------------------------------------
// Host launchers.

// Chunks per stats work item: one while a single round of work items fills
// the GPU (short critical path), two beyond (more loads in flight per item).
long long stats_items(long long n_rows, int n_chunks) {
  return n_rows * n_chunks * kPartsPerChunk;
}

// Workgroups of a kernel that fit on the current device at once (cached per
// kernel slot and device).
template <typename K>
static int resident_blocks(int slot, K kernel, int threads) {
  static std::atomic<int> cache[8][kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) dev = 0;
  int c = cache[slot][dev].load(std::memory_order_relaxed);
  if (c == 0) {
    int n_cu = 0, occ = 0;
    if (hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      n_cu = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, kernel, threads, 0) != hipSuccess)
      occ = 0;
    c = std::max(1, n_cu) * std::max(1, occ);
    cache[slot][dev].store(c, std::memory_order_relaxed);
  }
  return c;
}

static int stats_resident_blocks(int dt, int ring) {
  if (dt == 1)
    return ring == 4 ? resident_blocks(0, stats_kernel<1, 4>, kThreads)
                     : resident_blocks(1, stats_kernel<1, 2>, kThreads);
  return resident_blocks(2, stats_kernel<0, 2>, kThreads);
}

static int mass_resident_blocks(int dt) {
  return dt == 1 ? resident_blocks(3, linear_mass_kernel<1, true>, kFinThreads)
                 : resident_blocks(4, linear_mass_kernel<0, true>, kFinThreads);
}

// Pass 1.  Launched with events, the events bracket the kernel's dispatch.
hipError_t launch_stats(int dtype, const StatsArgs& a, hipStream_t st, hipEvent_t ev_start,
                        hipEvent_t ev_stop) {
  const long long units = stats_items(a.n_rows, a.n_chunks);
  if (units <= 0) return hipSuccess;
  const int dt = dtype == 1 ? 1 : 0;
  const bool timed = ev_start && ev_stop;
  const dim3 block(kThreads);
#define SV_LAUNCH(K)                                                          \
  do {                                                                        \
    if (timed) hipExtLaunchKernelGGL(K, grid, block, 0, st, ev_start, ev_stop, 0, a); \
    else K<<<grid, block, 0, st>>>(a);                                        \
  } while (0)
  const long long want = (units + kWaves - 1) / kWaves;
  // a whole chunk in flight per wave when one round of waves covers the call
  const int ring = (dt == 1 && want <= stats_resident_blocks(1, 4)) ? 4 : 2;
  const dim3 grid((unsigned)(std::min<long long>(want, stats_resident_blocks(dt, ring)) +
                             gather_blocks(a)));
  if (dt == 1 && ring == 4) SV_LAUNCH((stats_kernel<1, 4>));
  else if (dt == 1) SV_LAUNCH((stats_kernel<1, 2>));
  else SV_LAUNCH((stats_kernel<0, 2>));
#undef SV_LAUNCH
  return hipGetLastError();
}

hipError_t launch_linear_finish(int dtype, const LinearArgs& a, hipStream_t st) {
  const dim3 rows((unsigned)a.B), block(kFinThreads);
  if (a.n_chunks == 1) {
    if (dtype == 1) linear_row_kernel<1><<<rows, block, 0, st>>>(a);
    else linear_row_kernel<0><<<rows, block, 0, st>>>(a);
    return hipGetLastError();
  }
  const long long units = (long long)a.B * a.n_chunks;
  hipError_t e;
  if (a.n_chunks <= 4) {
    const dim3 items((unsigned)units);
    if (dtype == 1) linear_decide_mass_kernel<1><<<items, block, 0, st>>>(a);
    else linear_decide_mass_kernel<0><<<items, block, 0, st>>>(a);
    e = hipGetLastError();
  } else {
    if (dtype == 1) linear_decide_kernel<1><<<rows, block, 0, st>>>(a);
    else linear_decide_kernel<0><<<rows, block, 0, st>>>(a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    const dim3 mgrid((unsigned)std::min<long long>(units, mass_resident_blocks(dtype == 1 ? 1 : 0)));
    if (a.B <= kMassRecCache) {
      if (dtype == 1) linear_mass_kernel<1, true><<<mgrid, block, 0, st>>>(a);
      else linear_mass_kernel<0, true><<<mgrid, block, 0, st>>>(a);
    } else {
      if (dtype == 1) linear_mass_kernel<1, false><<<mgrid, block, 0, st>>>(a);
      else linear_mass_kernel<0, false><<<mgrid, block, 0, st>>>(a);
    }
    e = hipGetLastError();
  }
  if (e != hipSuccess) return e;
  if (dtype == 1) linear_select_kernel<1><<<rows, dim3(64), 0, st>>>(a);
  else linear_select_kernel<0><<<rows, dim3(64), 0, st>>>(a);
  return hipGetLastError();
}

hipError_t launch_tree_finish(int dtype, const TreeArgs& a, hipStream_t st) {
  if (dtype == 1) tree_kernel<1><<<dim3((unsigned)a.B), dim3(kFinThreads), 0, st>>>(a);
  else tree_kernel<0><<<dim3((unsigned)a.B), dim3(kFinThreads), 0, st>>>(a);
  return hipGetLastError();
}

hipError_t launch_philox_words(uint64_t seed, uint64_t step, const uint32_t* row_ids,
                               int n_rows, int n_slots, uint32_t* out, hipStream_t st) {
  const long long n = (long long)n_rows * n_slots;
  const long long blocks = (n + kThreads - 1) / kThreads;
  philox_words_kernel<<<dim3((unsigned)blocks), dim3(kThreads), 0, st>>>(seed, step, row_ids,
                                                                         n_rows, n_slots, out);
  return hipGetLastError();
}

}  // namespace sv
