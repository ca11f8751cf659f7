// Pass 1 of the vocabulary-wide verify (linear and tree), gfx950.
//
// stats_kernel: a resident grid in which each wave reduces whole 8192-logit
// chunks of the logit rows (one HBM read of every logit, with non-temporal
// 16-byte loads in flight ahead of the reduction) into one Partial per (row,
// chunk): an integer log2 offset and a float64 sum of exponentials for a
// sampled row, the maximum and its first index for a greedy row.  Its first
// work items gather the logits at the draft tokens.
//
// Sources: the softmax statistics that the acceptance ratio and the draws
// need (kwkr.cn/news/620872 §2.3, §4.1; blog.lonae.com/posts/
// 2026-draft-model-kv-jDwzYp, formal-definition paragraph).
#include <hip/hip_ext.h>

#include <algorithm>

#include "sv_common.h"
#include "sv_internal.h"
#include "sv_pass.h"

namespace sv {

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

constexpr int kStatsCache = 1024;  // batch rows whose offsets/temperatures go to LDS
constexpr int kInnerCache = 512;   // trees whose inner-node masks go to LDS (compacted rows)

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

// As wave_find_batch_row for a uniform x, by a binary search of scalar loads
// (offsets non-decreasing): the loads are waited for on the scalar counter,
// so vector loads issued before them are not waited for with them.
__device__ __forceinline__ int scalar_find_batch_row(const int* off, int B, long long x, int add) {
  int lo = 0, hi = B;   // off[lo] + add lo <= x; keys at hi and above exceed x
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if ((long long)load_uniform_i32(off + mid) + (long long)add * mid <= x) lo = mid;
    else hi = mid;
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
// draft row i); tree, node j's token under its parent's target row at [j]
// and, with draft rows, under its parent's draft row at [B N + j].  Tokens
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
    if (a.rows_b) a.gath[n + it] = load_logit<DT>(a.rows_b, xr * V + tc);
  } else {
    const int b = cache ? lane_batch_row(s_off, a.B, it) : lane_batch_row(a.offsets, a.B, it);
    a.gath[it] = load_logit<DT>(a.rows_a, (it + b) * V + tc);
    a.gath[n + it] = load_logit<DT>(a.rows_b, it * V + tc);
  }
}

// The k-th set bit of m (whole waves; 0 if m has fewer than k + 1 bits).
__device__ __forceinline__ int wave_kth_bit(unsigned long long m, int k) {
  const int lane = threadIdx.x & 63;
  const bool set = ((m >> lane) & 1ull) != 0ull;
  const int rank = __popcll(m & ((1ull << lane) - 1ull));
  const unsigned long long hit = __ballot(set && rank == k);
  return hit ? __ffsll((long long)hit) - 1 : 0;
}

// RING = sub-segments in flight per wave: 2, or 4 (a whole chunk) with fewer
// resident waves; the launch takes the one whose grid ends in the fuller
// round.
//
// A tree's rows read here are those of the nodes that have children (their
// children are tested against them): the target rows and, with draft rows,
// the draft rows.  A leaf's target row is read only by a walk that stops at
// that leaf, which forms its statistics itself.  The rows are compacted when
// the trees' shapes fit in LDS: the units run over the used rows only (the
// target rows of each tree's inner nodes, then their draft rows), so that
// every wave gets an equal share of the work whatever the shapes.  Otherwise
// unused rows are skipped as they come.
template <int DT, int RING>
__global__ __launch_bounds__(kThreads) void stats_kernel(StatsArgs a) {
  __shared__ int s_i[kStatsCache + 1];
  __shared__ float s_f0[kStatsCache], s_f1[kStatsCache];
  __shared__ unsigned long long s_inner[kInnerCache];   // tree b: bit n set if node n has a child
  __shared__ int s_pt[kInnerCache + 1];   // used-row prefix (inner nodes per tree)
  __shared__ double s_scan[kWaves];

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
  uint32_t total = (uint32_t)a.n_rows * nc;   // < 2^31 (checked by the host)
  const uint32_t G = (gridDim.x - n_gblk) * kWaves;
  const uint32_t Gq = G / nc, Gr = G - Gq * nc;
  const long long rowbytes = (long long)V * SegLoad<DT>::ES;
  auto row_ptr = [&](uint32_t r) -> const char* {
    return r < a.n_a ? (const char*)a.rows_a + (long long)r * rowbytes
                     : (const char*)a.rows_b + ((long long)r - a.n_a) * rowbytes;
  };

  const bool cache = a.B <= kStatsCache;
  // Tree rows are read only for nodes with children.
  const bool tree_q = a.tree && a.rows_b;
  const bool compact = a.tree && a.B <= kInnerCache;

  uint32_t u = blk * kWaves + wave;
  uint32_t ur = u / nc, ch = u - ur * nc;   // ur: row in the order the units run

  SegLoad<DT> ring[RING];
  // The first chunk's loads go out before anything else, except for
  // compacted trees, whose row map needs the inner-node masks first.  Trees
  // skipped as they come issue them for row ur; an unused tree row is still
  // allocated, so reading it is harmless.
  if (a.vec_ok && u < total && !compact) {
#pragma unroll
    for (int r = 0; r < RING; ++r) ring[r].issue(row_ptr(ur), V, (int)ch * kChunk + r * kSubSpan);
  }
  if (cache) {
    for (int i = threadIdx.x; i <= a.B; i += kThreads) {
      if (a.tree) {
        if (i < a.B) {
          const int nn = a.n_nodes ? a.n_nodes[i] : a.N;
          s_i[i] = (nn >= 1 && nn <= a.N) ? nn : 0;   // a bad count: no row is read
          s_f0[i] = a.temp_a[i];
          s_f1[i] = a.temp_b[i];
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
  // Exclusive prefix over the trees of cnt(b) (two trees per thread) into pre.
  auto tree_prefix = [&](int* pre, auto cnt) {
    const int i0 = 2 * threadIdx.x;
    const int c0 = i0 < a.B ? cnt(i0) : 0, c1 = i0 + 1 < a.B ? cnt(i0 + 1) : 0;
    double tot;
    const int ex = (int)block_exclusive_scan<kWaves>((double)(c0 + c1), s_scan, &tot);
    if (i0 < a.B) pre[i0] = ex;
    if (i0 + 1 < a.B) pre[i0 + 1] = ex + c0;
    if (threadIdx.x == 0) pre[a.B] = (int)tot;
    __syncthreads();
  };
  uint32_t n_t = 0;   // compacted: used target rows (they come first)
  // The row of iteration row x (once the inner masks are known): the x-th
  // used target row, then the used draft rows.
  auto row_of = [&](uint32_t x) -> uint32_t {
    if (!compact) return x;
    const int N = a.N;
    if (x < n_t) {
      const int b = wave_find_batch_row(s_pt, a.B, (long long)x, 0);
      return (uint32_t)(b * N + wave_kth_bit(s_inner[b], (int)x - s_pt[b]));
    }
    const uint32_t y = x - n_t;   // the draft rows of the same nodes, in the same order
    const int b = wave_find_batch_row(s_pt, a.B, (long long)y, 0);
    return (uint32_t)a.n_a + (uint32_t)(b * N + wave_kth_bit(s_inner[b], (int)y - s_pt[b]));
  };
  if (compact) {
    // one wave per tree (a lane per node, N <= 64): the mask is the OR of the
    // lanes' parent bits; a wave's trees are taken 16 at a time, their
    // parents loaded together (clamped indices: no load behind a branch)
    const int N = a.N;
    constexpr int kMaskBatch = 16;
    const int c = lane < N ? lane : N - 1;
    for (int b0 = wave; b0 < a.B; b0 += kWaves * kMaskBatch) {
      int pv[kMaskBatch];
#pragma unroll
      for (int k = 0; k < kMaskBatch; ++k)
        pv[k] = a.parents[(long long)min(b0 + k * kWaves, a.B - 1) * N + c];
#pragma unroll
      for (int k = 0; k < kMaskBatch; ++k) {
        const int b = b0 + k * kWaves;
        const int bc = b < a.B ? b : a.B - 1;
        const int par = pv[k];
        const bool kid = b < a.B && lane > 0 && lane < s_i[bc] && par >= 0 && par < lane;
        const unsigned long long m = wave_or_u64(kid ? 1ull << par : 0ull);
        if (lane == 0 && b < a.B) s_inner[b] = m;
      }
    }
    __syncthreads();
  }
  if (compact) {
    tree_prefix(s_pt, [&](int b) { return __popcll(s_inner[b]); });
    n_t = (uint32_t)s_pt[a.B];
    total = (tree_q ? 2u * n_t : n_t) * nc;
  }
  if (u >= total) return;
  uint32_t row = row_of(ur);
  if (compact && a.vec_ok) {
#pragma unroll
    for (int r = 0; r < RING; ++r) ring[r].issue(row_ptr(row), V, (int)ch * kChunk + r * kSubSpan);
  }

  // Whether a row's partials are needed (always, for compacted rows): tree
  // rows past n_nodes are not, nor the rows of nodes without children.
  // Called by whole waves.
  auto row_used = [&](uint32_t r) -> bool {
    if (!a.tree || compact) return true;
    const bool is_q = r >= a.n_a;
    const uint32_t x = is_q ? r - (uint32_t)a.n_a : r;
    const uint32_t b = x / (uint32_t)a.N;
    const int node = (int)(x - b * (uint32_t)a.N);
    int nn = cache ? s_i[b] : (a.n_nodes ? a.n_nodes[b] : a.N);
    if (nn > a.N) nn = 0;
    if (node >= nn) return false;
    const int c = lane;
    const bool kid = c > node && c < nn && a.parents[(long long)b * a.N + c] == node;
    return __ballot(kid) != 0ull;
  };
  auto row_temp = [&](uint32_t r) -> float {
    if (a.tree) {
      const bool is_q = r >= a.n_a;
      const uint32_t b = (is_q ? r - (uint32_t)a.n_a : r) / (uint32_t)a.N;
      if (is_q) return cache ? s_f1[b] : a.temp_b[b];
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
    for (; u < total; u += G, advance(ur, ch)) {
      row = row_of(ur);
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

  // The wave's next unit whose row is used (u >= total: none), so that the
  // loads in flight always belong to a unit that is reduced.
  auto next_used = [&](uint32_t& uu, uint32_t& x, uint32_t& c, uint32_t& r) {
    do {
      uu += G;
      advance(x, c);
    } while (uu < total && !row_used(r = row_of(x)));
  };
  bool used = row_used(row);
  float T = used ? row_temp(row) : 0.0f;
  for (;;) {
    uint32_t u1 = u, ur1 = ur, ch1 = ch, row1 = row;
    next_used(u1, ur1, ch1, row1);
    const bool has1 = u1 < total;
    const bool used1 = has1;
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
    u = u1;
    ur = ur1;
    ch = ch1;
    row = row1;
    used = used1;
    T = T1;
  }
}
// Linear batches that one round of work items covers: a work item of four
// waves per (row, chunk), wave w reducing sub-segment w (2048 logits, all of
// its loads in flight at once), the four wave partials merged in LDS.
// Shorter waves than one chunk each spread the exponentials evenly over the
// SIMDs when there are few chunks per SIMD.
template <int DT>
__global__ __launch_bounds__(kThreads) void stats_kernel_by_chunk(StatsArgs a) {
  __shared__ int s_off[kStatsCache + 1];   // the gather's batch-row offsets
  __shared__ Partial s_part[kWaves];

  const int n_gblk = gather_blocks(a);
  if ((int)blockIdx.x < n_gblk) {
    gather_logits<DT>(a, s_off);
    return;
  }
  const uint32_t nc = (uint32_t)a.n_chunks;
  const uint32_t unit = blockIdx.x - n_gblk;
  const uint32_t r = unit / nc, c = unit - r * nc;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int V = a.V;
  const long long rowbytes = (long long)V * SegLoad<DT>::ES;
  const char* rowp = r < a.n_a ? (const char*)a.rows_a + (long long)r * rowbytes
                               : (const char*)a.rows_b + ((long long)r - a.n_a) * rowbytes;
  const int seg0 = (int)c * kChunk + wave * kSubSpan;
  SegLoad<DT> seg;
  if (a.vec_ok) seg.issue(rowp, V, seg0);
  // the row's temperature, its batch row found from the offsets (scalar
  // loads, done while the row's loads are in flight)
  const bool is_t = r < a.n_a;
  const int bb = is_t ? scalar_find_batch_row(a.offsets, a.B, (long long)r, 1)
                      : scalar_find_batch_row(a.offsets, a.B, (long long)r - a.n_a, 0);
  const float T = load_uniform_f32((is_t ? a.temp_a : a.temp_b) + bb);
  const bool ok = temp_ok(T);   // a bad temperature is reported by the finish pass
  const bool greedy = T == 0.0f;
  const float k2 = greedy ? 0.0f : log2e_over_t(T);
  LaneStats st{-__builtin_huge_valf(), seg0 + lane * SegLoad<DT>::EPV, 0.0};
  if (ok) {
    float v[kPerLane];
    if (a.vec_ok) seg.unpack(v);
    else seg_load_scalar<DT>(rowp, V, seg0, v);
    lane_fold<DT>(v, seg0, greedy, k2, st);
  }
  const Partial p = ok ? wave_combine(st, greedy) : Partial{0.0f, 0, 0.0};
  if (lane == 0) s_part[wave] = p;
  __syncthreads();
  if (threadIdx.x == 0) {
    Partial out = s_part[0];
    if (ok && greedy) {
      // the largest value, at its lowest index (the waves' ranges increase)
      for (int w = 1; w < kWaves; ++w)
        if (s_part[w].c > out.c) out = s_part[w];
    } else if (ok) {
      float C = s_part[0].c;
      for (int w = 1; w < kWaves; ++w) C = fmaxf(C, s_part[w].c);
      double sum = 0.0;
      if (C > -__builtin_huge_valf()) {
        for (int w = 0; w < kWaves; ++w)
          if (s_part[w].s != 0.0) sum += scale_pow2(s_part[w].s, s_part[w].c - C);
      }
      out = Partial{C, 0, sum};
    }
    a.part[(long long)r * nc + c] = out;
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

// The hardware 2^x of every probability the verify forms (diagnostic entry
// point): one element per thread.
__global__ __launch_bounds__(kThreads) void exp2_words_kernel(const float* x, float* y, int n) {
  const long long i = (long long)blockIdx.x * kThreads + threadIdx.x;
  if (i >= n) return;
  y[i] = exp2_hw(x[i]);
}

// ---------------------------------------------------------------------------
// Host launchers.

// Chunks per stats work item: one while a single round of work items fills
// the GPU (short critical path), two beyond (more loads in flight per item).
long long stats_items(long long n_rows, int n_chunks) {
  return n_rows * n_chunks * kPartsPerChunk;
}

static int stats_resident_blocks(int dt, int ring) {
  if (dt == 1)
    return ring == 4 ? resident_blocks(0, stats_kernel<1, 4>, kThreads)
                     : resident_blocks(1, stats_kernel<1, 2>, kThreads);
  return resident_blocks(2, stats_kernel<0, 2>, kThreads);
}

static int stats_by_chunk_resident_blocks(int dt) {
  return dt == 1 ? resident_blocks(5, stats_kernel_by_chunk<1>, kThreads)
                 : resident_blocks(6, stats_kernel_by_chunk<0>, kThreads);
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
  // linear batches that one round of (row, chunk) work items covers
  if (!a.tree && units <= stats_by_chunk_resident_blocks(dt)) {
    const dim3 grid((unsigned)(units + gather_blocks(a)));
    if (dt == 1) SV_LAUNCH((stats_kernel_by_chunk<1>));
    else SV_LAUNCH((stats_kernel_by_chunk<0>));
    return hipGetLastError();
  }
  const long long want = (units + kWaves - 1) / kWaves;
  // A whole chunk in flight per wave (RING 4, fewer resident waves) when its
  // grid covers the units in whole rounds at least as well as RING 2's: the
  // last round of a streaming grid runs with too few waves to fill HBM, so
  // the fuller last round wins (bimodal batch 121.5 -> 118.6 us, SAMPLED_WOR
  // trees 60.7 -> 59.0 us; one round of waves is always whole).
  auto round_fill = [&](int r) {
    const long long items = std::min<long long>(want, stats_resident_blocks(dt, r));
    const long long waves = items * kWaves;
    const long long rounds = (units + waves - 1) / waves;
    return (double)units / (double)(rounds * waves);
  };
  // Tree calls read the inner nodes' rows only, about a third of B N in
  // 4-wide trees, which the host does not see: they take the larger grid
  // (TOPK 64 x 64 nodes: 20.6 -> 19.1 us; SAMPLED_WOR level).
  const int ring = (dt == 1 && !a.tree && round_fill(4) >= round_fill(2)) ? 4 : 2;
  const dim3 grid((unsigned)(std::min<long long>(want, stats_resident_blocks(dt, ring)) +
                             gather_blocks(a)));
  if (dt == 1 && ring == 4) SV_LAUNCH((stats_kernel<1, 4>));
  else if (dt == 1) SV_LAUNCH((stats_kernel<1, 2>));
  else SV_LAUNCH((stats_kernel<0, 2>));
#undef SV_LAUNCH
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

hipError_t launch_exp2_words(const float* x, float* y, int n, hipStream_t st) {
  const long long blocks = ((long long)n + kThreads - 1) / kThreads;
  exp2_words_kernel<<<dim3((unsigned)blocks), dim3(kThreads), 0, st>>>(x, y, n);
  return hipGetLastError();
}

}  // namespace sv
