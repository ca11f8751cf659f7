// Vocabulary-wide verify kernels (linear and tree), gfx950.
//
// Linear verify, three launches per call:
//
//   stats_kernel        one work item per (logit row, pair of 8192-element
//                       chunks): coalesced 16-byte loads of both chunks are
//                       issued together, then each chunk is reduced to a
//                       Partial -- an offset and a sum of exponentials for a
//                       sampled row, the max and its first index for a
//                       greedy row.  This pass reads every logit of the call
//                       exactly once and is the HBM-bound part.
//
//   linear_mass_kernel  one work item per (batch row, chunk).  Every item
//                       merges the row's partials, redoes the row's
//                       acceptance decisions (identical arithmetic, so
//                       identical results in every item) and computes the
//                       mass of the stop distribution over its chunk:
//                       max(0, p - q) after a rejection, p for the bonus
//                       token.  Item 0 also stores the row's decision.
//
//   linear_select_kernel one work item per batch row: picks the chunk that
//                       holds u * R, recomputes that chunk's weights with the
//                       same code as the mass pass and returns the first index
//                       whose cumulative mass exceeds u * R, in vocabulary order.
//
// Tree verify, two launches: the same stats_kernel, then tree_kernel (one
// work item per tree): it walks the tree level by level with one lane per
// sibling, takes the stop node's chunk masses from its partials (minus the
// rejected siblings), and selects in one chunk.
//
// Work items never wait for one another: a kernel boundary is the only
// synchronisation, because device-scope fences and atomics are costly here.
// The mass and select passes accumulate each thread's 32 contiguous weights
// sequentially in float64 and combine threads with the same block scan, so
// chunk totals and in-chunk cumulative sums agree bit for bit.
//
// Sources: acceptance rule and first-reject stop (kwkr.cn/news/620872 §2.3,
// §4.1, §4.3; cf-1.com/news/5632551 §2.2); residual and bonus draws
// (blog.lonae.com/posts/2026-draft-model-kv-jDwzYp, formal-definition
// paragraph); greedy exact match (kwkr §4.3); tree walk over top-k siblings
// (kwkr §5.3; lonae tree-attention paragraphs).
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
// Pass 1: per-chunk statistics of every logit row.

template <int DT>
struct ChunkLoad {
  static constexpr int ES = DT ? 2 : 4;          // bytes per element
  static constexpr int EPV = 16 / ES;            // elements per 16-byte load
  static constexpr int NV = kPerThread / EPV;    // loads per thread per chunk
  uint4 raw[NV];

  // Thread t's vector j covers elements c0 + (j * 256 + t) * EPV + [0, EPV).
  __device__ __forceinline__ void issue(const char* rowp, int V, int c0) {
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      const int e0 = c0 + (j * kThreads + threadIdx.x) * EPV;
      if (e0 < V) raw[j] = *(const uint4*)(rowp + (long long)e0 * ES);
      else raw[j] = make_uint4(0xff80ff80u, 0xff80ff80u, 0xff80ff80u, 0xff80ff80u);
    }
  }

  __device__ __forceinline__ void unpack(int V, int c0, float v[kPerThread]) const {
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      const int e0 = c0 + (j * kThreads + threadIdx.x) * EPV;
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
      if (e0 >= V) {
#pragma unroll
        for (int k = 0; k < EPV; ++k) v[j * EPV + k] = -__builtin_huge_valf();
      }
    }
  }
};

template <int DT>
__device__ __forceinline__ void load_scalar(const char* rowp, int V, int c0, float v[kPerThread]) {
  constexpr int EPV = ChunkLoad<DT>::EPV;
  constexpr int NV = ChunkLoad<DT>::NV;
#pragma unroll
  for (int j = 0; j < NV; ++j) {
#pragma unroll
    for (int k = 0; k < EPV; ++k) {
      const int e = c0 + (j * kThreads + threadIdx.x) * EPV + k;
      v[j * EPV + k] = e < V ? load_logit<DT>(rowp, e) : -__builtin_huge_valf();
    }
  }
}

struct StatsShared {
  float redf[kWaves];
  double red[kWaves];
  unsigned long long red64[kWaves];
};

// Reduce one chunk held as this thread's 32 values (index order as loaded).
template <int DT>
__device__ __forceinline__ Partial chunk_partial(float v[kPerThread], int c0, float T,
                                                 StatsShared* sh) {
  constexpr int EPV = ChunkLoad<DT>::EPV;
  constexpr int NV = ChunkLoad<DT>::NV;
  const int tid = threadIdx.x;
  if (T == 0.0f) {
    // First maximum: the thread's elements are in increasing index order.
    float bv = -__builtin_huge_valf();
    int bi = c0 + tid * EPV;
#pragma unroll
    for (int j = 0; j < NV; ++j) {
#pragma unroll
      for (int k = 0; k < EPV; ++k) {
        const float x = v[j * EPV + k];
        const bool gt = x > bv;
        bv = gt ? x : bv;
        bi = gt ? c0 + (j * kThreads + tid) * EPV + k : bi;
      }
    }
    const unsigned long long key =
        ((unsigned long long)float_order_key(bv) << 32) | (0xffffffffu - (uint32_t)bi);
    const unsigned long long best = block_max_u64(key, sh->red64);
    return Partial{float_from_order_key((uint32_t)(best >> 32)),
                   (int)(0xffffffffu - (uint32_t)best), 0.0};
  }
  // Sampled row: thread-local offset from the thread's own maximum, then a
  // pairwise sum of 2^(x k - c); threads are merged exactly in float64.
  const float k2 = log2e_over_t(T);
  float m = -__builtin_huge_valf();
#pragma unroll
  for (int e = 0; e < kPerThread; ++e) m = fmaxf(m, v[e]);
  const bool any = m > -__builtin_huge_valf();
  const float ct = any ? m * k2 : 0.0f;
#pragma unroll
  for (int e = 0; e < kPerThread; ++e) v[e] = exp2_hw(fmaf(v[e], k2, -ct));
#pragma unroll
  for (int w = kPerThread / 2; w >= 1; w >>= 1) {
#pragma unroll
    for (int e = 0; e < w; ++e) v[e] += v[e + w];
  }
  const float s = v[0];
  const float C = block_max(any ? ct : -__builtin_huge_valf(), sh->redf);
  const double contrib = (any && s > 0.0f) ? (double)s * exp2((double)ct - (double)C) : 0.0;
  const double S = block_sum(contrib, sh->red);
  return Partial{C, 0, S};
}

template <int DT>
__global__ __launch_bounds__(kThreads) void stats_kernel(StatsArgs a) {
  __shared__ int s_best;
  __shared__ StatsShared sh;

  const int tid = threadIdx.x;
  const long long item = blockIdx.x;
  const int n_tiles = (a.n_chunks + 1) >> 1;
  const long long row = item / n_tiles;
  const int tile = (int)(item - row * n_tiles);
  const int ca = 2 * tile, cb = ca + 1;
  const bool has_b = cb < a.n_chunks;
  const int V = a.V;
  const long long rowbytes = (long long)V * ChunkLoad<DT>::ES;
  const char* rowp = row < a.n_a ? (const char*)a.rows_a + row * rowbytes
                                 : (const char*)a.rows_b + (row - a.n_a) * rowbytes;

  // Issue both chunks' loads before looking up the row's temperature.
  ChunkLoad<DT> la, lb;
  if (a.vec_ok) {
    la.issue(rowp, V, ca * kChunk);
    if (has_b) lb.issue(rowp, V, cb * kChunk);
  }

  float T;
  if (a.tree) {
    const int b = (int)(row / a.N);
    const int node = (int)(row - (long long)b * a.N);
    const int nn = a.n_nodes ? a.n_nodes[b] : a.N;
    if (node >= nn) return;               // unused node row: never read
    T = a.temp_a[b];
  } else if (row < a.n_a) {
    T = a.temp_a[find_batch_row(a.offsets, a.B, row, 1, &s_best)];
  } else {
    T = a.temp_b[find_batch_row(a.offsets, a.B, row - a.n_a, 0, &s_best)];
  }

  Partial* out = a.part + row * a.n_chunks;
  if (!temp_ok(T)) {                      // the finish pass reports the row
    if (tid == 0) {
      out[ca] = Partial{0.0f, 0, 0.0};
      if (has_b) out[cb] = Partial{0.0f, 0, 0.0};
    }
    return;
  }

  float v[kPerThread];
  if (a.vec_ok) la.unpack(V, ca * kChunk, v);
  else load_scalar<DT>(rowp, V, ca * kChunk, v);
  const Partial pa = chunk_partial<DT>(v, ca * kChunk, T, &sh);
  if (tid == 0) out[ca] = pa;
  if (has_b) {
    if (a.vec_ok) lb.unpack(V, cb * kChunk, v);
    else load_scalar<DT>(rowp, V, cb * kChunk, v);
    const Partial pb = chunk_partial<DT>(v, cb * kChunk, T, &sh);
    if (tid == 0) out[cb] = pb;
  }
}

// ---------------------------------------------------------------------------
// Shared pieces of the finish passes.

struct RowStats {
  float c;     // log2 offset (sampled) or max logit (greedy)
  int amax;    // first argmax (greedy)
  double s;    // sum of 2^(x k - c) (sampled)
};

// Merge a row's chunk partials; returns false when the row has no finite maximum.
__device__ bool merge_row(const Partial* __restrict__ p, int n_chunks, bool greedy,
                          RowStats* out) {
  if (greedy) {
    float m = -__builtin_huge_valf();
    int am = 0;
    for (int j = 0; j < n_chunks; ++j) {
      const Partial q = p[j];
      if (j == 0 || q.c > m) {  // strict: ties keep the earlier chunk (lower index)
        m = q.c;
        am = q.amax;
      }
    }
    out->c = m;
    out->amax = am;
    out->s = 0.0;
    return m > -__builtin_huge_valf() && m < __builtin_huge_valf();
  }
  float C = -__builtin_huge_valf();
  for (int j = 0; j < n_chunks; ++j) C = fmaxf(C, p[j].c);
  double S = 0.0;
  for (int j = 0; j < n_chunks; ++j) {
    const Partial q = p[j];
    if (q.s > 0.0) S += q.s * exp2((double)q.c - (double)C);
  }
  out->c = C;
  out->amax = 0;
  out->s = S;
  const bool finite_c = C > -__builtin_huge_valf() && C < __builtin_huge_valf();
  return finite_c && S > 0.0 && S < __builtin_huge_val();
}

// Probability of token `tok` under a merged row, in float64.
__device__ __forceinline__ double row_prob(const RowStats& r, bool greedy, float k2, float x,
                                           int tok) {
  if (greedy) return tok == r.amax ? 1.0 : 0.0;
  return exp2((double)x * (double)k2 - (double)r.c) / r.s;
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

// This thread's 32 contiguous weights of chunk `chunk` (zero past V and for
// the bits set in `mask`).  The mass and select passes both call this.
template <int DT>
__device__ __forceinline__ void stop_weights(const StopDist& d, int V, int chunk, int vec_ok,
                                             uint32_t mask, float w[kPerThread]) {
  constexpr int ES = DT ? 2 : 4;
  constexpr int EPV = 16 / ES;
  const int e0 = chunk * kChunk + threadIdx.x * kPerThread;
  float xp[kPerThread], xq[kPerThread];
  const bool need_q = d.residual && !d.q_greedy;
  if (vec_ok && e0 + kPerThread <= V) {
    const uint4* pp = (const uint4*)((const char*)d.prow + (long long)e0 * ES);
    const uint4* qp = (const uint4*)((const char*)d.qrow + (long long)e0 * ES);
#pragma unroll
    for (int j = 0; j < kPerThread / EPV; ++j) {
      const uint4 r = pp[j];
      uint4 s = make_uint4(0, 0, 0, 0);
      if (need_q) s = qp[j];
      const uint32_t rw[4] = {r.x, r.y, r.z, r.w};
      const uint32_t sw[4] = {s.x, s.y, s.z, s.w};
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        if (DT == 1) {
          xp[j * 8 + 2 * h] = bf16_lo(rw[h]);
          xp[j * 8 + 2 * h + 1] = bf16_hi(rw[h]);
          xq[j * 8 + 2 * h] = bf16_lo(sw[h]);
          xq[j * 8 + 2 * h + 1] = bf16_hi(sw[h]);
        } else {
          xp[j * 4 + h] = __uint_as_float(rw[h]);
          xq[j * 4 + h] = __uint_as_float(sw[h]);
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
#pragma unroll
  for (int e = 0; e < kPerThread; ++e) {
    const int idx = e0 + e;
    float p = exp2_hw(fmaf(xp[e], d.p_k, -d.p_c)) * d.p_inv_s;
    if (d.residual) {
      const float q = d.q_greedy ? (idx == d.q_amax ? 1.0f : 0.0f)
                                 : exp2_hw(fmaf(xq[e], d.q_k, -d.q_c)) * d.q_inv_s;
      p = fmaxf(p - q, 0.0f);
    }
    if (idx >= V || ((mask >> e) & 1u)) p = 0.0f;
    w[e] = p;
  }
}

template <int DT>
__device__ double chunk_mass(const StopDist& d, int V, int chunk, int vec_ok, uint32_t mask,
                             double* s_scan) {
  float w[kPerThread];
  stop_weights<DT>(d, V, chunk, vec_ok, mask, w);
  double acc = 0.0;
#pragma unroll
  for (int e = 0; e < kPerThread; ++e) acc += (double)w[e];
  double total;
  block_exclusive_scan(acc, s_scan, &total);
  return total;
}

// First index of chunk `chunk` whose cumulative mass (starting at `base`)
// exceeds `target`; if rounding leaves it uncrossed, the last index with
// positive weight; if the chunk has none, its first index.
template <int DT>
__device__ int chunk_select(const StopDist& d, int V, int chunk, int vec_ok, uint32_t mask,
                            double base, double target, double* s_scan, int* s_misc) {
  float w[kPerThread];
  stop_weights<DT>(d, V, chunk, vec_ok, mask, w);
  double acc = 0.0;
#pragma unroll
  for (int e = 0; e < kPerThread; ++e) acc += (double)w[e];
  double total;
  const double excl = block_exclusive_scan(acc, s_scan, &total);
  const int e0 = chunk * kChunk + threadIdx.x * kPerThread;
  int found = 0x7fffffff, lastp = -1;
  double run = base + excl;
#pragma unroll
  for (int e = 0; e < kPerThread; ++e) {
    run += (double)w[e];
    if (found == 0x7fffffff && run > target && w[e] > 0.0f) found = e0 + e;
    if (w[e] > 0.0f) lastp = e0 + e;
  }
  if (threadIdx.x == 0) {
    s_misc[0] = 0x7fffffff;
    s_misc[1] = -1;
  }
  __syncthreads();
  if (found != 0x7fffffff) atomicMin(&s_misc[0], found);
  if (lastp >= 0) atomicMax(&s_misc[1], lastp);
  __syncthreads();
  const int k = s_misc[0], last = s_misc[1];
  __syncthreads();
  if (k != 0x7fffffff) return k;
  return last >= 0 ? last : chunk * kChunk;
}

// Thread 0 finds the chunk holding u * R (R = the sum of the chunk masses,
// in chunk order) and the mass before it.
__device__ void choose_chunk(const double* s_mass, int n_chunks, double u, int* s_jc,
                             double* s_base, double* s_t) {
  if (threadIdx.x == 0) {
    double R = 0.0;
    for (int j = 0; j < n_chunks; ++j) R += s_mass[j];
    const double t = u * R;
    double cum = 0.0, base = 0.0;
    int jc = -1;
    for (int j = 0; j < n_chunks; ++j) {
      const double nxt = cum + s_mass[j];
      if (nxt > t && s_mass[j] > 0.0) {
        jc = j;
        base = cum;
        break;
      }
      cum = nxt;
    }
    if (jc < 0) {  // rounding left u * R uncrossed: last chunk with mass
      jc = 0;
      for (int j = n_chunks - 1; j >= 0; --j) {
        if (s_mass[j] > 0.0) {
          jc = j;
          break;
        }
      }
      base = 0.0;
      for (int j = 0; j < jc; ++j) base += s_mass[j];
    }
    *s_jc = jc;
    *s_base = base;
    *s_t = t;
  }
  __syncthreads();
}

// ---------------------------------------------------------------------------
// Linear verify, pass 2: decisions and stop-distribution chunk masses.

constexpr int kKindReject = 0, kKindBonus = 1, kKindGreedy = 2, kKindError = 3,
              kKindBadShape = 4;

template <int DT>
__global__ __launch_bounds__(kThreads) void linear_mass_kernel(LinearArgs a) {
  __shared__ RowStats s_rows[2 * kMaxGamma + 1];
  __shared__ double s_p[kMaxGamma], s_q[kMaxGamma];
  __shared__ int s_flags, s_nacc;
  __shared__ double s_scan[kWaves];

  const int tid = threadIdx.x;
  const int n_chunks = a.n_chunks;
  const int b = blockIdx.x / n_chunks;
  const int c = blockIdx.x - b * n_chunks;
  const int V = a.V;
  LinRecord* rec = a.rec + b;

  const int o0 = a.off[b], o1 = a.off[b + 1];
  const int g = o1 - o0;
  const float Tt = a.temp_t[b], Td = a.temp_d[b];
  int err = 0;
  if (o0 < 0 || o1 < o0 || o1 > a.total_draft || g > kMaxGamma) err = kRowBadShape;
  else if (!temp_ok(Tt) || !temp_ok(Td)) err = kRowBadTemp;
  if (err) {
    if (c == 0 && tid == 0) {
      LinRecord r{};
      r.kind = err == kRowBadShape ? kKindBadShape : kKindError;
      r.flags = err;
      r.o0 = o0;
      r.g = g;
      *rec = r;
    }
    return;
  }
  const long long tr0 = (long long)o0 + b;  // first target row of b
  const bool gt = Tt == 0.0f, gd = Td == 0.0f;
  const float kt = gt ? 0.0f : log2e_over_t(Tt);
  const float kd = gd ? 0.0f : log2e_over_t(Td);

  if (tid == 0) s_flags = 0;
  __syncthreads();
  const int nr = 2 * g + 1;
  if (tid < nr) {
    const bool is_t = tid <= g;
    const long long row = is_t ? tr0 + tid : a.n_target_rows + o0 + (tid - g - 1);
    RowStats rs;
    if (!merge_row(a.part + row * n_chunks, n_chunks, is_t ? gt : gd, &rs))
      atomicOr(&s_flags, kRowNonFinite);
    s_rows[tid] = rs;
  }
  __syncthreads();

  if (tid < 64) {
    const int i = tid;
    const bool valid = i < g;
    bool reject = false;
    if (valid) {
      int tok = a.tokens[o0 + i];
      if (tok < 0 || tok >= V) {
        atomicOr(&s_flags, kRowBadToken);
        tok = 0;
      }
      const float x = load_logit<DT>(a.target, (tr0 + i) * (long long)V + tok);
      const float y = load_logit<DT>(a.draft, ((long long)o0 + i) * V + tok);
      const double p = row_prob(s_rows[i], gt, kt, x, tok);
      const double q = row_prob(s_rows[g + 1 + i], gd, kd, y, tok);
      double r;
      if (q > 0.0) {
        r = p / q;
      } else {
        atomicOr(&s_flags, kRowWarnQZero);
        r = p > 0.0 ? __builtin_huge_val() : 0.0;
      }
      const uint32_t rid = a.row_ids ? a.row_ids[b] : (uint32_t)b;
      const double u = word_to_uniform(verify_words(a.seed, a.step, rid, (uint32_t)(i + 1)).x);
      reject = !(u < r);
      s_p[i] = p;
      s_q[i] = q;
    }
    const unsigned long long rej = __ballot(reject);
    if (tid == 0) s_nacc = rej ? (__ffsll((long long)rej) - 1) : g;
  }
  __syncthreads();
  const int flags = s_flags;
  const int n_acc = s_nacc;

  if (flags & kRowErrorMask) {
    if (c == 0 && tid == 0) {
      LinRecord r{};
      r.kind = kKindError;
      r.flags = flags & kRowErrorMask;
      r.o0 = o0;
      r.g = g;
      *rec = r;
    }
    return;
  }
  if (c == 0) {
    if (a.p_at) for (int i = tid; i < g; i += kThreads) a.p_at[o0 + i] = (float)s_p[i];
    if (a.q_at) for (int i = tid; i < g; i += kThreads) a.q_at[o0 + i] = (float)s_q[i];
  }
  if (gt) {
    // greedy target: the draw is the argmax of target row n_acc (no randoms)
    if (c == 0 && tid == 0) {
      LinRecord r{};
      r.kind = kKindGreedy;
      r.flags = flags;
      r.n_acc = n_acc;
      r.token = s_rows[n_acc].amax;
      r.o0 = o0;
      r.g = g;
      *rec = r;
    }
    return;
  }

  const int pos = n_acc;
  StopDist d;
  d.prow = (const char*)a.target + (tr0 + pos) * (long long)V * (DT ? 2 : 4);
  d.residual = pos < g;
  d.qrow = d.residual ? (const char*)a.draft + ((long long)o0 + pos) * V * (DT ? 2 : 4) : d.prow;
  d.p_k = kt;
  d.p_c = s_rows[pos].c;
  d.p_inv_s = (float)(1.0 / s_rows[pos].s);
  d.q_greedy = d.residual ? gd : 0;
  d.q_amax = d.residual ? s_rows[g + 1 + pos].amax : 0;
  d.q_k = d.residual ? kd : 0.0f;
  d.q_c = d.residual ? s_rows[g + 1 + pos].c : 0.0f;
  d.q_inv_s = (d.residual && !gd) ? (float)(1.0 / s_rows[g + 1 + pos].s) : 0.0f;

  const double m = chunk_mass<DT>(d, V, c, a.vec_ok, 0u, s_scan);
  if (tid == 0) a.mass[(long long)b * n_chunks + c] = m;
  if (c == 0 && tid == 0) {
    LinRecord r{};
    r.kind = d.residual ? kKindReject : kKindBonus;
    r.flags = flags;
    r.n_acc = n_acc;
    r.o0 = o0;
    r.g = g;
    r.q_greedy = d.q_greedy;
    r.q_amax = d.q_amax;
    r.p_c = d.p_c;
    r.p_inv_s = d.p_inv_s;
    r.q_c = d.q_c;
    r.q_inv_s = d.q_inv_s;
    *rec = r;
  }
}

// Linear verify, pass 3: the draw and the outputs.
template <int DT>
__global__ __launch_bounds__(kThreads) void linear_select_kernel(LinearArgs a) {
  __shared__ LinRecord s_rec;
  __shared__ double s_mass[kMaxChunks];
  __shared__ double s_scan[kWaves];
  __shared__ int s_misc[2];
  __shared__ int s_jc;
  __shared__ double s_base, s_t;

  const int tid = threadIdx.x;
  const int b = blockIdx.x;
  const int n_chunks = a.n_chunks;
  const int V = a.V;
  if (tid == 0) s_rec = a.rec[b];
  if (tid < n_chunks) s_mass[tid] = a.mass[(long long)b * n_chunks + tid];
  const float Tt = a.temp_t[b], Td = a.temp_d[b];
  __syncthreads();
  const LinRecord r = s_rec;
  const int o0 = r.o0, g = r.g;
  const long long tr0 = (long long)o0 + b;

  if (r.kind == kKindBadShape || r.kind == kKindError) {
    if (r.kind == kKindError)
      for (int i = tid; i <= g; i += kThreads) a.out_tokens[tr0 + i] = -1;
    if (tid == 0) {
      a.num_accepted[b] = -1;
      if (a.row_status) a.row_status[b] = r.flags;
    }
    return;
  }
  const int n_acc = r.n_acc;
  int token = r.token;
  int warn = r.flags;
  if (r.kind != kKindGreedy) {
    StopDist d;
    d.prow = (const char*)a.target + (tr0 + n_acc) * (long long)V * (DT ? 2 : 4);
    d.residual = r.kind == kKindReject;
    d.qrow = d.residual ? (const char*)a.draft + ((long long)o0 + n_acc) * V * (DT ? 2 : 4)
                        : d.prow;
    d.p_k = log2e_over_t(Tt);
    d.p_c = r.p_c;
    d.p_inv_s = r.p_inv_s;
    d.q_greedy = r.q_greedy;
    d.q_amax = r.q_amax;
    d.q_k = (d.residual && Td > 0.0f) ? log2e_over_t(Td) : 0.0f;
    d.q_c = r.q_c;
    d.q_inv_s = r.q_inv_s;
    double R = 0.0;
    for (int j = 0; j < n_chunks; ++j) R += s_mass[j];
    if (!(R > 0.0)) {
      // zero residual mass (rounding only): draw from p at this position
      warn |= kRowWarnRZero;
      d.residual = 0;
      for (int j = 0; j < n_chunks; ++j) {
        const double mj = chunk_mass<DT>(d, V, j, a.vec_ok, 0u, s_scan);
        if (tid == 0) s_mass[j] = mj;
      }
      __syncthreads();
    }
    const uint32_t rid = a.row_ids ? a.row_ids[b] : (uint32_t)b;
    const double u = word_to_uniform(verify_words(a.seed, a.step, rid, (uint32_t)n_acc).y);
    choose_chunk(s_mass, n_chunks, u, &s_jc, &s_base, &s_t);
    token = chunk_select<DT>(d, V, s_jc, a.vec_ok, 0u, s_base, s_t, s_scan, s_misc);
  }
  for (int i = tid; i <= g; i += kThreads)
    a.out_tokens[tr0 + i] = i < n_acc ? a.tokens[o0 + i] : (i == n_acc ? token : -1);
  if (tid == 0) {
    a.num_accepted[b] = n_acc;
    if (a.row_status) a.row_status[b] = warn & ~kRowErrorMask;
  }
}

// ---------------------------------------------------------------------------
// Tree verify (TOPK): one work item per tree.

constexpr int kTreePartCache = 1024;   // partials kept in LDS when nn * n_chunks fits

template <int DT>
__global__ __launch_bounds__(kThreads) void tree_kernel(TreeArgs a) {
  __shared__ RowStats s_rows[kMaxNodes];
  __shared__ int s_par[kMaxNodes], s_tok[kMaxNodes], s_path[kMaxNodes];
  __shared__ double s_pn[kMaxNodes], s_u[kMaxNodes];
  __shared__ int s_flags, s_stop, s_depth;
  __shared__ unsigned long long s_removed;   // node bits of the rejected siblings
  __shared__ Partial s_part[kTreePartCache];
  __shared__ double s_scan[kWaves];
  __shared__ double s_mass[kMaxChunks];
  __shared__ int s_misc[2];
  __shared__ int s_jc;
  __shared__ double s_base, s_t;

  const int tid = threadIdx.x;
  const int n_chunks = a.n_chunks;
  const int b = blockIdx.x;
  const int V = a.V, N = a.N;
  const int nn = a.n_nodes ? a.n_nodes[b] : N;
  const float T = a.temp[b];
  const long long rb = (long long)b * N;

  if (tid == 0) s_flags = 0;
  __syncthreads();
  int err0 = 0;
  if (nn < 1 || nn > N) err0 = kRowBadShape;
  else if (!temp_ok(T)) err0 = kRowBadTemp;
  if (!err0 && tid < nn) {
    int par = -1, tok = 0;
    if (tid > 0) {
      par = a.parents[rb + tid];
      tok = a.tokens[rb + tid];
      if (par < 0 || par >= tid) atomicOr(&s_flags, kRowBadShape);
      if (tok < 0 || tok >= V) atomicOr(&s_flags, kRowBadToken);
    }
    s_par[tid] = par;
    s_tok[tid] = tok;
  }
  const bool greedy = T == 0.0f;
  const float k2 = (greedy || err0) ? 0.0f : log2e_over_t(T);
  const bool cache = !err0 && nn * n_chunks <= kTreePartCache;
  if (cache) {
    for (int i = tid; i < nn * n_chunks; i += kThreads) s_part[i] = a.part[rb * n_chunks + i];
  }
  __syncthreads();
  if (!err0 && tid < nn) {
    RowStats rs;
    const Partial* pp = cache ? s_part + tid * n_chunks : a.part + (rb + tid) * n_chunks;
    if (!merge_row(pp, n_chunks, greedy, &rs)) atomicOr(&s_flags, kRowNonFinite);
    s_rows[tid] = rs;
  }
  __syncthreads();
  const int err = err0 | (s_flags & kRowErrorMask);
  if (err) {
    for (int i = tid; i < N; i += kThreads) {
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

  const uint32_t rid = a.row_ids ? a.row_ids[b] : (uint32_t)b;
  if (tid > 0 && tid < nn) {
    const int par = s_par[tid], tok = s_tok[tid];
    const float x = load_logit<DT>(a.target, (rb + par) * (long long)V + tok);
    s_pn[tid] = row_prob(s_rows[par], greedy, k2, x, tok);
    s_u[tid] = word_to_uniform(verify_words(a.seed, a.step, rid, (uint32_t)tid).x);
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
      double incl = mass;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const double y = __shfl_up(incl, o, 64);
        if (i >= o) incl += y;
      }
      double excl = __shfl_up(incl, 1, 64);
      if (i == 0) excl = 0.0;
      const double denom = 1.0 - excl;
      const double ratio = (child && !dup && denom > 0.0) ? s_pn[i] / denom : 0.0;
      const unsigned long long acc = __ballot(child && s_u[i] < ratio);
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
    // chunk masses of p at the stop node from its partials, minus the
    // rejected siblings' probabilities
    if (tid < n_chunks) {
      const Partial q = cache ? s_part[stop * n_chunks + tid] : a.part[(rb + stop) * n_chunks + tid];
      double m = q.s > 0.0 ? q.s * exp2((double)q.c - (double)st.c) / st.s : 0.0;
      unsigned long long rm = removed;
      const int lo = tid * kChunk, hi = lo + kChunk;
      while (rm) {
        const int j = __ffsll((long long)rm) - 1;
        rm &= rm - 1ull;
        if (s_tok[j] >= lo && s_tok[j] < hi) m -= s_pn[j];
      }
      s_mass[tid] = m > 0.0 ? m : 0.0;
    }
    __syncthreads();
    double R = 0.0;
    for (int j = 0; j < n_chunks; ++j) R += s_mass[j];
    bool masked = removed != 0ull;
    if (!(R > 0.0)) {
      // every sibling's token took the whole mass (rounding only): draw from p
      warn |= kRowWarnRZero;
      masked = false;
      if (tid < n_chunks) {
        const Partial q = cache ? s_part[stop * n_chunks + tid] : a.part[(rb + stop) * n_chunks + tid];
        s_mass[tid] = q.s > 0.0 ? q.s * exp2((double)q.c - (double)st.c) / st.s : 0.0;
      }
      __syncthreads();
    }
    StopDist d;
    d.prow = (const char*)a.target + (rb + stop) * (long long)V * (DT ? 2 : 4);
    d.qrow = d.prow;
    d.residual = 0;
    d.p_k = k2;
    d.p_c = st.c;
    d.p_inv_s = (float)(1.0 / st.s);
    d.q_greedy = 0;
    d.q_amax = 0;
    d.q_k = d.q_c = d.q_inv_s = 0.0f;
    const double u = word_to_uniform(verify_words(a.seed, a.step, rid, (uint32_t)stop).y);
    choose_chunk(s_mass, n_chunks, u, &s_jc, &s_base, &s_t);
    const int jc = s_jc;
    // bits of this thread's 32 elements that belong to rejected siblings
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
    token = chunk_select<DT>(d, V, jc, a.vec_ok, mk, s_base, s_t, s_scan, s_misc);
  }

  for (int i = tid; i < N; i += kThreads) {
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

long long stats_items(long long n_rows, int n_chunks) { return n_rows * ((n_chunks + 1) / 2); }

hipError_t launch_stats(int dtype, const StatsArgs& a, hipStream_t st) {
  const long long n = stats_items(a.n_rows, a.n_chunks);
  if (dtype == 1) stats_kernel<1><<<dim3((unsigned)n), dim3(kThreads), 0, st>>>(a);
  else stats_kernel<0><<<dim3((unsigned)n), dim3(kThreads), 0, st>>>(a);
  return hipGetLastError();
}

hipError_t launch_linear_finish(int dtype, const LinearArgs& a, hipStream_t st) {
  const unsigned n2 = (unsigned)((long long)a.B * a.n_chunks);
  if (dtype == 1) linear_mass_kernel<1><<<dim3(n2), dim3(kThreads), 0, st>>>(a);
  else linear_mass_kernel<0><<<dim3(n2), dim3(kThreads), 0, st>>>(a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (dtype == 1) linear_select_kernel<1><<<dim3((unsigned)a.B), dim3(kThreads), 0, st>>>(a);
  else linear_select_kernel<0><<<dim3((unsigned)a.B), dim3(kThreads), 0, st>>>(a);
  return hipGetLastError();
}

hipError_t launch_tree_finish(int dtype, const TreeArgs& a, hipStream_t st) {
  if (dtype == 1) tree_kernel<1><<<dim3((unsigned)a.B), dim3(kThreads), 0, st>>>(a);
  else tree_kernel<0><<<dim3((unsigned)a.B), dim3(kThreads), 0, st>>>(a);
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
