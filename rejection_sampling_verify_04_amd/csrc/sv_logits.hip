// Vocabulary-wide verify kernels (linear and tree), gfx950.
//
// Linear verify, three launches per call:
//
//   stats_kernel        one work item per (logit row, 1 or 2 chunks of 8192
//                       elements); each wave reduces its own 2048 elements
//                       with coalesced 16-byte loads into a Partial -- an
//                       offset and a sum of exponentials for a sampled row,
//                       the max and its first index for a greedy row.  This
//                       pass reads every logit of the call exactly once and
//                       is the HBM-bound part.
//
//   linear_mass_kernel  one 1024-thread work item per (batch row, chunk).
//                       Every item merges the row's partials (one wave per
//                       logit row), redoes the row's acceptance decisions
//                       (identical arithmetic, so identical results in every
//                       item) and computes the mass of the stop distribution
//                       over its chunk: max(0, p - q) after a rejection, p
//                       for the bonus token.  Item 0 stores the row's
//                       decision and the accepted tokens.
//
//   linear_select_kernel one 1024-thread work item per batch row: picks the
//                       chunk that holds u * R, recomputes that chunk's
//                       weights with the same code as the mass pass and
//                       returns the first index whose cumulative mass exceeds
//                       u * R, in vocabulary order.
//
// Tree verify, two launches: the same stats_kernel, then tree_kernel (one
// 1024-thread work item per tree): it walks the tree level by level with one
// lane per sibling, takes the stop node's chunk masses from its partials
// (minus the rejected siblings), and selects in one chunk.
//
// Work items never wait for one another: a kernel boundary is the only
// synchronisation, because device-scope fences and atomics are costly here.
// The mass and select passes accumulate each thread's 8 contiguous weights
// sequentially in float64 and combine threads with the same block scan, so
// chunk totals and in-chunk cumulative sums agree bit for bit.
//
// Sources: acceptance rule and first-reject stop (kwkr.cn/news/620872 §2.3,
// §4.1, §4.3; cf-1.com/news/5632551 §2.2); residual and bonus draws
// (blog.lonae.com/posts/2026-draft-model-kv-jDwzYp, formal-definition
// paragraph); greedy exact match (kwkr §4.3); tree walk over top-k siblings
// (kwkr §5.3; lonae tree-attention paragraphs).
#include <hip/hip_ext.h>

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
// Pass 1: per-wave statistics of every logit row.

// One wave's 2048-element segment: lane l's vector j covers elements
// seg0 + (j * 64 + l) * EPV + [0, EPV), so each load instruction of the wave
// reads 1 KB of consecutive bytes.
template <int DT>
struct SegLoad {
  static constexpr int ES = DT ? 2 : 4;          // bytes per element
  static constexpr int EPV = 16 / ES;            // elements per 16-byte load
  static constexpr int NV = kPerLane / EPV;      // loads per lane per segment
  uint4 raw[NV];

  __device__ __forceinline__ void issue(const char* rowp, int V, int seg0) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      const int e0 = seg0 + (j * 64 + lane) * EPV;
      if (e0 < V) raw[j] = *(const uint4*)(rowp + (long long)e0 * ES);
      else raw[j] = make_uint4(0xff80ff80u, 0xff80ff80u, 0xff80ff80u, 0xff80ff80u);
    }
  }

  __device__ __forceinline__ void unpack(int V, int seg0, float v[kPerLane]) const {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      const int e0 = seg0 + (j * 64 + lane) * EPV;
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

// Reduce one wave's segment (this lane's 32 values, index order as loaded).
template <int DT>
__device__ __forceinline__ Partial seg_partial(float v[kPerLane], int seg0, float T) {
  constexpr int EPV = SegLoad<DT>::EPV;
  constexpr int NV = SegLoad<DT>::NV;
  const int lane = threadIdx.x & 63;
  if (T == 0.0f) {
    // First maximum: the lane's elements are in increasing index order.
    float bv = -__builtin_huge_valf();
    int bi = seg0 + lane * EPV;
#pragma unroll
    for (int j = 0; j < NV; ++j) {
#pragma unroll
      for (int k = 0; k < EPV; ++k) {
        const float x = v[j * EPV + k];
        const bool gt = x > bv;
        bv = gt ? x : bv;
        bi = gt ? seg0 + (j * 64 + lane) * EPV + k : bi;
      }
    }
    const unsigned long long key =
        ((unsigned long long)float_order_key(bv) << 32) | (0xffffffffu - (uint32_t)bi);
    const unsigned long long best = wave_max_u64(key);
    return Partial{float_from_order_key((uint32_t)(best >> 32)),
                   (int)(0xffffffffu - (uint32_t)best), 0.0};
  }
  // Sampled row: one offset for the wave, c = fl(max * k), then a pairwise
  // sum of 2^(x k - c) per lane and a float64 sum over the lanes.
  const float k2 = log2e_over_t(T);
  float m = -__builtin_huge_valf();
#pragma unroll
  for (int e = 0; e < kPerLane; ++e) m = fmaxf(m, v[e]);
  m = wave_max(m);
  if (!(m > -__builtin_huge_valf())) return Partial{-__builtin_huge_valf(), 0, 0.0};
  const float c = m * k2;
#pragma unroll
  for (int e = 0; e < kPerLane; ++e) v[e] = exp2_hw(fmaf(v[e], k2, -c));
#pragma unroll
  for (int w = kPerLane / 2; w >= 1; w >>= 1) {
#pragma unroll
    for (int e = 0; e < w; ++e) v[e] += v[e + w];
  }
  const double S = wave_sum((double)v[0]);
  return Partial{c, 0, S};
}

template <int DT, int CPW>
__global__ __launch_bounds__(kThreads) void stats_kernel(StatsArgs a) {
  __shared__ int s_best;

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const long long item = blockIdx.x;
  const int n_tiles = (a.n_chunks + CPW - 1) / CPW;
  const long long row = item / n_tiles;
  const int tile = (int)(item - row * n_tiles);
  const int V = a.V;
  const long long rowbytes = (long long)V * SegLoad<DT>::ES;
  const char* rowp = row < a.n_a ? (const char*)a.rows_a + row * rowbytes
                                 : (const char*)a.rows_b + (row - a.n_a) * rowbytes;

  // Issue this wave's loads for every chunk of the tile before looking up
  // the row's temperature.
  SegLoad<DT> ld[CPW];
  if (a.vec_ok) {
#pragma unroll
    for (int k = 0; k < CPW; ++k) {
      const int ch = tile * CPW + k;
      if (ch < a.n_chunks) ld[k].issue(rowp, V, ch * kChunk + wave * kWaveSpan);
    }
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

  Partial* out = a.part + row * (long long)a.n_chunks * kPartsPerChunk;
#pragma unroll
  for (int k = 0; k < CPW; ++k) {
    const int ch = tile * CPW + k;
    if (ch >= a.n_chunks) break;
    const int seg0 = ch * kChunk + wave * kWaveSpan;
    Partial p{0.0f, 0, 0.0};
    if (temp_ok(T)) {                     // a bad temperature is reported by the finish pass
      float v[kPerLane];
      if (a.vec_ok) ld[k].unpack(V, seg0, v);
      else seg_load_scalar<DT>(rowp, V, seg0, v);
      p = seg_partial<DT>(v, seg0, T);
    }
    if (lane == 0) out[ch * kPartsPerChunk + wave] = p;
  }
}

// ---------------------------------------------------------------------------
// Shared pieces of the finish passes.

struct RowStats {
  float c;     // log2 offset (sampled) or max logit (greedy)
  int amax;    // first argmax (greedy)
  double s;    // sum of 2^(x k - c) (sampled)
};

// Merge one row's partials with one wave (lanes over partials, in index
// order); returns false when the row has no finite maximum.
__device__ bool merge_row_wave(const Partial* __restrict__ p, int n_parts, bool greedy,
                               RowStats* out) {
  const int lane = threadIdx.x & 63;
  Partial q[kMaxChunks * kPartsPerChunk / 64];
#pragma unroll
  for (int k = 0; k < kMaxChunks * kPartsPerChunk / 64; ++k) {
    const int j = lane + 64 * k;
    q[k] = j < n_parts ? p[j] : Partial{-__builtin_huge_valf(), 0x7fffffff, 0.0};
  }
  if (greedy) {
    unsigned long long best = 0ull;
#pragma unroll
    for (int k = 0; k < kMaxChunks * kPartsPerChunk / 64; ++k) {
      const int j = lane + 64 * k;
      if (j < n_parts) {
        const unsigned long long key = ((unsigned long long)float_order_key(q[k].c) << 32) |
                                       (0xffffffffu - (uint32_t)q[k].amax);
        best = key > best ? key : best;
      }
    }
    best = wave_max_u64(best);
    const float m = float_from_order_key((uint32_t)(best >> 32));
    out->c = m;
    out->amax = (int)(0xffffffffu - (uint32_t)best);
    out->s = 0.0;
    return m > -__builtin_huge_valf() && m < __builtin_huge_valf();
  }
  float C = -__builtin_huge_valf();
#pragma unroll
  for (int k = 0; k < kMaxChunks * kPartsPerChunk / 64; ++k) C = fmaxf(C, q[k].c);
  C = wave_max(C);
  double S = 0.0;
#pragma unroll
  for (int k = 0; k < kMaxChunks * kPartsPerChunk / 64; ++k)
    if (q[k].s > 0.0) S += q[k].s * exp2((double)q[k].c - (double)C);
  S = wave_sum(S);
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

// This thread's 8 contiguous weights of chunk `chunk` (zero past V and for
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
  const int wf = fm ? __shfl(found, __ffsll((long long)fm) - 1, 64) : 0x7fffffff;
  const int wl = lm ? __shfl(lastp, 63 - __clzll((long long)lm), 64) : -1;
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
  double acc = 0.0;
#pragma unroll
  for (int e = 0; e < kPerThread; ++e) acc += (double)w[e];
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
    const double R = __shfl(incl, 63, 64);
    const double t = u * R;
    double excl = __shfl_up(incl, 1, 64);
    if (lane == 0) excl = 0.0;
    const unsigned long long hit = __ballot(lane < n_chunks && m > 0.0 && incl > t);
    const unsigned long long pos = __ballot(lane < n_chunks && m > 0.0);
    // rounding left u * R uncrossed: the last chunk with mass
    const int jc = hit ? __ffsll((long long)hit) - 1 : (pos ? 63 - __clzll((long long)pos) : 0);
    const double base = __shfl(excl, jc, 64);
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

struct LinShared {
  RowStats rows[2 * kMaxGamma + 1];
  double p[kMaxGamma], q[kMaxGamma];
  int tok[kMaxGamma];
  int flags, nacc;
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

  if (tid == 0) sh.flags = 0;
  int tok = 0;
  if (tid < g) {
    tok = a.tokens[o0 + tid];
    sh.tok[tid] = tok;
  }
  __syncthreads();
  const int nr = 2 * g + 1;  // target rows 0..g, then draft rows 0..g-1
  for (int rr = wave; rr < nr; rr += kFinWaves) {
    const bool is_t = rr <= g;
    const long long row = is_t ? tr0 + rr : a.n_target_rows + o0 + (rr - g - 1);
    RowStats rs;
    const bool ok = merge_row_wave(a.part + row * n_parts, n_parts, is_t ? gt : gd, &rs);
    if (lane == 0) {
      if (!ok) atomicOr(&sh.flags, kRowNonFinite);
      sh.rows[rr] = rs;
    }
  }
  __syncthreads();

  if (tid < 64) {
    const int i = tid;
    bool reject = false;
    if (i < g) {
      if (tok < 0 || tok >= V) {
        atomicOr(&sh.flags, kRowBadToken);
        tok = 0;
      }
      const float x = load_logit<DT>(a.target, (tr0 + i) * (long long)V + tok);
      const float y = load_logit<DT>(a.draft, ((long long)o0 + i) * V + tok);
      const double p = row_prob(sh.rows[i], gt, kt, x, tok);
      const double q = row_prob(sh.rows[g + 1 + i], gd, kd, y, tok);
      double rt;
      if (q > 0.0) {
        rt = p / q;
      } else {
        atomicOr(&sh.flags, kRowWarnQZero);
        rt = p > 0.0 ? __builtin_huge_val() : 0.0;
      }
      const uint32_t rid = a.row_ids ? a.row_ids[b] : (uint32_t)b;
      const double u = word_to_uniform(verify_words(a.seed, a.step, rid, (uint32_t)(i + 1)).x);
      reject = !(u < rt);
      sh.p[i] = p;
      sh.q[i] = q;
    }
    const unsigned long long rej = __ballot(reject);
    if (tid == 0) sh.nacc = rej ? (__ffsll((long long)rej) - 1) : g;
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
  const bool residual = n_acc < g;
  r.kind = residual ? kKindReject : kKindBonus;
  r.p_c = sh.rows[n_acc].c;
  r.p_inv_s = (float)(1.0 / sh.rows[n_acc].s);
  if (residual) {
    const RowStats& qs = sh.rows[g + 1 + n_acc];
    r.q_greedy = gd;
    r.q_amax = qs.amax;
    r.q_c = qs.c;
    r.q_inv_s = gd ? 0.0f : (float)(1.0 / qs.s);
  }
  return r;
}

// The stop distribution a non-greedy record describes.
template <int DT>
__device__ __forceinline__ StopDist record_dist(const LinearArgs& a, int b, const LinRecord& r,
                                                float Tt, float Td) {
  StopDist d;
  const long long tr0 = (long long)r.o0 + b;
  const long long es = DT ? 2 : 4;
  d.prow = (const char*)a.target + (tr0 + r.n_acc) * (long long)a.V * es;
  d.residual = r.kind == kKindReject;
  d.qrow = d.residual ? (const char*)a.draft + ((long long)r.o0 + r.n_acc) * a.V * es : d.prow;
  d.p_k = log2e_over_t(Tt);
  d.p_c = r.p_c;
  d.p_inv_s = r.p_inv_s;
  d.q_greedy = d.residual ? r.q_greedy : 0;
  d.q_amax = r.q_amax;
  d.q_k = (d.residual && Td > 0.0f) ? log2e_over_t(Td) : 0.0f;
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
// Linear verify, V <= 4 chunks: one work item per batch row does everything.

// The weights and masses of up to 4 chunks, kept in registers.
struct RowWeights {
  float w[4][kPerThread];
  double excl[4];
};

template <int DT>
__device__ __forceinline__ void row_weights(const StopDist& d, int V, int n_chunks, int vec_ok,
                                            RowWeights& rw, double* s_scan, double* s_mass) {
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    if (c < n_chunks) {
      stop_weights<DT>(d, V, c, vec_ok, 0u, rw.w[c]);
      double acc = 0.0;
#pragma unroll
      for (int e = 0; e < kPerThread; ++e) acc += (double)rw.w[c][e];
      double total;
      rw.excl[c] = block_exclusive_scan<kFinWaves>(acc, s_scan, &total);
      if (threadIdx.x == 0) s_mass[c] = total;
    }
  }
  __syncthreads();
}

template <int DT>
__global__ __launch_bounds__(kFinThreads) void linear_row_kernel(LinearArgs a) {
  __shared__ LinShared sh;
  __shared__ double s_scan[kFinWaves];
  __shared__ double s_mass[kMaxChunks];
  __shared__ int s_found[kFinWaves], s_last[kFinWaves];
  __shared__ int s_jc;
  __shared__ double s_base, s_t;

  const int b = blockIdx.x;
  const int n_chunks = a.n_chunks;
  const LinRecord r = linear_decide<DT>(a, b, true, sh);
  int warn = 0;
  if (r.kind == kKindReject || r.kind == kKindBonus) {
    const float Tt = a.temp_t[b], Td = a.temp_d[b];
    StopDist d = record_dist<DT>(a, b, r, Tt, Td);
    RowWeights rw;
    row_weights<DT>(d, a.V, n_chunks, a.vec_ok, rw, s_scan, s_mass);
    double R = 0.0;
    for (int c = 0; c < n_chunks; ++c) R += s_mass[c];
    if (!(R > 0.0) && d.residual) {
      // zero residual mass (rounding only): draw from p at this position
      warn |= kRowWarnRZero;
      d.residual = 0;
      row_weights<DT>(d, a.V, n_chunks, a.vec_ok, rw, s_scan, s_mass);
    }
    const uint32_t rid = a.row_ids ? a.row_ids[b] : (uint32_t)b;
    const double u = word_to_uniform(verify_words(a.seed, a.step, rid, (uint32_t)r.n_acc).y);
    choose_chunk(s_mass, n_chunks, u, &s_jc, &s_base, &s_t);
    const int jc = s_jc;
    float wj[kPerThread];
    double ej = 0.0;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      if (c == jc) {
#pragma unroll
        for (int e = 0; e < kPerThread; ++e) wj[e] = rw.w[c][e];
        ej = rw.excl[c];
      }
    }
    const int token = find_in_chunk(wj, jc, s_base, ej, s_t, s_found, s_last);
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

template <int DT>
__global__ __launch_bounds__(kFinThreads) void linear_mass_kernel(LinearArgs a) {
  __shared__ LinRecord s_rec;
  __shared__ double s_scan[kFinWaves];
  const int n_chunks = a.n_chunks;
  const int b = blockIdx.x / n_chunks;
  const int c = blockIdx.x - b * n_chunks;
  if (threadIdx.x == 0) s_rec = a.rec[b];
  const float Tt = a.temp_t[b], Td = a.temp_d[b];
  __syncthreads();
  const LinRecord r = s_rec;
  if (r.kind != kKindReject && r.kind != kKindBonus) return;
  const StopDist d = record_dist<DT>(a, b, r, Tt, Td);
  const double m = chunk_mass<DT>(d, a.V, c, a.vec_ok, 0u, s_scan);
  if (threadIdx.x == 0) a.mass[(long long)b * n_chunks + c] = m;
}

template <int DT>
__global__ __launch_bounds__(kFinThreads) void linear_select_kernel(LinearArgs a) {
  __shared__ LinRecord s_rec;
  __shared__ double s_mass[kMaxChunks];
  __shared__ double s_scan[kFinWaves];
  __shared__ int s_found[kFinWaves], s_last[kFinWaves];
  __shared__ int s_jc;
  __shared__ double s_base, s_t;

  const int tid = threadIdx.x;
  const int b = blockIdx.x;
  const int n_chunks = a.n_chunks;
  if (tid == 0) s_rec = a.rec[b];
  if (tid < n_chunks) s_mass[tid] = a.mass[(long long)b * n_chunks + tid];
  const float Tt = a.temp_t[b], Td = a.temp_d[b];
  __syncthreads();
  const LinRecord r = s_rec;
  int warn = 0;
  if (r.kind == kKindReject || r.kind == kKindBonus) {
    StopDist d = record_dist<DT>(a, b, r, Tt, Td);
    double R = 0.0;
    for (int j = 0; j < n_chunks; ++j) R += s_mass[j];
    if (!(R > 0.0)) {
      // zero residual mass (rounding only): draw from p at this position
      warn |= kRowWarnRZero;
      d.residual = 0;
      for (int j = 0; j < n_chunks; ++j) {
        const double mj = chunk_mass<DT>(d, a.V, j, a.vec_ok, 0u, s_scan);
        if (tid == 0) s_mass[j] = mj;
      }
      __syncthreads();
    }
    const uint32_t rid = a.row_ids ? a.row_ids[b] : (uint32_t)b;
    const double u = word_to_uniform(verify_words(a.seed, a.step, rid, (uint32_t)r.n_acc).y);
    choose_chunk(s_mass, n_chunks, u, &s_jc, &s_base, &s_t);
    const int token = chunk_select<DT>(d, a.V, s_jc, a.vec_ok, 0u, s_base, s_t, s_scan, s_found,
                                       s_last);
    if (tid == 0) a.out_tokens[(long long)r.o0 + b + r.n_acc] = token;
  }
  if (tid == 0) write_row_status(a, b, r, warn);
}

// ---------------------------------------------------------------------------
// Tree verify (TOPK): one work item per tree.

template <int DT>
__global__ __launch_bounds__(kFinThreads) void tree_kernel(TreeArgs a) {
  __shared__ RowStats s_rows[kMaxNodes];
  __shared__ int s_par[kMaxNodes], s_tok[kMaxNodes], s_path[kMaxNodes];
  __shared__ double s_pn[kMaxNodes], s_u[kMaxNodes];
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
  if (!err0) {
    for (int n = wave; n < nn; n += kFinWaves) {
      RowStats rs;
      const bool ok = merge_row_wave(a.part + (rb + n) * n_parts, n_parts, greedy, &rs);
      if (lane == 0) {
        if (!ok) atomicOr(&s_flags, kRowNonFinite);
        s_rows[n] = rs;
      }
    }
  }
  __syncthreads();
  const int err = err0 | (s_flags & kRowErrorMask);
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
      const double incl = wave_inclusive_scan(mass);
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
    const Partial* sp = a.part + (rb + stop) * n_parts;
    // chunk masses of p at the stop node from its partials, minus the
    // rejected siblings' probabilities
    if (tid < n_chunks) {
      double m = 0.0;
#pragma unroll
      for (int w = 0; w < kPartsPerChunk; ++w) {
        const Partial q = sp[tid * kPartsPerChunk + w];
        if (q.s > 0.0) m += q.s * exp2((double)q.c - (double)st.c);
      }
      m /= st.s;
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
      if (tid < n_chunks) {
        double m = 0.0;
#pragma unroll
        for (int w = 0; w < kPartsPerChunk; ++w) {
          const Partial q = sp[tid * kPartsPerChunk + w];
          if (q.s > 0.0) m += q.s * exp2((double)q.c - (double)st.c);
        }
        s_mass[tid] = m / st.s;
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
int stats_chunks_per_item(long long n_rows, int n_chunks) {
  return n_rows * n_chunks <= 2048 ? 1 : 2;
}

long long stats_items(long long n_rows, int n_chunks) {
  const int cpw = stats_chunks_per_item(n_rows, n_chunks);
  return n_rows * ((n_chunks + cpw - 1) / cpw);
}

// With both events set, they are attached to the kernel's dispatch packet
// (start and end of the kernel itself, as a profiler sees it).
hipError_t launch_stats(int dtype, const StatsArgs& a, hipStream_t st, hipEvent_t ev_start,
                        hipEvent_t ev_stop) {
  const long long n = stats_items(a.n_rows, a.n_chunks);
  const int cpw = stats_chunks_per_item(a.n_rows, a.n_chunks);
  const dim3 grid((unsigned)n), block(kThreads);
  const bool timed = ev_start && ev_stop;
#define SV_LAUNCH_STATS(DT, CPW)                                                             \
  do {                                                                                      \
    if (timed)                                                                              \
      hipExtLaunchKernelGGL(stats_kernel<DT, CPW>, grid, block, 0, st, ev_start, ev_stop, 0, a); \
    else                                                                                    \
      stats_kernel<DT, CPW><<<grid, block, 0, st>>>(a);                                     \
  } while (0)
  if (dtype == 1) {
    if (cpw == 1) SV_LAUNCH_STATS(1, 1);
    else SV_LAUNCH_STATS(1, 2);
  } else {
    if (cpw == 1) SV_LAUNCH_STATS(0, 1);
    else SV_LAUNCH_STATS(0, 2);
  }
#undef SV_LAUNCH_STATS
  return hipGetLastError();
}

hipError_t launch_linear_finish(int dtype, const LinearArgs& a, hipStream_t st) {
  const dim3 rows((unsigned)a.B), block(kFinThreads);
  if (a.n_chunks <= 4) {
    if (dtype == 1) linear_row_kernel<1><<<rows, block, 0, st>>>(a);
    else linear_row_kernel<0><<<rows, block, 0, st>>>(a);
    return hipGetLastError();
  }
  const dim3 items((unsigned)((long long)a.B * a.n_chunks));
  if (dtype == 1) linear_decide_kernel<1><<<rows, block, 0, st>>>(a);
  else linear_decide_kernel<0><<<rows, block, 0, st>>>(a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (dtype == 1) linear_mass_kernel<1><<<items, block, 0, st>>>(a);
  else linear_mass_kernel<0><<<items, block, 0, st>>>(a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (dtype == 1) linear_select_kernel<1><<<rows, block, 0, st>>>(a);
  else linear_select_kernel<0><<<rows, block, 0, st>>>(a);
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
