// Finish passes of the linear verify, gfx950.
//
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
//
// Work items never wait for one another: a kernel boundary is the only
// synchronisation, because device-scope fences and atomics are costly here.
//
// Sources: acceptance rule and first-reject stop (kwkr.cn/news/620872 §2.3,
// §4.1, §4.3; cf-1.com/news/5632551 §2.2); residual and bonus draws
// (blog.lonae.com/posts/2026-draft-model-kv-jDwzYp, formal-definition
// paragraph); greedy exact match (kwkr §4.3).
#include <hip/hip_ext.h>

#include <algorithm>

#include "sv_common.h"
#include "sv_internal.h"
#include "sv_finish.h"

namespace sv {

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
  // the draft tokens and the logits at them (gathered by the vocabulary pass)
  // (no branch around them, so that nothing waits for them before their use)
  const int li = min(lane, g > 0 ? g - 1 : 0);
  const int tok = *(g > 0 ? a.tokens + o0 + li : a.off);
  const float x = *(g > 0 ? a.gath + o0 + li : (const float*)a.off);
  const float y = *(g > 0 ? a.gath + a.total_draft + o0 + li : (const float*)a.off);
  // rows wave + 4 k (k < kDecideRowsPerWave), clamped into [0, nr): loaded
  // and merged unconditionally
  Partial q[kDecideRowsPerWave];
#pragma unroll
  for (int k = 0; k < kDecideRowsPerWave; ++k)
    q[k] = lane_partial(a.part + row_of(min(wave + k * kFinWaves, nr - 1)) * n_parts, n_parts);
  // lane l's Philox block of slot l, formed while the loads are in flight
  // (wave 0 uses it: word 0 tests d_{l-1}, word 1 is the draw at stop l)
  const uint32_t rid = a.row_ids ? load_uniform_u32(a.row_ids + b) : (uint32_t)b;
  const uint4 wl = verify_words(a.seed, a.step, rid, (uint32_t)lane);
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
  // each wave stores its own total (the wave scan's last lane, as the block
  // scan forms it), so the waves never wait for one another
  auto reduce = [&](const StopDist& dd, int bb, int cc, const StopVec<DT>& cur, int vec) {
    float w[kPerThread];
    stop_weights_from<DT>(dd, V, cc, vec, 0u, cur, w);
    const double incl = wave_inclusive_scan(thread_total(w));
    if ((threadIdx.x & 63) == 63)
      a.wsum[((long long)bb * nc + cc) * kFinWaves + (threadIdx.x >> 6)] = incl;
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
  const int n_chunks = a.n_chunks;
  const int b = blockIdx.x / n_chunks;
  const int c = blockIdx.x - b * n_chunks;
  const LinRecord r = linear_decide<DT>(a, b, c == 0, sh);
  if (c == 0 && threadIdx.x == 0) a.rec[b] = r;
  if (r.kind != kKindReject && r.kind != kKindBonus) return;
  const StopDist d = record_dist<DT>(a, b, r);
  float w[kPerThread];
  stop_weights<DT>(d, a.V, c, a.vec_ok, 0u, w);
  // each wave stores its own total (the wave scan's last lane)
  const double incl = wave_inclusive_scan(thread_total(w));
  if ((threadIdx.x & 63) == 63)
    a.wsum[((long long)b * n_chunks + c) * kFinWaves + (threadIdx.x >> 6)] = incl;
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
  // the record and the wave totals are in flight together: the record is
  // waited for here (its kind, as a scalar), the totals by their LDS stores
  asm volatile("" ::"s"(r.kind));
#pragma unroll
  for (int k = 0; k < kPerLaneWs; ++k)
    if (lane + 64 * k < nws) s_ws[lane + 64 * k] = wv[k];
  __syncthreads();
  int warn = 0;
  if (r.kind == kKindReject || r.kind == kKindBonus) {
    StopDist d = record_dist<DT>(a, b, r);
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
// Host launcher.

static int mass_resident_blocks(int dt) {
  return dt == 1 ? resident_blocks(3, linear_mass_kernel<1, true>, kFinThreads)
                 : resident_blocks(4, linear_mass_kernel<0, true>, kFinThreads);
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

}  // namespace sv
