// Finish passes of the tree verify, gfx950: one work item per tree.
//   TOPK          tree_kernel walks the tree with one lane per node and draws
//                 in one chunk of the stop row.
//   SAMPLED_WOR   tree_wor_kernel walks it with the whole block: one
//                 vocabulary pass over the node's target and draft rows per
//                 rejected sibling (the target term kept in LDS across a
//                 node's passes when V <= 32768), then the draw.
//
// Sources: tree walk over siblings drawn by top-k or by temperature sampling
// (kwkr.cn/news/620872 §5.3; blog.lonae.com/posts/
// 2026-draft-model-kv-jDwzYp, tree-attention paragraphs); acceptance rule
// and residual draw as in the linear verify (kwkr §2.3, §4.1; lonae
// formal-definition paragraph).
#include <hip/hip_ext.h>

#include <algorithm>

#include "sv_common.h"
#include "sv_internal.h"
#include "sv_finish.h"
#include "sv_pass.h"

namespace sv {

// The vocabulary pass reads the rows of the nodes that have children only.
// A leaf's target row is read here, when the walk stops at that leaf (its
// bonus draw): its chunk Partials formed with the pass's own per-wave
// arithmetic, one wave per chunk, then merged as the walk's prologue merges
// the other rows.  Leaves rs (and, for a sampled row, p's chunk masses
// cm[0..nc)) in LDS and returns whether the row has a finite maximum.  Called
// by every thread of the work item.
static_assert(kPartsPerChunk == 1, "one Partial per chunk");
template <int DT>
__device__ bool leaf_row_stats(const char* rowp, int V, int nc, int vec_ok, bool greedy, float k2,
                               Partial* s_part, RowStats* s_rs, double* s_cmv, int* s_ok) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  for (int c = wave; c < nc; c += kFinWaves) {
    const Partial p = wave_chunk_partial<DT>(rowp, V, c, vec_ok, greedy, k2);
    if (lane == 0) s_part[c] = p;
  }
  __syncthreads();
  if (wave == 0) {
    const Partial q = s_part[lane < nc ? lane : 0];
    RowStats rs;
    const bool ok = merge_parts_seg(q, lane < nc, seg_width(nc), greedy, &rs);
    if (lane == 0) {
      *s_rs = rs;
      *s_ok = ok;
    }
    if (!greedy && lane < nc) s_cmv[lane] = q.s > 0.0 ? scale_pow2(q.s, q.c - rs.c) / rs.s : 0.0;
  }
  __syncthreads();
  return *s_ok != 0;
}

// The outputs of a batch row in error.
__device__ __forceinline__ void tree_error_row(const TreeArgs& a, int b, int err) {
  const int N = a.N;
  const long long rb = (long long)b * N;
  for (int i = threadIdx.x; i < N; i += kFinThreads) {
    a.out_tokens[rb + i] = -1;
    if (i < N - 1) a.path_nodes[(long long)b * (N - 1) + i] = -1;
    if (a.p_at) a.p_at[rb + i] = 0.0f;
  }
  if (threadIdx.x == 0) {
    a.num_accepted[b] = -1;
    if (a.row_status) a.row_status[b] = err;
  }
}

// ---------------------------------------------------------------------------
// Tree verify (TOPK): one work item per tree.

template <int DT>
__global__ __launch_bounds__(kFinThreads) void tree_kernel(TreeArgs a) {
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
  __shared__ Partial s_leaf[kMaxChunks];
  __shared__ int s_leafok;

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

  // Partials of the node rows, merged in groups of P lanes per row (64 / P
  // rows per wave and round), and one node per lane: its parent, its token
  // and the logit of the token under the parent (gathered by the vocabulary
  // pass).  Only wave 0's lanes 1..nn-1 keep the latter.  The first round's
  // loads sit ahead of any branch.
  const int P = seg_width(n_parts), R = 64 / P;
  const int part = lane & (P - 1), sub = lane / P;
  auto load_part = [&](int row) {
    const int n = min(row, N - 1);
    return a.part[(rb + n) * n_parts + min(part, n_parts - 1)];
  };
  Partial q0 = load_part(wave * R + sub);
  const int li = lane < N ? lane : 0;
  int par = a.parents[rb + li];
  int tok = a.tokens[rb + li];
  const float x = a.gath[rb + li];   // gathered by the vocabulary pass
  const bool mine = !err0 && tid > 0 && tid < nn;
  const bool badpar = mine && (par < 0 || par >= tid);
  const bool badtok = mine && (tok < 0 || tok >= V);
  // the nodes with children, in every wave (the lanes hold nodes 0..63):
  // only their rows were read by the vocabulary pass
  const bool kid_l = !err0 && lane > 0 && lane < nn && par >= 0 && par < lane;
  const unsigned long long inner = wave_or_u64(kid_l ? 1ull << par : 0ull);
  if (!mine) {
    par = -1;
    tok = 0;
  }
  if (!err0) {
    for (int base = wave * R; base < nn; base += kFinWaves * R) {
      const Partial q = base == wave * R ? q0 : load_part(base + sub);
      const int n = base + sub;
      const bool used = n < nn && ((inner >> (n & 63)) & 1ull);
      RowStats rs;
      const bool ok = merge_parts_seg(q, used && part < n_parts, P, greedy, &rs);
      if (used) {
        if (part == 0) {
          s_rows[n] = rs;
          s_rowok[n] = ok;
        }
        if (!greedy && part < n_chunks)
          s_cm[n * n_chunks + part] = q.s > 0.0 ? scale_pow2(q.s, q.c - rs.c) / rs.s : 0.0;
      }
    }
  }
  if (tid < kMaxNodes) {
    s_par[tid] = par;
    s_tok[tid] = tok;
  }
  __syncthreads();
  if (tid < 64) {
    const bool read = tid < nn && ((inner >> tid) & 1ull);
    const int flags = (__ballot(badpar) ? kRowBadShape : 0) | (__ballot(badtok) ? kRowBadToken : 0) |
                      (__ballot(read && !err0 && !s_rowok[tid < kMaxNodes ? tid : 0])
                           ? kRowNonFinite : 0);
    if (tid == 0) s_flags = err0 | flags;
  }
  __syncthreads();
  const int err = s_flags & kRowErrorMask;
  if (err) {
    tree_error_row(a, b, err);
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
  if (!((inner >> stop) & 1ull)) {
    // a leaf: its row, for the bonus draw
    const char* lrow = (const char*)a.target + (rb + stop) * (long long)V * (DT ? 2 : 4);
    if (!leaf_row_stats<DT>(lrow, V, n_chunks, a.vec_ok, greedy, k2, s_leaf, &s_rows[stop],
                            &s_cm[stop * n_chunks], &s_leafok)) {
      tree_error_row(a, b, kRowNonFinite);
      return;
    }
  }

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
// Tree verify (SAMPLED_WOR): the children of a node were drawn from the
// draft's q without replacement.  Child j is tested against p_j and q_j,
// where q_j is q without the tokens of the rejected siblings (renormalised);
// each rejection replaces p_j by the normalised residual max(0, p_j - q_j).
//
// No residual is ever stored.  With a = p(v) and b = q(v), every p_j has the
// form max(0, a - L_v b) / P: L_v = lambda for tokens still in q_j, and the
// value lambda took when a rejected sibling's token left q (it leaves with
// the residual taken at its own test).  Rejecting child j with
// Q = q's mass left in q_j sets mu = lambda + P / Q and
// G = sum_v max(0, a - L'_v b), L'_v = mu for tokens still in q_j; then
// lambda = mu and P = G (both unchanged when G = 0: the residual is empty).
// One vocabulary pass over the node's weights forms G (and, when q(t_j) is
// more than half of Q, the draft mass that stays once t_j leaves; otherwise
// that is Q - q(t_j)), so a walk costs one pass per rejected sibling, plus
// the draw.  When every child is rejected, the draw's weights are the last
// pass's.  Without the cache a pass reads the node's two rows and forms two
// exponentials per element; with it (V of at most 4 chunks) only a node's
// first pass does, and the later ones form max(0, a - L b) from LDS and
// registers.

// The rows of one tree node as the SAMPLED_WOR passes read them, with
// p(v) = 2^(x p_k - p_c) p_inv_s + [v = p_amax] (and q likewise): a sampled
// row has p_amax = -1; a greedy one has p_k = 1, p_c = +inf, p_inv_s = 0,
// so that the exponential term is 0 (its x is finite or -inf: rows with a
// +inf logit are reported before any pass).  An unread draft row has every
// q term 0.  Every field is uniform over the block.
struct WorDist {
  const char* xrow;      // target row of the node
  const char* yrow;      // draft row of the node (the target row when unread)
  float p_k, p_c, p_inv_s;
  int p_amax;
  float q_k, q_c, q_inv_s;
  int q_amax;
  int onehot;            // a greedy row is present (one-hot terms to add)
};

// lambda as the float32 weights use it (finite: -lambda * 0 must stay 0).
__device__ __forceinline__ float lam_f32(double lam) { return uni((float)fmin(lam, 3.0e38)); }

// The node's distributions; `use_q` = 0 leaves q at 0 (bonus draw at a leaf).
__device__ __forceinline__ WorDist wor_dist(const char* xrow, const char* yrow, const RowStats& ps,
                                            const RowStats& qs, bool gt, bool gd, float kt,
                                            float kd, bool use_q) {
  const float inf = __builtin_huge_valf();
  WorDist d;
  d.xrow = xrow;
  d.yrow = use_q ? yrow : xrow;
  d.p_k = uni(gt ? 1.0f : kt);
  d.p_c = uni(gt ? inf : ps.c);
  d.p_inv_s = uni(gt ? 0.0f : (float)ps.inv_s);
  d.p_amax = uni(gt ? ps.amax : -1);
  const bool qe = use_q && !gd;   // sampled draft term
  d.q_k = uni(qe ? kd : 1.0f);
  d.q_c = uni(qe ? qs.c : inf);
  d.q_inv_s = uni(qe ? (float)qs.inv_s : 0.0f);
  d.q_amax = uni((use_q && gd) ? qs.amax : -1);
  d.onehot = d.p_amax >= 0 || d.q_amax >= 0;
  return d;
}

constexpr int kWorGroup = 2;   // chunks whose loads are in flight together


// This thread's 16-byte loads of one chunk of both rows (VEC: V a multiple
// of the vector width and rows 16-byte aligned; addresses clamped into the
// row past V).
template <int DT, bool VEC>
__device__ __forceinline__ void wor_load(const WorDist& d, int V, int chunk, StopVec<DT>& r) {
  if (!VEC) return;   // the weights load element by element
  constexpr int ES = StopVec<DT>::ES, EPV = StopVec<DT>::EPV;
  const int e0 = chunk * kChunk + threadIdx.x * kPerThread;
#pragma unroll
  for (int j = 0; j < StopVec<DT>::NV; ++j) {
    const int ej = e0 + j * EPV;
    const long long off = ej < V ? (long long)ej * ES : 0;
    r.p[j] = *(const uint4*)(d.xrow + off);
    r.q[j] = *(const uint4*)(d.yrow + off);
  }
}

// Weights of this thread's 8 elements of `chunk`: w = max(0, a - L b), with
// L = lam or, for the tokens in ex_tok, their own ex_lam; be = b outside
// ex_tok and t_cur (WANT_E only).  Both are 0 past V.  Every pass and the
// draw form weights through this code.
template <int DT, bool VEC, bool WANT_E>
__device__ __forceinline__ void wor_weights(const WorDist& d, int V, int chunk,
                                            const StopVec<DT>& r, float lam, const int* ex_tok,
                                            const float* ex_lam, int nex, int t_cur,
                                            float w[kPerThread], float be[kPerThread]) {
  constexpr int EPV = StopVec<DT>::EPV;
  const int e0 = chunk * kChunk + threadIdx.x * kPerThread;
  float xp[kPerThread], xq[kPerThread];
  if (VEC) {
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
    // indices clamped into the row: every load is issued, none behind a branch
#pragma unroll
    for (int e = 0; e < kPerThread; ++e) {
      const int idx = e0 + e, ic = idx < V ? idx : V - 1;
      const float p = load_logit<DT>(d.xrow, ic), q = load_logit<DT>(d.yrow, ic);
      xp[e] = idx < V ? p : 0.0f;
      xq[e] = idx < V ? q : 0.0f;
    }
  }
  float lv[kPerThread];
#pragma unroll
  for (int e = 0; e < kPerThread; ++e) lv[e] = lam;
  uint32_t exm = 0u;
  for (int k = 0; k < nex; ++k) {
    const int off = ex_tok[k] - e0;
    if ((unsigned)off < (unsigned)kPerThread) {
      const float l = ex_lam[k];
#pragma unroll
      for (int e = 0; e < kPerThread; ++e) {
        if (e == off) {
          lv[e] = l;
          exm |= 1u << e;
        }
      }
    }
  }
  if (WANT_E && (unsigned)(t_cur - e0) < (unsigned)kPerThread) exm |= 1u << (t_cur - e0);
  if (!d.onehot && e0 + kPerThread <= V) {
    // sampled rows, elements all inside the row (the same values as below)
#pragma unroll
    for (int e = 0; e < kPerThread; ++e) {
      const float a = exp2_hw(fmaf(xp[e], d.p_k, -d.p_c)) * d.p_inv_s;
      const float b = exp2_hw(fmaf(xq[e], d.q_k, -d.q_c)) * d.q_inv_s;
      w[e] = fmaxf(fmaf(-lv[e], b, a), 0.0f);
      if (WANT_E) be[e] = ((exm >> e) & 1u) ? 0.0f : b;
    }
    return;
  }
#pragma unroll
  for (int e = 0; e < kPerThread; ++e) {
    const int idx = e0 + e;
    const float a = fmaf(exp2_hw(fmaf(xp[e], d.p_k, -d.p_c)), d.p_inv_s,
                         idx == d.p_amax ? 1.0f : 0.0f);
    const float b = fmaf(exp2_hw(fmaf(xq[e], d.q_k, -d.q_c)), d.q_inv_s,
                         idx == d.q_amax ? 1.0f : 0.0f);
    const float wv = fmaxf(fmaf(-lv[e], b, a), 0.0f);
    const bool in = idx < V;
    w[e] = in ? wv : 0.0f;
    if (WANT_E) be[e] = (in && !((exm >> e) & 1u)) ? b : 0.0f;
  }
}

// Block totals of NV per-thread values, each formed exactly as
// block_exclusive_scan forms its total (so a chunk's mass here equals the
// total of the draw's in-chunk scan bit for bit).  Lane i of wave 0 forms
// total i (the wave-order sum) and shares it; all threads get them.
// s_red holds (kFinWaves + 1) * NV values.
template <int NV>
__device__ __forceinline__ void block_totals(const double v[NV], double* s_red, double t[NV]) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  __syncthreads();
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const double incl = wave_inclusive_scan(v[i]);
    if (lane == 63) s_red[w * NV + i] = incl;
  }
  __syncthreads();
  if (threadIdx.x < NV) {
    double s = s_red[threadIdx.x];
#pragma unroll
    for (int k = 1; k < kFinWaves; ++k) s += s_red[k * NV + threadIdx.x];
    s_red[kFinWaves * NV + threadIdx.x] = s;
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < NV; ++i) t[i] = s_red[kFinWaves * NV + i];
}

// One pass over the node's rows: chunk masses of the weights into s_mass
// (written by thread 0), their sum G returned to every thread, and with
// WANT_E the draft mass outside ex_tok and t_cur in *E.
template <int DT, bool VEC, bool WANT_E>
__device__ double wor_pass(const WorDist& d, int V, int nc, float lam,
                           const int* ex_tok, const float* ex_lam, int nex, int t_cur,
                           double* s_mass, double* s_red, double* E) {
  double e_acc = 0.0, G = 0.0;
  for (int g0 = 0; g0 < nc; g0 += kWorGroup) {
    StopVec<DT> r[kWorGroup];
#pragma unroll
    for (int k = 0; k < kWorGroup; ++k) wor_load<DT, VEC>(d, V, min(g0 + k, nc - 1), r[k]);
    double v[kWorGroup + 1];
#pragma unroll
    for (int k = 0; k < kWorGroup; ++k) {
      float w[kPerThread], be[kPerThread];
      const int c = g0 + k;
      wor_weights<DT, VEC, WANT_E>(d, V, min(c, nc - 1), r[k], lam, ex_tok, ex_lam, nex, t_cur, w,
                                   be);
      v[k] = c < nc ? thread_total(w) : 0.0;
      if (WANT_E && c < nc) e_acc += thread_total(be);
    }
    v[kWorGroup] = e_acc;
    double t[kWorGroup + 1];
    block_totals<kWorGroup + 1>(v, s_red, t);
#pragma unroll
    for (int k = 0; k < kWorGroup; ++k) {
      if (g0 + k < nc) {
        G += t[k];
        if (threadIdx.x == 0) s_mass[g0 + k] = t[k];
      }
    }
    if (WANT_E) *E = t[kWorGroup];
  }
  return G;
}

// Vocabularies of at most this many chunks keep a node's terms in a cache
// (a(v) in LDS, b(v) in registers; below).
constexpr int kWorCacheChunks = 4;   // V <= 32768

// threadIdx.x as a value the compiler cannot prove invariant: what a pass
// derives from it (addresses, element indices) is formed inside the pass
// instead of being hoisted out of the walk and held in registers throughout.
__device__ __forceinline__ int opaque_tid() {
  int t = threadIdx.x;
  asm volatile("" : "+v"(t));
  return t;
}

// With the vocabulary in at most NC chunks, a node's target term a(v) = p(v)
// is kept in LDS and its draft term b(v) = q(v) in registers (this thread's
// NC * 8 elements), filled by the node's first pass: between the passes of
// one node only lambda changes, so every later pass forms max(0, a - L b)
// with no global load and no exponential.  a and b are formed by the
// expressions of wor_weights (elements past V hold 0, whose weight is 0), so
// every weight is the same value as the draw forms from memory.  Each thread
// reads back only the a values it wrote, so the LDS cache needs no barrier.
//
// A pass needs only the total G of the new weights (and sometimes the draft
// mass left): one block reduction of two values.  The chunk masses, which
// only the draw needs, are formed once, by wor_masses_r, when the walk ends
// on a rejection.

// This thread's weights of chunk c from the cache (and, for WANT_E, the
// draft terms outside the excluded tokens and t_cur).
template <int NC, bool WANT_E>
__device__ __forceinline__ void wor_chunk_r(const float* s_a, const float (&rb)[NC * kPerThread],
                                            int c, int tix, bool hit, float lam,
                                            const int* ex_tok, const float* ex_lam, int nex,
                                            int t_cur, float w[kPerThread], float be[kPerThread]) {
  const int e0 = c * kChunk + tix * kPerThread;
  const float4* ca = (const float4*)(s_a + e0);
  const float4 lo = ca[0], hi = ca[1];
  const float av[kPerThread] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
  if (!hit) {
#pragma unroll
    for (int e = 0; e < kPerThread; ++e) {
      const float bv = rb[c * kPerThread + e];
      w[e] = fmaxf(fmaf(-lam, bv, av[e]), 0.0f);
      if (WANT_E) be[e] = bv;
    }
    return;
  }
  float lv[kPerThread];
#pragma unroll
  for (int e = 0; e < kPerThread; ++e) lv[e] = lam;
  uint32_t exm = 0u;
  for (int k = 0; k < nex; ++k) {
    const int off = ex_tok[k] - e0;
    if ((unsigned)off < (unsigned)kPerThread) {
      const float l = ex_lam[k];
#pragma unroll
      for (int e = 0; e < kPerThread; ++e) {
        if (e == off) {
          lv[e] = l;
          exm |= 1u << e;
        }
      }
    }
  }
  if (WANT_E && (unsigned)(t_cur - e0) < (unsigned)kPerThread) exm |= 1u << (t_cur - e0);
#pragma unroll
  for (int e = 0; e < kPerThread; ++e) {
    const float bv = rb[c * kPerThread + e];
    w[e] = fmaxf(fmaf(-lv[e], bv, av[e]), 0.0f);
    if (WANT_E) be[e] = ((exm >> e) & 1u) ? 0.0f : bv;
  }
}

// The chunks in which an excluded token (or t_cur) falls among this thread's
// elements: one scan of the list.
__device__ __forceinline__ uint32_t wor_hits(int tix, const int* ex_tok, int nex, int t_cur) {
  uint32_t hit = 0u;
  for (int k = 0; k < nex; ++k) {
    const int t = ex_tok[k], c = t / kChunk;
    if ((t - c * kChunk) / kPerThread == tix) hit |= 1u << c;
  }
  if (t_cur >= 0) {
    const int c = t_cur / kChunk;
    if ((t_cur - c * kChunk) / kPerThread == tix) hit |= 1u << c;
  }
  return hit;
}

// G (and E) of one pass from the cache: one block reduction of two values.
template <int NC, bool WANT_E>
__device__ __forceinline__ double wor_total_r(const float* s_a, const float (&rb)[NC * kPerThread],
                                              float lam, const int* ex_tok, const float* ex_lam,
                                              int nex, int t_cur, double* s_red, double* E) {
  const int tix = opaque_tid();
  const uint32_t hit = wor_hits(tix, ex_tok, nex, WANT_E ? t_cur : -1);
  double v[2] = {0.0, 0.0};
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    float w[kPerThread], be[kPerThread];
    wor_chunk_r<NC, WANT_E>(s_a, rb, c, tix, ((hit >> c) & 1u) != 0u, lam, ex_tok, ex_lam, nex,
                            t_cur, w, be);
    v[0] += thread_total(w);
    if (WANT_E) v[1] += thread_total(be);
  }
  double t[2];
  block_totals<2>(v, s_red, t);
  if (WANT_E) *E = t[1];
  return t[0];
}

// The chunk masses of the current weights into s_mass (formed as the draw's
// block scan forms its total); returns their sum.  The weights replace a(v)
// in LDS (each thread its own elements), for the draw that follows.
template <int NC>
__device__ __forceinline__ double wor_masses_r(float* s_a, const float (&rb)[NC * kPerThread],
                                               float lam, const int* ex_tok, const float* ex_lam,
                                               int nex, double* s_mass, double* s_red) {
  const int tix = opaque_tid();
  const uint32_t hit = wor_hits(tix, ex_tok, nex, -1);
  double v[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    float w[kPerThread], be[kPerThread];
    wor_chunk_r<NC, false>(s_a, rb, c, tix, ((hit >> c) & 1u) != 0u, lam, ex_tok, ex_lam, nex, -1,
                           w, be);
    v[c] = thread_total(w);
    float4* cw = (float4*)(s_a + c * kChunk + tix * kPerThread);
    cw[0] = make_float4(w[0], w[1], w[2], w[3]);
    cw[1] = make_float4(w[4], w[5], w[6], w[7]);
  }
  double t[NC];
  block_totals<NC>(v, s_red, t);
  double G = 0.0;
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    G += t[c];
    if (threadIdx.x == 0) s_mass[c] = t[c];
  }
  return G;
}

// A node's first pass: fills the cache (a into LDS, b into registers) and
// forms the pass's G (and E) from the same values, every chunk's loads of
// both rows in flight together (one round trip; two chunks at a time took
// 1.6 us more per walk).  No token is excluded yet at a node's first pass.
template <int DT, int NC, bool WANT_E>
__device__ __forceinline__ double wor_fill_total(const WorDist& d, int V, float* s_a,
                                                 float (&rb)[NC * kPerThread], float lam,
                                                 int t_cur, double* s_red, double* E) {
  constexpr int ES = StopVec<DT>::ES, EPV = StopVec<DT>::EPV, NV = StopVec<DT>::NV;
  constexpr int kGroup = NC;
  const int tix = opaque_tid();
  const int wave_first = __builtin_amdgcn_readfirstlane(tix) & ~63;   // the wave's first thread
  double v[2] = {0.0, 0.0};
#pragma unroll
  for (int g0 = 0; g0 < NC; g0 += kGroup) {
    uint4 rx[kGroup][NV], ry[kGroup][NV];
#pragma unroll
    for (int k = 0; k < kGroup; ++k) {
      const int c = g0 + k < NC ? g0 + k : NC - 1;
      const int e0 = c * kChunk + tix * kPerThread;
#pragma unroll
      for (int j = 0; j < NV; ++j) {
        const int ej = e0 + j * EPV;
        const long long off = ej < V ? (long long)ej * ES : 0;
        rx[k][j] = *(const uint4*)(d.xrow + off);
        ry[k][j] = *(const uint4*)(d.yrow + off);
      }
    }
#pragma unroll
    for (int k = 0; k < kGroup; ++k) {
      const int c = g0 + k;
      if (c >= NC) break;
      const int e0 = c * kChunk + tix * kPerThread;
      float xp[kPerThread], xq[kPerThread], av[kPerThread], w[kPerThread], be[kPerThread];
#pragma unroll
      for (int j = 0; j < NV; ++j) {
        const uint32_t rw[4] = {rx[k][j].x, rx[k][j].y, rx[k][j].z, rx[k][j].w};
        const uint32_t sw[4] = {ry[k][j].x, ry[k][j].y, ry[k][j].z, ry[k][j].w};
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
      // The short form first: a = 2^(x k - c) s and b likewise.  The
      // one-hot terms (a greedy row: its exponential term is 0), the
      // elements past V and t_cur are then set as the full form sets them,
      // each behind a wave-uniform test, so the values are wor_weights' own.
      float bv[kPerThread];
#pragma unroll
      for (int e = 0; e < kPerThread; ++e) {
        av[e] = exp2_hw(fmaf(xp[e], d.p_k, -d.p_c)) * d.p_inv_s;
        bv[e] = exp2_hw(fmaf(xq[e], d.q_k, -d.q_c)) * d.q_inv_s;
      }
      const int we0 = c * kChunk + wave_first * kPerThread;   // the wave's 512 elements
      if (d.onehot) {
        const int dp = d.p_amax - e0, dq = d.q_amax - e0;
#pragma unroll
        for (int e = 0; e < kPerThread; ++e) {
          av[e] = dp == e ? 1.0f : av[e];
          bv[e] = dq == e ? 1.0f : bv[e];
        }
      }
      if (we0 + 64 * kPerThread > V) {
        const int rem = V - e0;
#pragma unroll
        for (int e = 0; e < kPerThread; ++e) {
          av[e] = e < rem ? av[e] : 0.0f;
          bv[e] = e < rem ? bv[e] : 0.0f;
        }
      }
#pragma unroll
      for (int e = 0; e < kPerThread; ++e) {
        rb[c * kPerThread + e] = bv[e];
        w[e] = fmaxf(fmaf(-lam, bv[e], av[e]), 0.0f);
      }
      if (WANT_E) {
        // the draft terms without t_cur: a copy only in the wave that holds it
        if ((unsigned)(t_cur - we0) < 64u * kPerThread) {
          const int dt = t_cur - e0;
#pragma unroll
          for (int e = 0; e < kPerThread; ++e) be[e] = dt == e ? 0.0f : bv[e];
          v[1] += thread_total(be);
        } else {
          v[1] += thread_total(bv);
        }
      }
      float4* ca = (float4*)(s_a + e0);
      ca[0] = make_float4(av[0], av[1], av[2], av[3]);
      ca[1] = make_float4(av[4], av[5], av[6], av[7]);
      v[0] += thread_total(w);
    }
  }
  double t[2];
  block_totals<2>(v, s_red, t);
  if (WANT_E) *E = t[1];
  return t[0];
}

template <int DT, bool VEC, int NC>
__global__ __launch_bounds__(kFinThreads) void tree_wor_kernel(TreeArgs a) {
  __shared__ RowStats s_rows[kMaxNodes], s_qrows[kMaxNodes];
  __shared__ int s_par[kMaxNodes], s_tok[kMaxNodes], s_path[kMaxNodes];
  __shared__ int s_rowok[kMaxNodes], s_qrowok[kMaxNodes];
  __shared__ double s_pa[kMaxNodes], s_qb[kMaxNodes], s_uacc[kMaxNodes];
  __shared__ double s_cm[kMaxNodes * (NC ? NC : kMaxChunks)];  // p's mass per (node, chunk)

  __shared__ __attribute__((aligned(16))) float s_a[NC ? NC * kChunk : 4];   // a(v) of cached_node
  __shared__ int s_ex_tok[kMaxNodes];              // tokens of the rejected siblings
  __shared__ float s_ex_lamf[kMaxNodes];           // their lambda (weights)
  __shared__ double s_ex_lam[kMaxNodes];           // their lambda (ratios)
  __shared__ unsigned long long s_inner;
  __shared__ int s_flags;
  __shared__ double s_red[(kFinWaves + 1) * ((NC > kWorGroup ? NC : kWorGroup) + 1)];
  __shared__ double s_scan[kFinWaves];
  __shared__ double s_mass[kMaxChunks];
  __shared__ int s_found[kFinWaves], s_last[kFinWaves];
  __shared__ int s_jc;
  __shared__ double s_base, s_t;
  __shared__ Partial s_leaf[kMaxChunks];
  __shared__ int s_leafok;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nc = NC ? NC : a.n_chunks;
  const int n_parts = nc * kPartsPerChunk;
  const int b = blockIdx.x;
  const int V = a.V, N = a.N;
  const int nn = uni(a.n_nodes ? a.n_nodes[b] : N);
  const float Tt = uni(a.temp[b]), Td = uni(a.temp_d[b]);
  const long long rb = (long long)b * N;
  const long long qb = (long long)a.B * N;   // first draft row / draft gathers

  int err0 = 0;
  if (nn < 1 || nn > N) err0 = kRowBadShape;
  else if (!temp_ok(Tt) || !temp_ok(Td)) err0 = kRowBadTemp;
  const bool gt = Tt == 0.0f, gd = Td == 0.0f;
  const float kt = uni((gt || err0) ? 0.0f : log2e_over_t(Tt));
  const float kd = uni((gd || err0) ? 0.0f : log2e_over_t(Td));
  const uint32_t rid = uni((int)(a.row_ids ? a.row_ids[b] : (uint32_t)b));

  // Partials of the 2 nn rows (target rows of the nodes, then their draft
  // rows), merged in groups of P lanes per row, and one node per lane.  The
  // first round's loads sit ahead of any branch.
  const int P = seg_width(n_parts), R = 64 / P;
  const int part = lane & (P - 1), sub = lane / P;
  const int n_rows = err0 ? 0 : 2 * nn;
  auto load_part = [&](int row) {
    const int r = min(row, 2 * N - 1);
    const long long at = r < nn ? rb + r : qb + rb + min(r - nn, N - 1);
    return a.part[at * n_parts + min(part, n_parts - 1)];
  };
  Partial q0 = load_part(wave * R + sub);
  const int li = lane < N ? lane : 0;
  int par = a.parents[rb + li];
  int tok = a.tokens[rb + li];
  const float xg = a.gath[rb + li];
  const float yg = a.gath[qb + rb + li];
  const bool mine = !err0 && tid > 0 && tid < nn;
  const bool badpar = mine && (par < 0 || par >= tid);
  const bool badtok = mine && (tok < 0 || tok >= V);
  // the nodes with children, in every wave (the lanes hold nodes 0..63):
  // only their rows were read by the vocabulary pass
  const bool kid_l = !err0 && lane > 0 && lane < nn && par >= 0 && par < lane;
  const unsigned long long inner_w = wave_or_u64(kid_l ? 1ull << par : 0ull);
  if (!mine || badpar) {
    par = -1;
    tok = 0;
  }
  for (int base = wave * R; base < n_rows; base += kFinWaves * R) {
    const Partial q = base == wave * R ? q0 : load_part(base + sub);
    const int r = base + sub;
    const bool draft = r >= nn;
    const int n = draft ? r - nn : r;
    const bool used = r < n_rows && ((inner_w >> (n & 63)) & 1ull);
    RowStats rs;
    // a wave may hold target and draft rows: the greedy choice is per lane
    const bool g = draft ? gd : gt;
    const bool ok = merge_parts_seg(q, used && part < n_parts, P, g, &rs);
    if (used) {
      if (part == 0) {
        if (draft) {
          s_qrows[n] = rs;
          s_qrowok[n] = ok;
        } else {
          s_rows[n] = rs;
          s_rowok[n] = ok;
        }
      }
      if (!draft && !gt && part < nc)
        s_cm[n * nc + part] = q.s > 0.0 ? scale_pow2(q.s, q.c - rs.c) / rs.s : 0.0;
    }
  }
  if (tid < kMaxNodes) {
    s_par[tid] = par;
    s_tok[tid] = tok;
  }
  __syncthreads();
  if (tid < 64) {   // the nodes with children: a wave OR of the parent bits
    const unsigned long long m = wave_or_u64(par >= 0 ? 1ull << par : 0ull);
    if (tid == 0) s_inner = m;
  }
  __syncthreads();
  if (tid < 64) {
    const unsigned long long inner = s_inner;
    const int n = tid < kMaxNodes ? tid : 0;
    const bool bad_row = tid < nn && !err0 && ((inner >> n) & 1ull) &&
                         (!s_rowok[n] || !s_qrowok[n]);
    const int flags = (__ballot(badpar) ? kRowBadShape : 0) | (__ballot(badtok) ? kRowBadToken : 0) |
                      (__ballot(bad_row) ? kRowNonFinite : 0);
    if (tid == 0) s_flags = err0 | flags;
  }
  __syncthreads();
  const int err = s_flags & kRowErrorMask;
  if (err) {
    tree_error_row(a, b, err);
    return;
  }

  // p and q of each node's token under its parent (float64), and the node's
  // acceptance uniform.
  if (tid > 0 && tid < nn) {
    s_pa[tid] = row_prob(s_rows[par], gt, kt, xg, tok);
    s_qb[tid] = row_prob(s_qrows[par], gd, kd, yg, tok);
    s_uacc[tid] = word_to_uniform(verify_words(a.seed, a.step, rid, (uint32_t)tid).x);
  }
  __syncthreads();

  // The walk.  Every thread runs it on the same values (read from shared
  // memory and made scalar), so its control flow is uniform; thread 0 writes
  // what is shared.
  const int es = DT ? 2 : 4;
  const long long rowbytes = (long long)V * es;
  int node = 0, depth = 0, warn = 0;
  unsigned long long kids;
  WorDist d;
  double lam = 0.0;
  int nex = 0;
  bool have_masses = false;   // s_mass holds the masses of the current weights
  int cached_node = -1;       // the node whose a(v), b(v) s_a, reg_b hold (NC > 0)
  float reg_b[NC ? NC * kPerThread : 1];   // b(v) of cached_node
  // One pass at this node: wor_pass, or from the registers (filled at the
  // node's first pass) wor_pass_r.
  auto pass = [&](bool want_e, float lamf, int t_cur, double* E) -> double {
    if constexpr (NC > 0) {
      if (cached_node != node) {
        cached_node = node;
        return want_e ? wor_fill_total<DT, NC, true>(d, V, s_a, reg_b, lamf, t_cur, s_red, E)
                      : wor_fill_total<DT, NC, false>(d, V, s_a, reg_b, lamf, -1, s_red, E);
      }
      return want_e ? wor_total_r<NC, true>(s_a, reg_b, lamf, s_ex_tok, s_ex_lamf, nex, t_cur,
                                            s_red, E)
                    : wor_total_r<NC, false>(s_a, reg_b, lamf, s_ex_tok, s_ex_lamf, nex, t_cur,
                                             s_red, E);
    } else {
      return want_e ? wor_pass<DT, VEC, true>(d, V, nc, lamf, s_ex_tok, s_ex_lamf, nex, t_cur,
                                              s_mass, s_red, E)
                    : wor_pass<DT, VEC, false>(d, V, nc, lamf, s_ex_tok, s_ex_lamf, nex, t_cur,
                                               s_mass, s_red, E);
    }
  };
  for (;;) {
    kids = __ballot(lane > node && lane < nn && s_par[lane] == node);
    d = wor_dist((const char*)a.target + (rb + node) * rowbytes,
                 (const char*)a.draft + (rb + node) * rowbytes, s_rows[node], s_qrows[node], gt,
                 gd, kt, kd, kids != 0ull);
    lam = 0.0;
    double P = 1.0, Q = 1.0;
    nex = 0;
    have_masses = false;
    int accepted = -1;
    unsigned long long rest = kids;
    while (rest) {
      const int c = __ffsll((long long)rest) - 1;
      rest &= rest - 1ull;
      const int t = uni(s_tok[c]);
      int dupk = -1;
      for (int k = 0; k < nex; ++k)
        if (uni(s_ex_tok[k]) == t) dupk = k;
      const double av = uni(s_pa[c]), bv = uni(s_qb[c]);
      double ratio;
      if (dupk >= 0) {
        // the token already left q: q_j(t) = 0
        warn |= kRowWarnQZero;
        ratio = fmax(av - uni(s_ex_lam[dupk]) * bv, 0.0) > 0.0 ? __builtin_huge_val() : 0.0;
      } else {
        const double pj = fmax(av - lam * bv, 0.0) / P;
        const double qj = Q > 0.0 ? bv / Q : 0.0;
        if (qj > 0.0) {
          ratio = pj / qj;
        } else {
          warn |= kRowWarnQZero;
          ratio = pj > 0.0 ? __builtin_huge_val() : 0.0;
        }
      }
      if (uni(s_uacc[c]) < ratio) {
        accepted = c;
        break;
      }
      // (bounded so that a near-empty q cannot make it infinite: 0 * inf)
      const double mu = fmin(Q > 0.0 ? lam + P / Q : lam, 1.0e300);
      // The draft mass left once t leaves q: Q - q(t) while that difference
      // is well conditioned, else summed over the vocabulary in the pass.
      double E = Q;
      double G;
      if (dupk < 0 && bv > 0.5 * Q) {
        G = uni(pass(true, lam_f32(mu), t, &E));
        E = uni(E);
      } else {
        G = uni(pass(false, lam_f32(mu), -1, nullptr));
        if (dupk < 0) E = Q - bv;
      }
      if (G > 0.0) {
        lam = mu;
        P = G;
        have_masses = true;
      } else {
        warn |= kRowWarnRZero;   // p_j <= q_j everywhere: the residual is empty
        have_masses = false;
      }
      if (dupk < 0) {
        if (tid == 0) {
          s_ex_tok[nex] = t;
          s_ex_lamf[nex] = lam_f32(lam);
          s_ex_lam[nex] = lam;
        }
        ++nex;
      }
      Q = E;
      __syncthreads();
    }
    if (accepted < 0) break;
    if (tid == 0) s_path[depth] = accepted;
    ++depth;
    node = accepted;
  }
  const int stop = node;
  if (!kids) {
    // a leaf: its target row, for the bonus draw (d was formed before it
    // had statistics)
    if (!leaf_row_stats<DT>(d.xrow, V, nc, a.vec_ok, gt, kt, s_leaf, &s_rows[stop],
                            &s_cm[stop * nc], &s_leafok)) {
      tree_error_row(a, b, kRowNonFinite);
      return;
    }
    d = wor_dist(d.xrow, d.xrow, s_rows[stop], s_qrows[stop], gt, gd, kt, kd, false);
  }

  int token;
  if (gt) {
    // p is one-hot at the argmax, and so is every residual of it
    token = s_rows[stop].amax;
  } else {
    if (!kids) {
      // leaf: bonus draw from p
      if (tid < nc) s_mass[tid] = s_cm[stop * nc + tid];
    } else {
      if constexpr (NC > 0) {
        // every child rejected: the chunk masses of the current weights,
        // from the node's cache (its passes formed totals only)
        wor_masses_r<NC>(s_a, reg_b, lam_f32(lam), s_ex_tok, s_ex_lamf, nex, s_mass, s_red);
      } else {
        // the last rejection left p_j as it was: masses of its weights
        if (!have_masses) pass(false, lam_f32(lam), -1, nullptr);
      }
    }
    __syncthreads();
    double R = 0.0;
    for (int j = 0; j < nc; ++j) R += s_mass[j];
    R = uni(R);
    __syncthreads();
    // every child rejected at a cached node: the chosen chunk's weights come
    // from the cache too (the same values as from memory)
    bool from_cache = false;
    if constexpr (NC > 0) from_cache = kids != 0ull && cached_node == stop && R > 0.0;
    if (!(R > 0.0)) {
      // rounding emptied the weights: draw from p
      warn |= kRowWarnRZero;
      if (tid < nc) s_mass[tid] = s_cm[stop * nc + tid];
      d = wor_dist(d.xrow, d.xrow, s_rows[stop], s_qrows[stop], gt, gd, kt, kd, false);
      lam = 0.0;
      nex = 0;
      __syncthreads();
    }
    const double u = word_to_uniform(verify_words(a.seed, a.step, rid, (uint32_t)stop).y);
    choose_chunk(s_mass, nc, u, &s_jc, &s_base, &s_t);
    const int jc = uni(s_jc);
    float w[kPerThread], be[kPerThread];
    if (from_cache) {
      // the weights wor_masses_r left in place of a(v) (this thread's own)
      const float4* cw = (const float4*)(s_a + jc * kChunk + opaque_tid() * kPerThread);
      const float4 lo = cw[0], hi = cw[1];
      w[0] = lo.x; w[1] = lo.y; w[2] = lo.z; w[3] = lo.w;
      w[4] = hi.x; w[5] = hi.y; w[6] = hi.z; w[7] = hi.w;
    } else {
      StopVec<DT> r;
      wor_load<DT, VEC>(d, V, jc, r);
      wor_weights<DT, VEC, false>(d, V, jc, r, lam_f32(lam), s_ex_tok, s_ex_lamf, nex, -1, w, be);
    }
    const double acc = thread_total(w);
    double total;
    const double excl = block_exclusive_scan<kFinWaves>(acc, s_scan, &total);
    token = find_in_chunk(w, jc, s_base, excl, s_t, s_found, s_last);
  }
  __syncthreads();

  for (int i = tid; i < N; i += kFinThreads) {
    a.out_tokens[rb + i] = i < depth ? s_tok[s_path[i]] : (i == depth ? token : -1);
    if (i < N - 1) a.path_nodes[(long long)b * (N - 1) + i] = i < depth ? s_path[i] : -1;
    if (a.p_at) a.p_at[rb + i] = (i > 0 && i < nn) ? (float)s_pa[i] : 0.0f;
  }
  if (tid == 0) {
    a.num_accepted[b] = depth;
    if (a.row_status) a.row_status[b] = warn;
  }
}

// ---------------------------------------------------------------------------
// Host launcher.

hipError_t launch_tree_finish(int dtype, const TreeArgs& a, hipStream_t st) {
  const dim3 grid((unsigned)a.B), block(kFinThreads);
  if (a.mode == 1) {
    // vocabularies of up to kWorCacheChunks chunks keep a(v) in LDS
#define SV_WOR_C(DT_, NC_)                                                   \
  case NC_:                                                                  \
    tree_wor_kernel<DT_, true, NC_><<<grid, block, 0, st>>>(a);              \
    break;
    if (a.vec_ok && a.n_chunks <= kWorCacheChunks) {
      if (dtype == 1) {
        switch (a.n_chunks) { SV_WOR_C(1, 1) SV_WOR_C(1, 2) SV_WOR_C(1, 3) SV_WOR_C(1, 4) }
      } else {
        switch (a.n_chunks) { SV_WOR_C(0, 1) SV_WOR_C(0, 2) SV_WOR_C(0, 3) SV_WOR_C(0, 4) }
      }
    } else if (dtype == 1 && a.vec_ok) tree_wor_kernel<1, true, 0><<<grid, block, 0, st>>>(a);
    else if (dtype == 1) tree_wor_kernel<1, false, 0><<<grid, block, 0, st>>>(a);
    else if (a.vec_ok) tree_wor_kernel<0, true, 0><<<grid, block, 0, st>>>(a);
    else tree_wor_kernel<0, false, 0><<<grid, block, 0, st>>>(a);
#undef SV_WOR_C
  } else {
    if (dtype == 1) tree_kernel<1><<<grid, block, 0, st>>>(a);
    else tree_kernel<0><<<grid, block, 0, st>>>(a);
  }
  return hipGetLastError();
}

}  // namespace sv
