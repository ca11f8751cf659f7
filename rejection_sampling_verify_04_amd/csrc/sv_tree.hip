// Finish pass of the tree verify, gfx950: one work item per tree walks it
// with one lane per node and draws in one chunk of the stop row.
//
// Sources: tree walk over top-k siblings (kwkr.cn/news/620872 §5.3;
// blog.lonae.com/posts/2026-draft-model-kv-jDwzYp, tree-attention
// paragraphs); acceptance rule and residual draw as in the linear verify
// (kwkr §2.3, §4.1; lonae formal-definition paragraph).
#include <hip/hip_ext.h>

#include <algorithm>

#include "sv_common.h"
#include "sv_internal.h"
#include "sv_finish.h"

namespace sv {

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
// Host launcher.

hipError_t launch_tree_finish(int dtype, const TreeArgs& a, hipStream_t st) {
  if (dtype == 1) tree_kernel<1><<<dim3((unsigned)a.B), dim3(kFinThreads), 0, st>>>(a);
  else tree_kernel<0><<<dim3((unsigned)a.B), dim3(kFinThreads), 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace sv
