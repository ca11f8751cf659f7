// Drafting helpers on the device, gfx950: the top-k candidates of draft
// rows and the pruning of a drafted candidate forest into the round's tree
// (blog.lonae.com/posts/2026-draft-model-kv-jDwzYp, tree-attention
// paragraphs: every draft position branches into the draft's top-k
// candidates; the tree is pruned by cumulative draft probability up to a
// node budget rather than fully expanded).
//
// draft_topk_kernel: one work item of 1024 threads per row.  A row of up to
// 64 KB is read once from HBM, every thread's four 16-byte loads in flight
// together, and kept in registers as order-preserving keys (larger or
// unaligned rows are re-read from memory by every step).  The softmax
// normaliser at the row's temperature comes first.  L, the k-th largest of
// the threads' largest keys, bounds the top k from below (at least k keys
// are >= L), so the keys >= L are gathered and ranked directly (larger logit
// first, lower id on ties).  When too many keys tie at the top for that, a
// radix select over the row (2 passes of 8 bits for bf16, 4 for fp32) finds
// the k-th largest, and the keys above it and, in index order (each thread
// owns a contiguous range), enough keys equal to it are ranked.
//
// tree_prune_kernel: one work item per batch row; every candidate's depth,
// cumulative log q and sibling rank, its place in the keep order (larger
// cumulative log q, then shallower, earlier parent, lower rank), then a
// breadth-first renumbering of the kept set (at most 63 nodes, one wave),
// level by level.  With log q
// <= 0 the cumulative value never grows along a path, so the first
// n_max - 1 finite candidates of the keep order are closed under parents.
#include <hip/hip_runtime.h>

#include "sv_common.h"
#include "sv_internal.h"

namespace sv {

constexpr int kTopkMax = 64;

// Order-preserving key of a logit's bits, with -0 and +0 one key (they
// compare equal as values; ties go to the lower id).
template <int DT>
__device__ __forceinline__ uint32_t key_of_bits(uint32_t b) {
  if (DT == 1) {
    b = (b & 0x7FFFu) ? b : 0u;
    return (b & 0x8000u) ? (~b & 0xFFFFu) : (b | 0x8000u);
  }
  b = (b & 0x7FFFFFFFu) ? b : 0u;
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
template <int DT>
__device__ __forceinline__ float value_of_key(uint32_t key) {
  if (DT == 1) {
    const uint32_t b = (key & 0x8000u) ? (key & 0x7FFFu) : (~key & 0xFFFFu);
    return __uint_as_float(b << 16);
  }
  return float_from_order_key(key);
}

// Keys of one row, read from memory.
template <int DT>
struct RowKeys {
  const char* row;
  __device__ __forceinline__ uint32_t operator()(int v) const {
    const uint32_t b = DT == 1 ? (uint32_t)((const uint16_t*)row)[v] : ((const uint32_t*)row)[v];
    return key_of_bits<DT>(b);
  }
};

constexpr int kTopkRegVecs = 4;   // 16-byte vectors per thread: rows of up to 64 KB
constexpr int kTopkCand = 1024;          // candidates ranked directly

// Rows re-read from memory (REG false) are bound by the latency of those
// reads: they take 64 registers, so that two rows' work items share a
// compute unit (a few values spill; 1.5x faster than one work item per unit).
template <int DT, bool REG>
__global__ __launch_bounds__(kFinThreads) __attribute__((amdgpu_waves_per_eu(REG ? 1 : 8)))
void draft_topk_kernel(const void* logits, int V, int k, const float* temp, int* tokens,
                       float* logprob) {
  constexpr int kBits = DT == 1 ? 16 : 32;
  constexpr int ES = DT == 1 ? 2 : 4;
  constexpr int EPV = 16 / ES;
  // digit histograms, one per pair of waves (LDS atomics on a concentrated
  // digit distribution contend within a pair only), and their sum
  constexpr int kHists = kFinWaves / 2;
  __shared__ uint32_t s_hists[kHists][256];
  __shared__ uint32_t s_hist[256];
  __shared__ double s_scan[kFinWaves];
  __shared__ float s_wm[kFinWaves];
  __shared__ double s_ws[kFinWaves];
  __shared__ uint32_t s_key[kTopkMax];
  __shared__ int s_idx[kTopkMax];
  __shared__ uint32_t s_sel[2];   // digit chosen, count above it
  __shared__ uint32_t s_tmax[kFinThreads];               // each thread's largest key
  __shared__ float s_cval[kTopkCand];                    // candidates: values >= L
  __shared__ int s_cidx[kTopkCand];

  const int r = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const char* row = (const char*)logits + (long long)r * V * ES;
  const float T = temp ? temp[r] : 1.0f;
  if (!temp_ok(T)) {   // reported as token -1 and a NaN log-probability
    if (tid < k) {
      tokens[(long long)r * k + tid] = -1;
      logprob[(long long)r * k + tid] = __builtin_nanf("");
    }
    return;
  }
  const bool greedy = T == 0.0f;
  const float k2 = greedy ? 0.0f : log2e_over_t(T);
  const RowKeys<DT> key_at{row};

  // REG: this thread's vectors tid + 1024 j, all loads issued together
  // (vectors past the row read vector 0 and are never used), unpacked once
  constexpr int kRegElems = REG ? kTopkRegVecs * EPV : 1;
  float xv[kRegElems];
  bool okv[REG ? kTopkRegVecs : 1];
  if (REG) {
    u32x4_t raw[kTopkRegVecs];
#pragma unroll
    for (int j = 0; j < kTopkRegVecs; ++j) {
      const int vj = tid + j * kFinThreads;
      okv[j] = vj * EPV < V;
      raw[j] = __builtin_nontemporal_load((const u32x4_t*)(row + (long long)(okv[j] ? vj : 0) * 16));
    }
    // keep the unpacking below the last load: otherwise the scheduler starts
    // unpacking the first vector, and waits for it, before the others go out
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < kTopkRegVecs; ++j) {
      const uint32_t w[4] = {raw[j].x, raw[j].y, raw[j].z, raw[j].w};
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        if (DT == 1) {
          xv[j * EPV + 2 * h] = bf16_lo(w[h]);
          xv[j * EPV + 2 * h + 1] = bf16_hi(w[h]);
        } else {
          xv[j * EPV + h] = __uint_as_float(w[h]);
        }
      }
    }
  }
  // element e of this thread's registers is logit (tid + 1024 (e / EPV)) EPV + e % EPV
  auto reg_index = [&](int e) { return (tid + (e / EPV) * kFinThreads) * EPV + e % EPV; };

  // the row maximum and each thread's largest key
  float m = -__builtin_huge_valf();
  uint32_t tmax = 0u;
  if (REG) {
    bool any = false;
#pragma unroll
    for (int e = 0; e < kRegElems; ++e) {
      if (okv[e / EPV]) {
        m = fmaxf(m, xv[e]);
        any = true;
      }
    }
    tmax = any ? key_of_bits<DT>(DT == 1 ? __float_as_uint(m) >> 16 : __float_as_uint(m)) : 0u;
  } else {
    for (int v = tid; v < V; v += kFinThreads) {
      const uint32_t key = key_at(v);
      tmax = max(tmax, key);
      m = fmaxf(m, value_of_key<DT>(key));
    }
  }
  s_tmax[tid] = tmax;
  m = wave_max(m);
  if (lane == 0) s_wm[wave] = m;
  __syncthreads();
  // L = the k-th largest of the waves' largest values (k <= 16; each wave
  // finds it from the 16 values itself) or of the threads' largest keys (a
  // radix select): at least k logits are >= L, so the top k are among them.
  float L;
  if (k <= kFinWaves) {
    const float mw = lane < kFinWaves ? s_wm[lane] : -__builtin_huge_valf();
    int ge = 0;
#pragma unroll
    for (int j = 0; j < kFinWaves; ++j)
      ge += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(mw), j)) >= mw;
    // the largest wave maximum with at least k wave maxima at or above it
    L = wave_max((lane < kFinWaves && ge >= k) ? mw : -__builtin_huge_valf());
  }
  m = s_wm[0];
  for (int w = 1; w < kFinWaves; ++w) m = fmaxf(m, s_wm[w]);
  // softmax normaliser: the sum of 2^((x - m) k2), eight terms at a time in
  // float32 (pairwise), then in float64
  double s = 0.0;
  if (!greedy) {
    if (REG) {
#pragma unroll
      for (int j = 0; j < kTopkRegVecs; ++j) {
        float t[EPV];
#pragma unroll
        for (int h = 0; h < EPV; ++h) t[h] = exp2_hw((xv[j * EPV + h] - m) * k2);
#pragma unroll
        for (int w2 = EPV / 2; w2 >= 1; w2 >>= 1) {
#pragma unroll
          for (int h = 0; h < w2; ++h) t[h] = t[2 * h] + t[2 * h + 1];
        }
        if (okv[j]) s += (double)t[0];
      }
    } else {
      for (int v = tid; v < V; v += kFinThreads)
        s += (double)exp2_hw((value_of_key<DT>(key_at(v)) - m) * k2);
    }
  }
  s = wave_sum(s);
  if (lane == 0) s_ws[wave] = s;
  // the rank-th output: token and log softmax(x / T) (s_ws is read after a
  // barrier on every path)
  auto write_out = [&](int rank, float x, int idx) {
    double S = 0.0;
    for (int w = 0; w < kFinWaves; ++w) S += s_ws[w];
    double lp;
    if (greedy) lp = rank == 0 ? 0.0 : -__builtin_huge_val();
    else lp = ((double)x - (double)m) * ((double)k2 / kLog2e) - log(S);
    tokens[(long long)r * k + rank] = idx;
    logprob[(long long)r * k + rank] = (float)lp;
  };

  // Radix select of the k-th largest of n keys, 8 bits at a time from the
  // top: the key, and how many keys equal to it are needed beside the ones
  // above it.
  auto radix_kth = [&](auto key_of, int n, uint32_t* need_out) -> uint32_t {
  uint32_t prefix = 0u, need = (uint32_t)k;
  for (int shift = kBits - 8; shift >= 0; shift -= 8) {
    for (int i = tid; i < kHists * 256; i += kFinThreads) (&s_hists[0][0])[i] = 0u;
    __syncthreads();
    const uint32_t hi_mask = shift + 8 >= 32 ? 0u : (0xFFFFFFFFu << (shift + 8));
    uint32_t* hist = s_hists[wave >> 1];
    for (int v = tid; v < n; v += kFinThreads) {
      const uint32_t key = key_of(v);
      if ((key & hi_mask) == (prefix & hi_mask)) atomicAdd(&hist[(key >> shift) & 0xFFu], 1u);
    }
    __syncthreads();
    if (tid < 256) {
      uint32_t t = 0u;
#pragma unroll
      for (int h = 0; h < kHists; ++h) t += s_hists[h][tid];
      s_hist[tid] = t;
    }
    __syncthreads();
    if (wave == 0) {
      // digit d with count(> d) < need <= count(>= d), scanning from the top
      uint32_t c[4], tot = 0u;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        c[j] = s_hist[255 - (lane * 4 + j)];
        tot += c[j];
      }
      const double incl = wave_inclusive_scan((double)tot);
      uint32_t above = (uint32_t)(incl - (double)tot);
      int found = -1;
      uint32_t above_found = 0u;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (found < 0 && above < need && above + c[j] >= need) {
          found = 255 - (lane * 4 + j);
          above_found = above;
        }
        above += c[j];
      }
      const unsigned long long hit = __ballot(found >= 0);
      const int src = hit ? __ffsll((long long)hit) - 1 : 0;
      const int d = __shfl(found, src);
      const uint32_t ab = __shfl(above_found, src);
      if (lane == 0) {
        s_sel[0] = (uint32_t)max(d, 0);
        s_sel[1] = ab;
      }
    }
    __syncthreads();
    prefix |= s_sel[0] << shift;
    need -= s_sel[1];
  }
  *need_out = need;
  return prefix;
  };

  if (k > kFinWaves) {
    uint32_t need_l;
    L = value_of_key<DT>(radix_kth([&](int v) { return s_tmax[v]; }, kFinThreads, &need_l));
  }
  uint32_t n_cand = 0u;
  if (REG) {
#pragma unroll
    for (int e = 0; e < kRegElems; ++e) n_cand += okv[e / EPV] && xv[e] >= L;
  } else {
    for (int v = tid; v < V; v += kFinThreads) n_cand += value_of_key<DT>(key_at(v)) >= L;
  }
  double c_tot;
  const uint32_t c_pos = (uint32_t)block_exclusive_scan<kFinWaves>((double)n_cand, s_scan, &c_tot);
  const int C = (int)c_tot;
  if (C <= kTopkCand) {
    uint32_t at = c_pos;
    auto put = [&](float x, int v) {
      s_cval[at] = x;
      s_cidx[at] = v;
      ++at;
    };
    if (REG) {
#pragma unroll
      for (int e = 0; e < kRegElems; ++e)
        if (okv[e / EPV] && xv[e] >= L) put(xv[e], reg_index(e));
    } else {
      for (int v = tid; v < V; v += kFinThreads) {
        const float x = value_of_key<DT>(key_at(v));
        if (x >= L) put(x, v);
      }
    }
    __syncthreads();
    // rank: larger value first, lower id on ties
    if (tid < C) {
      const float x = s_cval[tid];
      const int idx = s_cidx[tid];
      int rank = 0;
      for (int j = 0; j < C; ++j) {
        const float xj = s_cval[j];
        rank += xj > x || (xj == x && s_cidx[j] < idx);
      }
      if (rank < k) {
        s_key[rank] = __float_as_uint(x);
        s_idx[rank] = idx;
      }
    }
    __syncthreads();
    if (tid < k) write_out(tid, __uint_as_float(s_key[tid]), s_idx[tid]);
    return;
  }

  // Many keys tie at the top: radix select over the whole row (read from
  // memory again).
  uint32_t need;
  const uint32_t thr = radix_kth(key_at, V, &need);   // the k-th largest; `need` equal keys
  // keys above the threshold (fewer than k, any order), and the equal keys of
  // lowest index: each thread owns a contiguous range for the latter
  const int E = (V + kFinThreads - 1) / kFinThreads;
  const int v0 = min(tid * E, V), v1 = min(v0 + E, V);
  uint32_t n_above = 0u, n_eq = 0u;
  for (int v = v0; v < v1; ++v) {
    const uint32_t key = key_at(v);
    n_above += key > thr;
    n_eq += key == thr;
  }
  double tot_above;
  const uint32_t pos_above =
      (uint32_t)block_exclusive_scan<kFinWaves>((double)n_above, s_scan, &tot_above);
  double tot_eq;
  const uint32_t pos_eq = (uint32_t)block_exclusive_scan<kFinWaves>((double)n_eq, s_scan, &tot_eq);
  uint32_t pa = pos_above, pe = pos_eq;
  for (int v = v0; v < v1; ++v) {
    const uint32_t key = key_at(v);
    if (key > thr) {
      s_key[pa] = key;
      s_idx[pa] = v;
      ++pa;
    } else if (key == thr) {
      if (pe < need) {
        const uint32_t at = (uint32_t)tot_above + pe;
        s_key[at] = key;
        s_idx[at] = v;
      }
      ++pe;
    }
  }
  __syncthreads();
  // rank the k entries: larger key first, lower index on ties
  if (tid < k) {
    const uint32_t key = s_key[tid];
    const int idx = s_idx[tid];
    int rank = 0;
    for (int j = 0; j < k; ++j) {
      const uint32_t kj = s_key[j];
      rank += kj > key || (kj == key && s_idx[j] < idx);
    }
    write_out(rank, value_of_key<DT>(key), idx);
  }
}

constexpr int kPruneMax = 1024;   // candidates per batch row

__global__ __launch_bounds__(kFinThreads) void tree_prune_kernel(TreePruneArgs a) {
  __shared__ __align__(16) int s_par[kPruneMax];
  __shared__ int s_depth[kPruneMax], s_rank[kPruneMax], s_new[kPruneMax];
  __shared__ __align__(16) double s_cum[kPruneMax];
  __shared__ int s_before[kPruneMax];   // candidates ahead in the keep order
  __shared__ int s_cnt[kPruneMax], s_off[kPruneMax], s_cur[kPruneMax], s_list[kPruneMax];
  static_assert(kFinThreads == kPruneMax, "one thread per candidate and per parent slot");
  __shared__ int s_klist[64];
  __shared__ __align__(16) uint32_t s_tie[kPruneMax];
  __shared__ double s_scan[kFinWaves];
  __shared__ int s_bad, s_maxd, s_pass;

  const int b = blockIdx.x, tid = threadIdx.x;
  const int C = min(a.n_cand ? a.n_cand[b] : a.C, a.C);
  const long long cb = (long long)b * a.C;
  if (tid == 0) {
    s_bad = C < 0;
    s_maxd = 0;
    s_pass = 0;
  }
  __syncthreads();
  const int i = tid;
  const bool mine = i < C;
  int par = -1;
  double lq = 0.0;
  if (mine) {
    par = a.cand_parent[cb + i];
    lq = (double)a.cand_logq[cb + i];
    if (par < -1 || par >= i) s_bad = 1;
    s_par[i] = par;
  }
  __syncthreads();
  const bool bad = s_bad != 0;
  // Each parent's children (slot par + 1; -1 is the roots' parent), listed
  // in no particular order: counts by LDS atomics, offsets by a block scan,
  // then slots taken through per-parent cursors.
  s_cnt[tid] = 0;
  s_cur[tid] = 0;
  __syncthreads();
  if (mine && !bad) atomicAdd(&s_cnt[par + 1], 1);
  __syncthreads();
  double n_tot;
  s_off[tid] = (int)block_exclusive_scan<kFinWaves>((double)s_cnt[tid], s_scan, &n_tot);
  __syncthreads();
  if (mine && !bad) s_list[s_off[par + 1] + atomicAdd(&s_cur[par + 1], 1)] = i;
  __syncthreads();
  // depth (walk to the root) and rank among the siblings (the siblings of
  // smaller index, from the parent's list)
  int depth = 0, rank = 0;
  if (mine && !bad) {
    for (int x = i; x >= 0; x = s_par[x]) ++depth;
    const int o = s_off[par + 1], n = s_cnt[par + 1];
    for (int k = 0; k < n; ++k) rank += s_list[o + k] < i;
    s_depth[i] = depth;
    s_rank[i] = rank;
  }
  {
    // the deepest candidate: a wave maximum, then one LDS atomic per wave
    const int wm = (int)wave_max_u64((unsigned long long)depth);
    if ((tid & 63) == 0 && wm > 0) atomicMax(&s_maxd, wm);
  }
  __syncthreads();
  const int maxd = bad ? 0 : min(s_maxd, kPruneMax);
  // cumulative log q, one level at a time: parent's value plus the node's
  double cum = 0.0;
  for (int d = 1; d <= maxd; ++d) {
    if (mine && !bad && depth == d) {
      cum = (par < 0 ? 0.0 : s_cum[par]) + lq;
      s_cum[i] = cum;
    }
    __syncthreads();
  }
  // place in the keep order; kept if finite and among the first n_max - 1.
  // The tie order (depth, parent, rank) packs into one word: 11, 11, 10 bits.
  if (mine && !bad) s_tie[i] = ((uint32_t)depth << 21) | ((uint32_t)(par + 1) << 10) | (uint32_t)rank;
  const int C8 = (C + 7) & ~7;
  if (i >= C && i < C8) {   // the pad entries read by the eight-wide loop
    s_cum[i] = -__builtin_huge_val();
    s_tie[i] = 0xFFFFFFFFu;
  }
  if (i < C) s_before[i] = 0;
  __syncthreads();
  // The candidates ahead of each one, counted by G groups of threads (as
  // many as the block holds, each share at least eight wide), each over its
  // share of the candidates; the shares are summed by LDS atomics.
  if (!bad && C > 0) {
    const int G = max(1, min(kFinThreads / C, C8 / 8));
    const int S = ((C8 + 8 * G - 1) / (8 * G)) * 8;
    const int ci = tid % C, g = tid / C;
    if (g < G) {
      const double cum_c = s_cum[ci];
      const uint32_t tie = s_tie[ci];
      int before = 0;
      // eight candidates per step, all loads unconditional (the arrays are
      // padded past C with entries that never count: -inf and the largest tie)
      const int j1 = min(g * S + S, C8);
      for (int j = g * S; j < j1; j += 8) {
        double2 c2[4];
        uint2 t2[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          c2[u] = ((const double2*)s_cum)[(j >> 1) + u];
          t2[u] = ((const uint2*)s_tie)[(j >> 1) + u];
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          before += (c2[u].x > cum_c) | ((c2[u].x == cum_c) & (t2[u].x < tie));
          before += (c2[u].y > cum_c) | ((c2[u].y == cum_c) & (t2[u].y < tie));
        }
      }
      if (before) atomicAdd(&s_before[ci], before);
    }
  }
  __syncthreads();
  int keep = 0;
  if (mine && !bad) {
    keep = cum > -__builtin_huge_val() && s_before[i] < a.n_max - 1;
    s_new[i] = -1;
  }
  __syncthreads();
  // breadth-first numbering of the kept nodes (at most 63), gathered in keep
  // order, by one wave, level by level: (depth, new parent index, rank)
  double k_tot;
  const int kpos = (int)block_exclusive_scan<kFinWaves>((double)(keep ? 1 : 0), s_scan, &k_tot);
  const int K = (int)k_tot;
  if (keep) s_klist[kpos] = i;
  __syncthreads();
  if (tid < 64) {
    const int q = tid;
    const int ci = q < K ? s_klist[q] : 0;
    const int dq = q < K ? s_depth[ci] : 0;
    const int pq = q < K ? s_par[ci] : -1;
    const int rq = q < K ? s_rank[ci] : 0;
    int base = 1;
    for (int d = 1; d <= maxd; ++d) {
      const bool here = q < K && dq == d;
      // this level's order key: the parent's new index (numbered at the level
      // above), then the sibling rank; the other lanes get a key that never
      // counts
      const int np = pq < 0 ? 0 : (here ? s_new[pq] : 0);
      const uint32_t key = here ? ((uint32_t)np << 10) | (uint32_t)rq : 0xFFFFFFFFu;
      // every lane, unrolled: a lane not at this level holds a key that
      // never counts
      int pos = 0;
#pragma unroll
      for (int j = 0; j < 64; ++j) pos += (uint32_t)__builtin_amdgcn_readlane((int)key, j) < key;
      const int n_here = __popcll(__ballot(here));
      if (here) s_new[ci] = base + pos;
      base += n_here;
    }
  }
  __syncthreads();
  const int base = 1 + K;
  const int n = bad ? 0 : base;
  const long long ob = (long long)b * a.n_max;
  if (mine && !bad && keep) {
    const int ni = s_new[i];
    a.parents[ob + ni] = par < 0 ? 0 : s_new[par];
    a.tokens[ob + ni] = a.cand_token[cb + i];
    a.cum_logprob[ob + ni] = (float)cum;
  }
  {
    // kept nodes of cumulative probability >= tau: a count per wave
    const int np = __popcll(__ballot(mine && !bad && keep && exp(cum) >= a.tau));
    if ((tid & 63) == 0 && np > 0) atomicAdd(&s_pass, np);
  }
  if (tid == 0 && !bad) {
    a.parents[ob] = -1;
    a.tokens[ob] = -1;
    a.cum_logprob[ob] = 0.0f;
  }
  for (int j = tid; j < a.n_max; j += kFinThreads) {
    if (j >= n && (j > 0 || bad)) {
      a.parents[ob + j] = -1;
      a.tokens[ob + j] = -1;
      a.cum_logprob[ob + j] = -__builtin_huge_valf();
    }
  }
  __syncthreads();
  if (tid == 0) {
    a.n_nodes[b] = n;
    if (a.n_pass) a.n_pass[b] = bad ? 0 : s_pass;
  }
}

// Small top-k (k <= 4) of bf16 rows of up to 32768 logits, aligned: one work
// item of 256 threads per row, so that four rows share a compute unit
// and their loads and ALU work overlap.  Each thread keeps its 16 vectors
// (128 logits) packed in registers.  Each wave gathers its logits at or
// above its own bound (the k-th largest of its threads' maxima), and after
// one barrier one wave ranks all of them (larger value first, lower id on
// ties).  More than kTopkWaveCand of them in one wave (ties at the top)
// take k rounds of a block-wide argmax instead.  The softmax normaliser is
// formed online in the same pass as the maximum, so each pair of vectors is
// reduced as it arrives.
constexpr int kTopkSmallThreads = 256;
constexpr int kTopkSmallWaves = kTopkSmallThreads / 64;
constexpr int kTopkSmallVecs = 16;                     // 16-byte vectors per thread
constexpr int kTopkSmallK = kTopkSmallWaves;           // k <= the waves' count
constexpr int kTopkSmallMaxV = kTopkSmallVecs * kTopkSmallThreads * 8;
constexpr int kTopkWaveCand = kTopkCand / kTopkSmallWaves;   // candidates ranked per wave

__global__ __launch_bounds__(kTopkSmallThreads) void draft_topk_small_kernel(
    const void* logits, int V, int k, const float* temp, int* tokens, float* logprob) {
  __shared__ float s_wc[kTopkSmallWaves];
  __shared__ double s_ws[kTopkSmallWaves];
  __shared__ unsigned long long s_wk[kTopkSmallWaves];
  __shared__ unsigned long long s_top[kTopkSmallK];
  __shared__ uint32_t s_ckey[kTopkSmallWaves][kTopkWaveCand];   // each wave's candidates' keys
  __shared__ uint32_t s_wn[kTopkSmallWaves];                      // and their count

  const int r = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const char* row = (const char*)logits + (long long)r * V * 2;
  // every load is issued before anything waits: the temperature as a scalar
  const float T = temp ? load_uniform_f32(temp + r) : 1.0f;
  u32x4_t raw[kTopkSmallVecs];
#pragma unroll
  for (int j = 0; j < kTopkSmallVecs; ++j) {
    const int vj = tid + j * kTopkSmallThreads;
    raw[j] = __builtin_nontemporal_load((const u32x4_t*)(row + (long long)(vj * 8 < V ? vj : 0) * 16));
  }
  __builtin_amdgcn_sched_barrier(0);
  if (!temp_ok(T)) {   // reported as token -1 and a NaN log-probability
    if (tid < k) {
      tokens[(long long)r * k + tid] = -1;
      logprob[(long long)r * k + tid] = __builtin_nanf("");
    }
    return;
  }
  const bool greedy = T == 0.0f;
  const float k2 = greedy ? 0.0f : log2e_over_t(T);
  // logit h of vector j: element (tid + 256 j) 8 + h
  auto val = [&](int j, int h) -> float {
    const int q = h >> 1;
    const uint32_t word = q == 0 ? raw[j].x : (q == 1 ? raw[j].y : (q == 2 ? raw[j].z : raw[j].w));
    return (h & 1) ? bf16_hi(word) : bf16_lo(word);
  };
  auto valid = [&](int j) { return (tid + j * kTopkSmallThreads) * 8 < V; };
  auto index = [&](int j, int h) { return (tid + j * kTopkSmallThreads) * 8 + h; };
  // the packed words as values the compiler cannot reuse across phases: each
  // phase unpacks them again (one operation per logit) instead of keeping
  // 128 unpacked floats live
  auto fence_raw = [&]() {
#pragma unroll
    for (int j = 0; j < kTopkSmallVecs; ++j) asm volatile("" : "+v"(raw[j]));
  };

  // One pass as the vectors arrive (loads complete in issue order): the row
  // maximum and, online, the softmax normaliser: a running integer offset
  // c = ceil(max x k2) and the sum of 2^(x k2 - c), sixteen terms (two
  // vectors) pairwise in float32 and then in float64, rescaled by exact
  // powers of two when c grows.
  // No branch in this loop: a load whose value crosses a branch join is
  // waited for at the join, which would make the first vector wait for all
  // of them.  A vector past V (its load reads the row's first vector) has
  // maximum -inf and sum 0, by two selects; a greedy row (k2 = 0) forms its
  // offsets with k2 = 1 and never reads the sum.
  const float kc = greedy ? 1.0f : k2;
  float m = -__builtin_huge_valf(), c = -__builtin_huge_valf();
  double sacc = 0.0;
  // each pair of vectors' maxima, as two bf16 (a maximum of bf16 values is one)
  uint32_t vmp[kTopkSmallVecs / 2];
  // two vectors per step: one offset update and one float64 add per 16 logits
#pragma unroll
  for (int j = 0; j < kTopkSmallVecs; j += 2) {
    float xv[16];
    float mp = -__builtin_huge_valf();
    float mq[2];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
#pragma unroll
      for (int h = 0; h < 8; ++h) xv[8 * q + h] = val(j + q, h);
      float mj = xv[8 * q];
#pragma unroll
      for (int h = 1; h < 8; ++h) mj = fmaxf(mj, xv[8 * q + h]);
      // a vector past V (loaded from the row's start) counts for nothing:
      // its maximum is -inf and its sum 0
      mj = valid(j + q) ? mj : -__builtin_huge_valf();
      mq[q] = mj;
      mp = fmaxf(mp, mj);
    }
    // the two maxima's high halves (bytes 2, 3 of each) in one word
    vmp[j / 2] = __builtin_amdgcn_perm(__float_as_uint(mq[1]), __float_as_uint(mq[0]), 0x07060302u);
    m = fmaxf(m, mp);
    const float cn = fmaxf(c, ceilf(mp * kc));
    // the sum is 0 while c is -inf, so its rescale needs no test
    sacc = scale_pow2(sacc, c - cn);
    c = cn;
    // all -inf so far: the offset -FLT_MAX keeps the terms 2^-inf = 0
    const float cu = fmaxf(c, -__FLT_MAX__);
#pragma unroll
    for (int h = 0; h < 16; ++h) xv[h] = exp2_hw(fmaf(xv[h], kc, -cu));
#pragma unroll
    for (int w2 = 8; w2 >= 2; w2 >>= 1) {
#pragma unroll
      for (int h = 0; h < w2; ++h) xv[h] = xv[2 * h] + xv[2 * h + 1];
    }
    // xv[0], xv[1]: the two vectors' sums
    sacc += (double)((valid(j) ? xv[0] : 0.0f) + (valid(j + 1) ? xv[1] : 0.0f));
  }
  fence_raw();
  // Each wave bounds its own candidates: Lw, the k-th largest of its
  // threads' maxima (each a bf16 value, never NaN), which at least k of the
  // wave's logits reach.  A logit of the wave below Lw has k larger ones, so
  // the row's top k lie among the waves' logits >= their own bounds, and no
  // barrier comes before the gather.  Lane keys: the maximum's order key
  // above the lane; k rounds of a wave-wide maximum, each below the last.
  const uint32_t mkey = (key_of_bits<1>(__float_as_uint(m) >> 16) << 6) | (uint32_t)lane;
  uint32_t below_m = ~0u, key_top = 0u, key_kth = 0u;
#pragma unroll
  for (int i = 0; i < kTopkSmallK; ++i) {
    const uint32_t best = wave_max_u32(mkey < below_m ? mkey : 0u);
    key_top = i == 0 ? best : key_top;
    key_kth = i < k ? best : key_kth;
    below_m = best;
  }
  const float L = value_of_key<1>(key_kth >> 6);
  // the wave's maximum, offset and normaliser (the sum brought to the wave's
  // offset); a thread's offset is ceil(m kc) (the rounded product is
  // monotone in m), so the wave's offset follows from the wave's maximum
  const float mw = value_of_key<1>(key_top >> 6);
  const float cw = ceilf(mw * kc);
  const double sw = wave_sum(sacc != 0.0 ? scale_pow2(sacc, c - cw) : 0.0);
  // the row's offset and normaliser, from the waves' (after the barrier):
  // sum_v 2^(x_v k2 - c_row), the waves' sums in wave order
  float c_row = 0.0f;
  double S = 0.0;
  auto row_normaliser = [&]() {
    const bool wl = lane < kTopkSmallWaves;
    const float cwl = wl ? s_wc[lane] : -__builtin_huge_valf();
    const double swl = wl ? s_ws[lane] : 0.0;
    c_row = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(cwl), 0));
#pragma unroll
    for (int w = 1; w < kTopkSmallWaves; ++w)
      c_row = fmaxf(c_row, __int_as_float(__builtin_amdgcn_readlane(__float_as_int(cwl), w)));
    const double swr = swl != 0.0 ? scale_pow2(swl, cwl - c_row) : 0.0;
#pragma unroll
    for (int w = 0; w < kTopkSmallWaves; ++w) S += readlane_f64(swr, w);
  };
  // the rank-th output: token and log softmax(x / T) = (x k2 - c_row) ln 2 - ln S
  // (ln S is formed by the writing wave only, after the ranking's barrier)
  auto write_out = [&](int rank, float x, int idx, double lnS) {
    double lp;
    if (greedy) lp = rank == 0 ? 0.0 : -__builtin_huge_val();
    else lp = ((double)x * (double)k2 - (double)c_row) * (1.0 / kLog2e) - lnS;
    tokens[(long long)r * k + rank] = idx;
    logprob[(long long)r * k + rank] = (float)lp;
  };

  // the wave's logits >= L; only a vector whose maximum reaches L can hold
  // one.  Each wave gathers its own candidates into its
  // LDS slots (ballots give the positions: no atomics, no count pass), as
  // 32-bit keys that order them: the value's order key above the complement
  // of the id (ids stay below 2^15), so a larger key ranks higher and -0 and
  // +0 tie on the value.
  uint32_t vmask = 0u;
#pragma unroll
  for (int j = 0; j < kTopkSmallVecs; ++j) {
    const float vm = (j & 1) ? bf16_hi(vmp[j / 2]) : bf16_lo(vmp[j / 2]);
    vmask |= (uint32_t)(vm >= L) << j;
  }
  // this thread's vectors inside the row: the first n_in (0..16)
  const int n_in = (V / 8 - tid + kTopkSmallThreads - 1) / kTopkSmallThreads;
  vmask &= (1u << n_in) - 1u;
  uint32_t n_w = 0u;   // the wave's candidates so far (the same in every lane)
#pragma unroll
  for (int j = 0; j < kTopkSmallVecs; ++j) {
    const bool vj = (vmask >> j) & 1u;
    if (__ballot(vj) != 0ull) {
      // the vector's logits >= L as bits, then one slot per set bit: each
      // round places every lane's lowest remaining bit (ballot positions)
      uint32_t m8 = 0u;
#pragma unroll
      for (int h = 0; h < 8; ++h) m8 |= (uint32_t)(val(j, h) >= L) << h;
      m8 = vj ? m8 : 0u;
      for (;;) {
        const unsigned long long bal = __ballot(m8 != 0u);
        if (bal == 0ull) break;
        if (m8 != 0u) {
          const int h = __builtin_ctz(m8);
          m8 &= m8 - 1u;
          const uint32_t at =
              n_w + __builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32),
                                              __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u));
          // the word of logit h: two selects on the bits of h / 2
          const uint32_t w01 = (h & 2) ? raw[j].y : raw[j].x;
          const uint32_t w23 = (h & 2) ? raw[j].w : raw[j].z;
          const uint32_t word = (h & 4) ? w23 : w01;
          const uint32_t bits = (h & 1) ? word >> 16 : word & 0xFFFFu;
          if (at < (uint32_t)kTopkWaveCand)
            s_ckey[wave][at] = (key_of_bits<1>(bits) << 15) | (0x7FFFu - (uint32_t)index(j, h));
        }
        n_w += (uint32_t)__popcll(bal);
      }
    }
  }
  fence_raw();
  if (lane == 0) {
    s_wc[wave] = cw;
    s_ws[wave] = sw;
    s_wn[wave] = n_w;
  }
  __syncthreads();
  uint32_t n_max = s_wn[0];
#pragma unroll
  for (int w = 1; w < kTopkSmallWaves; ++w) n_max = max(n_max, s_wn[w]);
  if (n_max <= (uint32_t)kTopkWaveCand) {
    // one wave ranks them: k rounds of a wave-wide maximum of the keys, each
    // below the previous winner (a key is never 0: NaN is no candidate).
    // Lane l reads the candidates of wave l / 16, from entry l % 16 on.
    if (wave != 0) return;
    row_normaliser();
    const int cwv = lane >> 4, e0 = lane & 15;
    const int nw = (int)s_wn[cwv];
    const uint32_t first = e0 < nw ? s_ckey[cwv][e0] : 0u;
    uint32_t below = ~0u, top = 0u;
    double lnS;
    if (n_max <= 16u) {
      // one candidate a lane at most: straight-line rounds, ln S beside them
      lnS = log(S);
#pragma unroll
      for (int i = 0; i < kTopkSmallK; ++i) {
        const uint32_t best = wave_max_u32(first < below ? first : 0u);
        top = (i < k && lane == i) ? best : top;
        below = best;
      }
    } else {
      lnS = log(S);
      for (int i = 0; i < k; ++i) {
        uint32_t best = first < below ? first : 0u;
        for (int e = e0 + 16; e < nw; e += 16) {
          const uint32_t key = s_ckey[cwv][e];
          best = (key < below && key > best) ? key : best;
        }
        best = wave_max_u32(best);
        top = lane == i ? best : top;
        below = best;
      }
    }
    if (lane < k && top != 0u)
      write_out(lane, value_of_key<1>(top >> 15), (int)(0x7FFFu - (top & 0x7FFFu)), lnS);
    return;
  }
  // More than kTopkWaveCand logits of one wave tie at the top: k rounds of
  // a block-wide argmax over the row, read again from memory (this path is
  // rare), each below the previous winner, on keys (order key of the value,
  // then the complement of the index: lower id wins a tie).
  row_normaliser();
  const RowKeys<1> key_at{row};
  unsigned long long below = ~0ull;
  for (int i = 0; i < k; ++i) {
    unsigned long long best = 0ull;
    for (int v = tid; v < V; v += kTopkSmallThreads) {
      const unsigned long long key =
          ((unsigned long long)key_at(v) << 32) | (0xFFFFFFFFu - (uint32_t)v);
      if (key < below && key > best) best = key;
    }
    best = wave_max_u64(best);
    if (lane == 0) s_wk[wave] = best;
    __syncthreads();
    unsigned long long b = s_wk[0];
#pragma unroll
    for (int w = 1; w < kTopkSmallWaves; ++w) b = s_wk[w] > b ? s_wk[w] : b;
    if (tid == 0) s_top[i] = b;
    below = b;
    __syncthreads();
  }
  if (tid < k) {
    const unsigned long long b = s_top[tid];
    write_out(tid, value_of_key<1>((uint32_t)(b >> 32)), (int)(0xFFFFFFFFu - (uint32_t)b), log(S));
  }
}

hipError_t launch_draft_topk(int dtype, const void* logits, int R, int V, int k, const float* temp,
                             int* tokens, float* logprob, hipStream_t st) {
  const int es = dtype == 1 ? 2 : 4;
  const bool vec_ok = ((long long)V * es) % 16 == 0 && ((uintptr_t)logits & 15u) == 0;
  // keys in registers: aligned rows of up to 4 vectors per thread
  const bool reg = vec_ok && (long long)V * es <= (long long)kTopkRegVecs * kFinThreads * 16;
  const dim3 grid((unsigned)R), block(kFinThreads);
  if (dtype == 1 && vec_ok && V <= kTopkSmallMaxV && k <= kTopkSmallK) {
    draft_topk_small_kernel<<<grid, dim3(kTopkSmallThreads), 0, st>>>(logits, V, k, temp, tokens,
                                                                      logprob);
    return hipGetLastError();
  }
  if (dtype == 1) {
    if (reg) draft_topk_kernel<1, true><<<grid, block, 0, st>>>(logits, V, k, temp, tokens, logprob);
    else draft_topk_kernel<1, false><<<grid, block, 0, st>>>(logits, V, k, temp, tokens, logprob);
  } else {
    if (reg) draft_topk_kernel<0, true><<<grid, block, 0, st>>>(logits, V, k, temp, tokens, logprob);
    else draft_topk_kernel<0, false><<<grid, block, 0, st>>>(logits, V, k, temp, tokens, logprob);
  }
  return hipGetLastError();
}

hipError_t launch_tree_prune(const TreePruneArgs& a, hipStream_t st) {
  tree_prune_kernel<<<dim3((unsigned)a.B), dim3(kFinThreads), 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace sv
