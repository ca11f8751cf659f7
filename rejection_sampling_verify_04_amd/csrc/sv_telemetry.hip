// Round telemetry of the verify step, gfx950: counters accumulated on the
// device over a window of calls, and the derived health signals.
//
// The signals are those blog.lonae.com/posts/2026-draft-model-kv-jDwzYp
// names for a speculative deployment (observability paragraphs): the
// acceptance rate with a per-request histogram that keeps the low and the
// high peak apart, Speculative Efficiency = acceptance_rate *
// avg_accepted_tokens / draft_steps, and Tree Width Effective = paths hit /
// paths offered.  draft_steps of a round is gamma for a linear row and the
// depth of the deepest node for a tree; a tree path is hit when the round
// accepted its first node below the root.
//
// Linear rows: one thread per row; the counters every row adds to are summed
// per wave first, the histogram bins counted in LDS; one device-scope atomic
// add per non-zero counter per work item.
#include <hip/hip_runtime.h>

#include "spec_verify.h"
#include "sv_common.h"
#include "sv_internal.h"

namespace sv {

constexpr int kTmFields = 7;
constexpr int kTmCounters = kTmFields + SV_TELEM_ACC_BINS + SV_TELEM_POS_BINS + SV_TELEM_RANK_BINS;
static_assert(sizeof(sv_telemetry) == kTmCounters * sizeof(uint64_t), "flat counter block");
constexpr int kTmRounds = 0, kTmErrors = 1, kTmDrafted = 2, kTmAccepted = 3, kTmFull = 4,
              kTmPaths = 5, kTmPathsHit = 6, kTmRate = kTmFields,
              kTmPos = kTmRate + SV_TELEM_ACC_BINS, kTmRank = kTmPos + SV_TELEM_POS_BINS;

// Bin of n / g (g > 0): the k with k / 20 <= n / g < (k + 1) / 20, in integers.
__device__ __forceinline__ int rate_bin(int n, int g) {
  return min(SV_TELEM_ACC_BINS - 1, (SV_TELEM_ACC_BINS * n) / g);
}

__global__ __launch_bounds__(256) void telemetry_linear_kernel(const int* num_accepted,
                                                               const int* off, int B,
                                                               unsigned long long* acc) {
  __shared__ uint32_t s_c[kTmCounters];
  for (int i = threadIdx.x; i < kTmCounters; i += 256) s_c[i] = 0u;
  __syncthreads();
  const int b = blockIdx.x * 256 + threadIdx.x;
  const int bc = b < B ? b : B - 1;   // clamped: every lane loads
  const int n = num_accepted[bc];
  const int g = off[bc + 1] - off[bc];
  const bool err = b < B && (n < 0 || g < 0 || n > g);
  const bool ok = b < B && !err;
  // the counters every row adds to: a wave's total, one LDS atomic per wave
  const unsigned long long m_ok = __ballot(ok), m_err = __ballot(err),
                           m_full = __ballot(ok && n == g);
  const uint32_t drafted = (uint32_t)wave_sum(ok ? (double)g : 0.0);
  const uint32_t accepted = (uint32_t)wave_sum(ok ? (double)n : 0.0);
  if ((threadIdx.x & 63) == 0) {
    if (m_err) atomicAdd(&s_c[kTmErrors], (uint32_t)__popcll(m_err));
    if (m_ok) {
      atomicAdd(&s_c[kTmRounds], (uint32_t)__popcll(m_ok));
      atomicAdd(&s_c[kTmDrafted], drafted);
      atomicAdd(&s_c[kTmAccepted], accepted);
    }
    if (m_full) atomicAdd(&s_c[kTmFull], (uint32_t)__popcll(m_full));
  }
  // histogram bins, spread over their addresses
  if (ok) {
    if (g > 0) atomicAdd(&s_c[kTmRate + rate_bin(n, g)], 1u);
    atomicAdd(&s_c[kTmPos + min(n, SV_TELEM_POS_BINS - 1)], 1u);
  }
  __syncthreads();
  for (int i = threadIdx.x; i < kTmCounters; i += 256)
    if (s_c[i]) atomicAdd(&acc[i], (unsigned long long)s_c[i]);
}

// Tree rows: one wave per tree, one lane per node, kTmTreeWaves trees per
// block.  Depth and the depth-1 ancestor come from pointer jumping over the
// lanes (six doublings cover 63 levels), the inner-node mask from a wave OR,
// sibling ranks from one ballot per inner node; a tree's counters go to the
// block's LDS copy, which adds to the device block once per non-zero counter.
constexpr int kTmTreeWaves = 4;

__global__ __launch_bounds__(64 * kTmTreeWaves) void telemetry_tree_kernel(
    const int* num_accepted, const int* path, const int* parents, const int* n_nodes, int B,
    int N, unsigned long long* acc) {
  __shared__ uint32_t s_c[kTmCounters];
  for (int i = threadIdx.x; i < kTmCounters; i += 64 * kTmTreeWaves) s_c[i] = 0u;
  const int lane = threadIdx.x & 63;
  const int b = blockIdx.x * kTmTreeWaves + (threadIdx.x >> 6);
  const bool live = b < B;             // wave-uniform
  const int bc = live ? b : B - 1;     // clamped: every wave loads in bounds
  // every load at once, each index clamped into its row
  const int nn = n_nodes ? n_nodes[bc] : N;
  const int n = num_accepted[bc];
  const int par_ld = parents[(long long)bc * N + min(lane, N - 1)];
  const int pj_ld = N > 1 ? path[(long long)bc * (N - 1) + min(lane, N - 2)] : 0;
  const bool node = lane < nn && lane < N;
  const int par = node && lane > 0 ? par_ld : -1;
  const bool shape_ok = nn >= 1 && nn <= N && n >= 0 && n < nn;
  const bool bad_par = node && lane > 0 && (par < 0 || par >= lane);
  const bool bad_path = lane < n && shape_ok && (pj_ld < 1 || pj_ld >= nn);
  const bool ok = live && shape_ok && !__ballot(bad_par) && !__ballot(bad_path);
  const bool child = ok && node && lane > 0;   // a node below the root of a valid tree
  const int p0 = child ? par : 0;
  const int pj = ok && lane < n ? pj_ld : 0;   // this lane's accepted node (lane < n)
  // depth: (a, d) = an ancestor and the distance to it; the root is its own, at 0
  int a = p0, d = child ? 1 : 0;
#pragma unroll
  for (int s = 0; s < 6; ++s) {
    d += __shfl(d, a);
    a = __shfl(a, a);
  }
  const int depth = d;
  // the depth-1 ancestor of every node (nodes at depth <= 1 are their own)
  int top = depth <= 1 ? lane : p0;
#pragma unroll
  for (int s = 0; s < 6; ++s) top = __shfl(top, top);
  const unsigned long long inner = wave_or_u64(child ? 1ull << p0 : 0ull);
  // rank among the siblings (test order = node index)
  int rank = 0;
  const unsigned long long below = (1ull << lane) - 1ull;
  for (unsigned long long m = inner; m; m &= m - 1ull) {
    const int p = __builtin_ctzll(m);
    const unsigned long long sib = __ballot(child && p0 == p);
    if (child && p0 == p) rank = __popcll(sib & below);
  }
  int g = depth;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) g = max(g, __shfl_xor(g, o));
  const bool leaf = ok && node && !((inner >> lane) & 1ull);
  const int first = __shfl(pj, 0);
  const bool hit = leaf && n > 0 && top == first;
  const int n_leaves = __popcll(__ballot(leaf));
  const int n_hit = __popcll(__ballot(hit));
  const int last = n > 0 ? __shfl(pj, n - 1) : 0;
  const int rank_acc = __shfl(rank, pj);   // rank of this lane's accepted node
  __syncthreads();   // s_c cleared
  if (ok && lane < n) atomicAdd(&s_c[kTmRank + min(rank_acc, SV_TELEM_RANK_BINS - 1)], 1u);
  if (lane == 0 && live) {
    if (!ok) {
      atomicAdd(&s_c[kTmErrors], 1u);
    } else {
      atomicAdd(&s_c[kTmRounds], 1u);
      atomicAdd(&s_c[kTmDrafted], (uint32_t)g);
      atomicAdd(&s_c[kTmAccepted], (uint32_t)n);
      if (!((inner >> last) & 1ull)) atomicAdd(&s_c[kTmFull], 1u);
      if (g > 0) atomicAdd(&s_c[kTmRate + rate_bin(n, g)], 1u);
      atomicAdd(&s_c[kTmPos + min(n, SV_TELEM_POS_BINS - 1)], 1u);
      atomicAdd(&s_c[kTmPaths], (uint32_t)n_leaves);
      atomicAdd(&s_c[kTmPathsHit], (uint32_t)n_hit);
    }
  }
  __syncthreads();
  for (int i = threadIdx.x; i < kTmCounters; i += 64 * kTmTreeWaves)
    if (s_c[i]) atomicAdd(&acc[i], (unsigned long long)s_c[i]);
}

// The derived signals of a window (one thread): acceptance rate, average
// accepted tokens, draft steps, Speculative Efficiency, Tree Width Effective
// (NaN where undefined), and the P50 / P95 / P99 bins of the per-row
// acceptance histogram (-1 when empty).
__global__ void telemetry_summary_kernel(const unsigned long long* acc, double* out) {
  if (threadIdx.x != 0 || blockIdx.x != 0) return;
  const double nan = __builtin_nan("");
  const double rounds = (double)acc[kTmRounds], drafted = (double)acc[kTmDrafted];
  const double accepted = (double)acc[kTmAccepted], paths = (double)acc[kTmPaths];
  const double rate = drafted > 0.0 ? accepted / drafted : nan;
  const double avg = rounds > 0.0 ? accepted / rounds : nan;
  const double steps = rounds > 0.0 ? drafted / rounds : nan;
  out[0] = rate;
  out[1] = avg;
  out[2] = steps;
  out[3] = (drafted > 0.0 && rounds > 0.0) ? rate * avg / steps : nan;
  out[4] = paths > 0.0 ? (double)acc[kTmPathsHit] / paths : nan;
  unsigned long long tot = 0ull;
  for (int k = 0; k < SV_TELEM_ACC_BINS; ++k) tot += acc[kTmRate + k];
  const int qs[3] = {50, 95, 99};
  for (int j = 0; j < 3; ++j) {
    int bin = -1;
    if (tot) {
      // first bin whose cumulative count reaches q% of the rows
      unsigned long long run = 0ull;
      bin = SV_TELEM_ACC_BINS - 1;
      for (int k = 0; k < SV_TELEM_ACC_BINS; ++k) {
        run += acc[kTmRate + k];
        if (run * 100ull >= (unsigned long long)qs[j] * tot) {
          bin = k;
          break;
        }
      }
    }
    out[5 + j] = (double)bin;
  }
}

hipError_t launch_telemetry_linear(const int* num_accepted, const int* off, int B,
                                   sv_telemetry* acc, hipStream_t st) {
  telemetry_linear_kernel<<<dim3((unsigned)((B + 255) / 256)), dim3(256), 0, st>>>(
      num_accepted, off, B, (unsigned long long*)acc);
  return hipGetLastError();
}

hipError_t launch_telemetry_tree(const int* num_accepted, const int* path, const int* parents,
                                 const int* n_nodes, int B, int N, sv_telemetry* acc,
                                 hipStream_t st) {
  telemetry_tree_kernel<<<dim3((unsigned)((B + kTmTreeWaves - 1) / kTmTreeWaves)),
                          dim3(64 * kTmTreeWaves), 0, st>>>(num_accepted, path, parents, n_nodes,
                                                            B, N, (unsigned long long*)acc);
  return hipGetLastError();
}

hipError_t launch_telemetry_summary(const sv_telemetry* acc, double* out, hipStream_t st) {
  telemetry_summary_kernel<<<dim3(1), dim3(64), 0, st>>>((const unsigned long long*)acc, out);
  return hipGetLastError();
}

}  // namespace sv
