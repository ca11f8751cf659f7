// Speculation control between rounds, gfx950: the dynamic speculation
// length of blog.lonae.com/posts/2026-draft-model-kv-jDwzYp (bimodal-
// acceptance paragraph).  A request's acceptance rate over its last 16
// steps sets its next gamma: 8 above 60%, 4 from 30% to 60%, 2 below 30%;
// with temperature coupling, a request above temperature 0.8 drafts one
// token.  A step is one tested draft position: a round that accepted n of
// gamma drafts adds n ones, then a zero if it stopped on a rejection.
//
// History word per request: bits 0..15 the outcomes (bit 0 the newest),
// bits 16..20 how many are valid.  One work item of 1024 threads walks the
// batch in slices; the next draft offsets are the running sum of the new
// gammas (block scan with a carry between slices).
#include <hip/hip_runtime.h>

#include "sv_common.h"
#include "sv_internal.h"

namespace sv {

// Only the newest 16 outcomes survive a push, so at most 16 are shifted in:
// the last min(steps, 16) of n ones followed (after a rejection) by a zero.
// The loop is bounded whatever num_accepted holds.
__device__ __forceinline__ uint32_t history_push(uint32_t w, int n, int g) {
  if (n < 0) return w;
  uint32_t hist = w & 0xFFFFu, count = (w >> 16) & 0x1Fu;
  const int z = n < g ? 1 : 0;
  const int k = n >= 16 ? 16 : min(n + z, 16);
  for (int s = 0; s < k; ++s) {
    hist = ((hist << 1) | (s < k - z ? 1u : 0u)) & 0xFFFFu;
    count = min(count + 1u, 16u);
  }
  return hist | (count << 16);
}

__device__ __forceinline__ int gamma_from(uint32_t w) {
  const uint32_t hist = w & 0xFFFFu, count = (w >> 16) & 0x1Fu;
  if (count == 0u) return 4;
  const int ones = __popc(hist & ((1u << count) - 1u));
  if (5 * ones > 3 * (int)count) return 8;          // rate > 60%
  if (10 * ones >= 3 * (int)count) return 4;        // 30% <= rate <= 60%
  return 2;
}

__global__ __launch_bounds__(kFinThreads) void gamma_update_kernel(uint32_t* history,
                                                                   const int* num_accepted,
                                                                   const int* off,
                                                                   const float* temp,
                                                                   int couple, int B,
                                                                   int* gamma_next,
                                                                   int* off_next) {
  __shared__ double s_scan[kFinWaves];
  double carry = 0.0;
  for (int b0 = 0; b0 < B; b0 += kFinThreads) {
    const int b = b0 + threadIdx.x;
    int g_new = 0;
    if (b < B) {
      // every load issued together, none behind a branch: the temperature
      // from a valid address whether or not it is used, and the offsets
      // held in registers (the asm) before the push, which uses them only
      // for a valid count
      const float tb = *(temp ? temp + b : (const float*)(num_accepted + b));
      const uint32_t h = history[b];
      const int n = num_accepted[b];
      const int o0 = off[b], o1 = off[b + 1];
      asm volatile("" ::"v"(o0), "v"(o1));
      const uint32_t w = history_push(h, n, o1 - o0);
      history[b] = w;
      g_new = (couple && temp && tb > 0.8f) ? 1 : gamma_from(w);
      gamma_next[b] = g_new;
    }
    double total;
    const double ex = block_exclusive_scan<kFinWaves>((double)g_new, s_scan, &total);
    if (off_next && b < B) off_next[b] = (int)(carry + ex);
    carry += total;
  }
  if (off_next && threadIdx.x == 0) off_next[B] = (int)carry;
}

hipError_t launch_gamma_update(uint32_t* history, const int* num_accepted, const int* off,
                               const float* temp, int couple, int B, int* gamma_next,
                               int* off_next, hipStream_t st) {
  gamma_update_kernel<<<dim3(1), dim3(kFinThreads), 0, st>>>(history, num_accepted, off, temp,
                                                             couple, B, gamma_next, off_next);
  return hipGetLastError();
}

}  // namespace sv
