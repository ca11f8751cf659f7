// KV-cache commit after a verify round, gfx950.
//
// The forward pass of a round wrote the entries of its N new tokens at slots
// [L, L + N) behind a prefix of length L.  The commit keeps the root at slot
// L and moves the entry of the i-th accepted node (slot L + path[i]) to slot
// L + 1 + i, so that the cache holds what an autoregressive decoder would
// have cached; what follows the new length L + 1 + n is dropped (cf-1.com/
// news/5632551 §3.3, keep the accepted positions and discard the rest;
// kwkr.cn/news/620872 §5.1, one pre-allocated cache spliced by offsets).
//
// One work item per (layer, batch row); each thread owns 16-byte columns of
// one head and moves them down the accepted rows.  Accepted node ids
// strictly increase and path[i] >= i + 1, so a source slot L + path[j] is
// never below the destination L + 1 + i of any row i <= j: a thread may
// issue the loads of a batch of rows before their stores, and a store can
// only hit the source of an earlier row, which that same thread has already
// read (per-address program order).  No two threads touch the same column.
// Moves from a slot to itself (a chain's prefix of the path) are skipped, so
// a linear round moves nothing.  The copy is bound by HBM bandwidth (16-byte
// vectors, each moved row read once and written once).
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include "sv_common.h"
#include "sv_internal.h"

namespace sv {

constexpr int kKvThreads = 256;
constexpr int kKvRows = 8;          // rows of a column whose loads are in flight together

__global__ __launch_bounds__(kKvThreads) void kv_commit_kernel(KvArgs a) {
  __shared__ int s_path[kMaxNodes];
  __shared__ int s_ok, s_i0;

  const int tid = threadIdx.x;
  const int B = a.B, H = a.H;
  const int b = blockIdx.x % B, layer = blockIdx.x / B;
  const int L = a.prefix_len[b];
  const int n = a.num_accepted[b];
  const int N = a.n_new;

  if (tid < 64) {
    const int i = tid;
    const bool mine = i < n && i < N - 1;
    int p = i + 1;
    if (mine && a.path) p = a.path[(long long)b * a.path_stride + i];
    s_path[i] = p;
    // strictly increasing node ids within [1, N); the first index that moves
    const int prev = __builtin_amdgcn_update_dpp(0, p, kDppWaveShr1, 0xf, 0xf, false);
    const bool bad = mine && (p <= (i == 0 ? 0 : prev) || p >= N);
    const unsigned long long badm = __ballot(bad);
    const unsigned long long moves = __ballot(mine && p != i + 1);
    if (tid == 0) {
      const bool shape_ok = L >= 0 && (long long)L + N <= a.S_max && n <= N - 1;
      s_ok = shape_ok && badm == 0ull;
      s_i0 = moves ? __ffsll((long long)moves) - 1 : 64;
    }
  }
  __syncthreads();
  const bool ok = s_ok != 0;
  if (layer == 0 && tid == 0) a.new_len[b] = n < 0 ? L : (ok ? L + 1 + n : -1);
  if (n <= 0 || !ok) return;
  const int i0 = s_i0;
  if (i0 >= n) return;
  const int m = n - i0;               // rows that move
  const int vr = a.d / 8;             // 16-byte columns per row
  const long long hs = (long long)a.S_max * a.d;   // elements per head
  const long long lb = (long long)layer * a.layer_stride + (long long)b * H * hs;

  for (int item = tid; item < H * vr; item += kKvThreads) {
    const int h = item / vr, c = item - (item / vr) * vr;
    const uint16_t* ks = a.k + lb + h * hs + c * 8;
    const uint16_t* vs = a.v + lb + h * hs + c * 8;
    for (int r0 = 0; r0 < m; r0 += kKvRows) {
      u32x4_t kr[kKvRows], vq[kKvRows];
#pragma unroll
      for (int j = 0; j < kKvRows; ++j) {
        const int i = i0 + min(r0 + j, m - 1);
        const long long src = (long long)(L + s_path[i]) * a.d;
        kr[j] = *(const u32x4_t*)(ks + src);
        vq[j] = *(const u32x4_t*)(vs + src);
      }
      // rows past m repeat the last row: the same value to the same slot
#pragma unroll
      for (int j = 0; j < kKvRows; ++j) {
        const long long dst = (long long)(L + 1 + i0 + min(r0 + j, m - 1)) * a.d;
        *(u32x4_t*)(a.k + lb + h * hs + c * 8 + dst) = kr[j];
        *(u32x4_t*)(a.v + lb + h * hs + c * 8 + dst) = vq[j];
      }
    }
  }
}

// Launched with events, the events bracket the kernel's dispatch.
hipError_t launch_kv_commit(const KvArgs& a, hipStream_t st, hipEvent_t ev_start,
                            hipEvent_t ev_stop) {
  const dim3 grid((unsigned)((long long)a.layers * a.B)), block(kKvThreads);
  if (ev_start && ev_stop)
    hipExtLaunchKernelGGL(kv_commit_kernel, grid, block, 0, st, ev_start, ev_stop, 0, a);
  else
    kv_commit_kernel<<<grid, block, 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace sv
