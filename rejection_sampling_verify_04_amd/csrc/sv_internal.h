// Argument blocks and launchers shared between the kernels and the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <atomic>

#include "spec_verify.h"
#include "sv_common.h"

namespace sv {

struct Partial;

struct StatsArgs {
  const void* rows_a;    // target rows (linear) or the node rows [B N] (tree)
  const void* rows_b;    // draft rows (linear, SAMPLED_WOR tree) or null
  long long n_a;         // rows in rows_a
  long long n_rows;      // rows_a + rows_b
  int V, n_chunks;
  int tree;              // 0: linear (temperatures via offsets), 1: tree (node row / N)
  const int* offsets;
  int B;
  int N;
  const int* n_nodes;
  const float* temp_a;   // temperature of rows_a rows (per batch row)
  const float* temp_b;   // temperature of rows_b rows
  Partial* part;         // [n_rows][n_chunks]
  int vec_ok;            // 16-byte vector loads are valid for every row
  // Logits gathered at the draft tokens: linear, x_i[d_i] at [i] and y_i[d_i]
  // at [total_draft + i]; tree, node n's token under its parent at [b N + n]
  // (target) and [B N + b N + n] (draft rows, when present).
  const int* tokens;
  const int* parents;
  int total_draft;
  float* gath;
};

// Decision of one linear batch row, handed from the mass pass to the select pass.
struct LinRecord {
  int kind, flags, n_acc, token;
  int o0, g, q_greedy, q_amax;
  float u_smp;               // uniform of the stop draw
  float p_k, p_c, p_inv_s;   // target: log2(e) / T, offset, 1 / sum
  float q_k, q_c, q_inv_s;   // draft, at a rejection
};

struct LinearArgs {
  const void* target;
  const void* draft;
  int V, n_chunks, B, total_draft;
  long long n_target_rows;
  const int* off;
  const int* tokens;
  const float* temp_t;
  const float* temp_d;
  uint64_t seed, step;
  const uint32_t* row_ids;
  const Partial* part;
  const float* gath;     // logits at the draft tokens (target, then draft)
  double* wsum;          // [B][n_chunks][16]: wave totals of each chunk's stop mass
  LinRecord* rec;        // [B]
  int* num_accepted;
  int* out_tokens;
  float* p_at;
  float* q_at;
  int* row_status;
  int vec_ok;
};

struct TreeArgs {
  const void* target;
  const void* draft;     // SAMPLED_WOR: draft rows [B N]
  int mode;              // 0: TOPK, 1: SAMPLED_WOR
  int V, n_chunks, B, N;
  const int* parents;
  const int* tokens;
  const int* n_nodes;
  const float* temp;
  const float* temp_d;   // SAMPLED_WOR: draft temperatures
  uint64_t seed, step;
  const uint32_t* row_ids;
  const Partial* part;    // [B N] target rows, then (SAMPLED_WOR) [B N] draft rows
  const float* gath;     // logit of each node's token under its parent (target, then draft)
  int* num_accepted;
  int* path_nodes;
  int* out_tokens;
  float* p_at;
  int* row_status;
  int vec_ok;
};

struct AttnArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const int* prefix_len;
  const int* parents;
  int B, H, N, S_max;
  float scale_log2;      // scale * log2(e)
  uint16_t* out;
  float* lse;
};

struct KvArgs {
  uint16_t* k;           // [layers][B][H][S_max][d] bf16 (layers layer_stride elements apart)
  uint16_t* v;
  long long layer_stride;
  const int* prefix_len;
  const int* num_accepted;
  const int* path;       // [B][path_stride] accepted node ids, or null (a chain)
  int path_stride;
  int layers, B, H, S_max, d, n_new;
  int* new_len;
};

struct TreePruneArgs {
  const int* cand_parent;    // [B][C]: -1 (a child of the root) or an earlier candidate
  const int* cand_token;     // [B][C]
  const float* cand_logq;    // [B][C] log q of the token under its parent's draft row
  const int* n_cand;         // [B] or null (C)
  int B, C, n_max;
  double tau;
  int* parents;              // [B][n_max] out
  int* tokens;
  float* cum_logprob;
  int* n_nodes;              // [B] out (0: a malformed forest)
  int* n_pass;               // [B] out or null: kept nodes with cumulative probability >= tau
};

// Workgroups of a kernel that fit on the current device at once (cached per
// kernel slot and device; slots are unique across the library).
template <typename K>
inline int resident_blocks(int slot, K kernel, int threads) {
  static std::atomic<int> cache[8][kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) dev = 0;
  int c = cache[slot][dev].load(std::memory_order_relaxed);
  if (c == 0) {
    int n_cu = 0, occ = 0;
    if (hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      n_cu = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, kernel, threads, 0) != hipSuccess)
      occ = 0;
    c = std::max(1, n_cu) * std::max(1, occ);
    cache[slot][dev].store(c, std::memory_order_relaxed);
  }
  return c;
}

long long stats_items(long long n_rows, int n_chunks);
hipError_t launch_stats(int dtype, const StatsArgs& a, hipStream_t st, hipEvent_t ev_start,
                        hipEvent_t ev_stop);
hipError_t launch_linear_finish(int dtype, const LinearArgs& a, hipStream_t st);
hipError_t launch_tree_finish(int dtype, const TreeArgs& a, hipStream_t st);
hipError_t launch_exp2_words(const float* x, float* y, int n, hipStream_t st);
hipError_t launch_philox_words(uint64_t seed, uint64_t step, const uint32_t* row_ids,
                               int n_rows, int n_slots, uint32_t* out, hipStream_t st);
hipError_t launch_attn(const AttnArgs& a, hipStream_t st, hipEvent_t ev_start, hipEvent_t ev_stop);
hipError_t launch_kv_commit(const KvArgs& a, hipStream_t st, hipEvent_t ev_start, hipEvent_t ev_stop);
hipError_t launch_telemetry_linear(const int* num_accepted, const int* off, int B,
                                   sv_telemetry* acc, hipStream_t st);
hipError_t launch_telemetry_tree(const int* num_accepted, const int* path, const int* parents,
                                 const int* n_nodes, int B, int N, sv_telemetry* acc,
                                 hipStream_t st);
hipError_t launch_telemetry_summary(const sv_telemetry* acc, double* out, hipStream_t st);
hipError_t launch_draft_topk(int dtype, const void* logits, int R, int V, int k, const float* temp,
                             int* tokens, float* logprob, hipStream_t st);
hipError_t launch_tree_prune(const TreePruneArgs& a, hipStream_t st);
hipError_t launch_gamma_update(uint32_t* history, const int* num_accepted, const int* off,
                               const float* temp, int couple, int B, int* gamma_next,
                               int* off_next, hipStream_t st);

}  // namespace sv
