// Argument blocks and launchers shared between the kernels and the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sv {

struct Partial;

struct StatsArgs {
  const void* rows_a;    // target rows (linear) or all node rows (tree)
  const void* rows_b;    // draft rows (linear) or null
  long long n_a;         // rows in rows_a
  long long n_rows;      // rows_a + rows_b
  int V, n_chunks;
  int tree;              // 0: linear (temperatures via offsets), 1: tree (row / N)
  const int* offsets;
  int B;
  int N;
  const int* n_nodes;
  const float* temp_a;   // temperature of rows_a rows (per batch row)
  const float* temp_b;   // temperature of rows_b rows
  Partial* part;         // [n_rows][n_chunks]
  int vec_ok;            // 16-byte vector loads are valid for every row
};

// Decision of one linear batch row, handed from the mass pass to the select pass.
struct LinRecord {
  int kind, flags, n_acc, token;
  int o0, g, q_greedy, q_amax;
  float p_c, p_inv_s, q_c, q_inv_s;
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
  double* mass;          // [B][n_chunks]
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
  int V, n_chunks, B, N;
  const int* parents;
  const int* tokens;
  const int* n_nodes;
  const float* temp;
  uint64_t seed, step;
  const uint32_t* row_ids;
  const Partial* part;
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

long long stats_items(long long n_rows, int n_chunks);
hipError_t launch_stats(int dtype, const StatsArgs& a, hipStream_t st, hipEvent_t ev_start,
                        hipEvent_t ev_stop);
hipError_t launch_linear_finish(int dtype, const LinearArgs& a, hipStream_t st);
hipError_t launch_tree_finish(int dtype, const TreeArgs& a, hipStream_t st);
hipError_t launch_philox_words(uint64_t seed, uint64_t step, const uint32_t* row_ids,
                               int n_rows, int n_slots, uint32_t* out, hipStream_t st);
hipError_t launch_attn(const AttnArgs& a, hipStream_t st, hipEvent_t ev_start, hipEvent_t ev_stop);

}  // namespace sv
