// Host-side check of the C ABI's argument validation, built with the host
// sanitizers (address + undefined behaviour, or thread) and run without a GPU.
// Eight threads call the validation paths, the workspace-size queries and the
// per-thread timing hook at once; every call must return its documented code
// before any kernel launch, so no HIP device call is made.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdio.h>

#include <atomic>
#include <climits>
#include <thread>
#include <vector>

#include "spec_verify.h"

namespace {

std::atomic<int> g_fail{0};

void expect(int got, int want, const char* what, int line) {
  if (got != want) {
    fprintf(stderr, "line %d: %s returned %d, want %d\n", line, what, got, want);
    g_fail.fetch_add(1);
  }
}
#define EXPECT(call, want) expect((call), (want), #call, __LINE__)

void* P(uintptr_t v) { return (void*)v; }

void worker(int tid, size_t ws_linear, size_t ws_tree) {
  const void* p = P(256);
  const int32_t* ip = (const int32_t*)p;
  const float* fp = (const float*)p;
  int32_t* op = (int32_t*)P(256);
  for (int it = 0; it < 2000; ++it) {
    // arm and clear this thread's timing hook (dummy handles, never used)
    EXPECT(spec_verify_profile_next((hipEvent_t)P(4096 + tid), (hipEvent_t)P(8192 + tid)), SV_OK);
    EXPECT(spec_verify_profile_next(nullptr, nullptr), SV_OK);
    if (spec_verify_linear_workspace_size(32, 160, 32000, SV_BF16) != ws_linear) g_fail++;
    if (spec_verify_tree_workspace_size(64, 64, 32000, SV_BF16) != ws_tree) g_fail++;
    if (spec_verify_linear_workspace_size(INT_MAX, INT_MAX, INT_MAX, SV_BF16) == 0) g_fail++;
    if (spec_verify_linear_workspace_size(-1, 0, 10, SV_BF16) != 0) g_fail++;
    if (spec_verify_tree_workspace_size(0, 0, 10, SV_BF16) != 0) g_fail++;
    // linear: dtype, sizes, gamma bound, null pointers, workspace, vocabulary bound
    EXPECT(spec_verify_linear(p, p, 7, 2, 100, 4, ip, ip, fp, fp, 0, 0, nullptr, op, op, nullptr,
                              nullptr, nullptr, P(256), 1 << 20, nullptr), SV_ERR_INVALID_ARG);
    EXPECT(spec_verify_linear(p, p, SV_BF16, INT_MAX, 100, INT_MAX, ip, ip, fp, fp, 0, 0, nullptr,
                              op, op, nullptr, nullptr, nullptr, P(256), 16, nullptr),
           SV_ERR_INVALID_ARG);
    EXPECT(spec_verify_linear(p, p, SV_BF16, 2, 100, 2 * 64 + 1, ip, ip, fp, fp, 0, 0, nullptr, op,
                              op, nullptr, nullptr, nullptr, P(256), 1 << 20, nullptr),
           SV_ERR_INVALID_ARG);
    EXPECT(spec_verify_linear(p, p, SV_BF16, 2, INT_MAX, 4, ip, ip, fp, fp, 0, 0, nullptr, op, op,
                              nullptr, nullptr, nullptr, P(256), 1 << 20, nullptr),
           SV_ERR_UNSUPPORTED);
    EXPECT(spec_verify_linear(nullptr, p, SV_BF16, 2, 100, 4, ip, ip, fp, fp, 0, 0, nullptr, op,
                              op, nullptr, nullptr, nullptr, P(256), 1 << 20, nullptr),
           SV_ERR_INVALID_ARG);
    EXPECT(spec_verify_linear(p, p, SV_BF16, 2, 100, 4, ip, ip, fp, fp, 0, 0, nullptr, op, op,
                              nullptr, nullptr, nullptr, P(128), 1 << 20, nullptr),
           SV_ERR_WORKSPACE);
    EXPECT(spec_verify_linear(p, p, SV_BF16, 0, 100, 0, ip, ip, fp, fp, 0, 0, nullptr, op, op,
                              nullptr, nullptr, nullptr, nullptr, 0, nullptr), SV_OK);
    // tree: node bound, mode, SAMPLED_WOR inputs, workspace
    EXPECT(spec_verify_tree(p, nullptr, SV_BF16, 4, 65, 100, ip, ip, nullptr, SV_TREE_TOPK, fp,
                            nullptr, 0, 0, nullptr, op, op, op, nullptr, nullptr, P(256), 1 << 20,
                            nullptr), SV_ERR_INVALID_ARG);
    EXPECT(spec_verify_tree(p, nullptr, SV_BF16, 4, 8, 100, ip, ip, nullptr, SV_TREE_SAMPLED_WOR,
                            fp, fp, 0, 0, nullptr, op, op, op, nullptr, nullptr, P(256), 1 << 20,
                            nullptr), SV_ERR_INVALID_ARG);
    EXPECT(spec_verify_tree(p, nullptr, SV_BF16, 4, 8, 100, ip, ip, nullptr, 9, fp, nullptr, 0, 0,
                            nullptr, op, op, op, nullptr, nullptr, P(256), 1 << 20, nullptr),
           SV_ERR_INVALID_ARG);
    EXPECT(spec_verify_tree(p, nullptr, SV_BF16, INT_MAX, 64, 100, ip, ip, nullptr, SV_TREE_TOPK,
                            fp, nullptr, 0, 0, nullptr, op, op, op, nullptr, nullptr, P(256), 16,
                            nullptr), SV_ERR_INVALID_ARG);
    EXPECT(spec_verify_tree(p, nullptr, SV_BF16, 4, 8, 100, ip, ip, nullptr, SV_TREE_TOPK, fp,
                            nullptr, 0, 0, nullptr, op, op, op, nullptr, nullptr, P(256), 16,
                            nullptr), SV_ERR_WORKSPACE);
    // attention, KV commit, telemetry, drafting, control, diagnostics
    EXPECT(spec_verify_attn(p, p, p, ip, nullptr, 2, 4, 8, 64, 100, 0.1f, P(256), nullptr, nullptr),
           SV_ERR_UNSUPPORTED);
    EXPECT(spec_verify_attn(p, p, p, ip, nullptr, 2, 4, 65, 128, 100, 0.1f, P(256), nullptr,
                            nullptr), SV_ERR_INVALID_ARG);
    EXPECT(spec_verify_attn(p, p, p, ip, nullptr, INT_MAX, INT_MAX, 8, 128, 100, 0.1f, P(256),
                            nullptr, nullptr), SV_ERR_INVALID_ARG);
    EXPECT(spec_verify_attn(p, p, P(258), ip, nullptr, 2, 4, 8, 128, 100, 0.1f, P(256), nullptr,
                            nullptr), SV_ERR_INVALID_ARG);
    EXPECT(spec_verify_kv_commit(P(256), P(256), 2, 16, ip, ip, nullptr, 0, 2, 4, 8, 128, 100, op,
                                 nullptr), SV_ERR_INVALID_ARG);
    EXPECT(spec_verify_kv_commit(P(256), P(256), INT_MAX, LLONG_MAX, ip, ip, nullptr, 0, INT_MAX,
                                 INT_MAX, 8, 128, INT_MAX, op, nullptr), SV_ERR_INVALID_ARG);
    EXPECT(spec_verify_telemetry_linear(ip, nullptr, 4, (sv_telemetry*)P(256), nullptr),
           SV_ERR_INVALID_ARG);
    EXPECT(spec_verify_telemetry_tree(ip, ip, ip, nullptr, 4, 65, (sv_telemetry*)P(256), nullptr),
           SV_ERR_INVALID_ARG);
    EXPECT(spec_verify_telemetry_summary(nullptr, (double*)P(256), nullptr), SV_ERR_INVALID_ARG);
    EXPECT(spec_verify_draft_topk(p, SV_BF16, 2, 100, 65, nullptr, op, (float*)P(256), nullptr),
           SV_ERR_INVALID_ARG);
    EXPECT(spec_verify_tree_prune(ip, ip, fp, nullptr, 2, 1025, 64, 0.1, op, op, (float*)P(256), op,
                                  nullptr, nullptr), SV_ERR_INVALID_ARG);
    EXPECT(spec_verify_gamma_update((uint32_t*)P(256), ip, ip, nullptr, 1, 4, op, nullptr, nullptr),
           SV_ERR_INVALID_ARG);
    EXPECT(spec_verify_gamma_update((uint32_t*)P(256), ip, ip, nullptr, 0, INT_MAX, op, nullptr,
                                   nullptr), SV_ERR_INVALID_ARG);
    EXPECT(spec_verify_philox_words(0, 0, nullptr, INT_MAX, INT_MAX, (uint32_t*)P(256), nullptr),
           SV_ERR_INVALID_ARG);
    EXPECT(spec_verify_philox_words(0, 0, nullptr, 3, 5, (uint32_t*)P(8), nullptr),
           SV_ERR_INVALID_ARG);
    EXPECT(spec_verify_linear_noalloc(p, p, 7, 2, 100, 4, ip, ip, fp, fp, 0, 0, nullptr, op, op,
                                      nullptr, nullptr, nullptr, nullptr), SV_ERR_INVALID_ARG);
    EXPECT(spec_verify_linear_noalloc(p, p, SV_BF16, 4096, 152064, 4096 * 8, ip, ip, fp, fp, 0, 0,
                                      nullptr, op, op, nullptr, nullptr, nullptr, nullptr),
           SV_ERR_SCRATCH);
    EXPECT(spec_verify_linear_noalloc(p, p, SV_BF16, INT_MAX, INT_MAX, INT_MAX, ip, ip, fp, fp, 0,
                                      0, nullptr, op, op, nullptr, nullptr, nullptr, nullptr),
           SV_ERR_UNSUPPORTED);
    EXPECT(spec_verify_exp2(fp, (float*)P(256), -1, nullptr), SV_ERR_INVALID_ARG);
    EXPECT(spec_verify_exp2(nullptr, (float*)P(256), 5, nullptr), SV_ERR_INVALID_ARG);
    EXPECT(spec_verify_exp2(nullptr, nullptr, 0, nullptr), SV_OK);
    if (spec_verify_status_string(SV_ERR_HIP)[0] == 0) g_fail++;
  }
}

}  // namespace

int main() {
  const size_t ws_linear = spec_verify_linear_workspace_size(32, 160, 32000, SV_BF16);
  const size_t ws_tree = spec_verify_tree_workspace_size(64, 64, 32000, SV_BF16);
  std::vector<std::thread> th;
  for (int t = 0; t < 8; ++t) th.emplace_back(worker, t, ws_linear, ws_tree);
  for (auto& t : th) t.join();
  if (g_fail.load()) {
    fprintf(stderr, "%d failed checks\n", g_fail.load());
    return 1;
  }
  printf("abi host check ok\n");
  return 0;
}
