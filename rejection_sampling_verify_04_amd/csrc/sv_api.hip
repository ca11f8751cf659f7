// C ABI of the verify library: host-side argument checks, workspace layout
// and kernel launches.  Declarations and contracts are in include/spec_verify.h.
#include "spec_verify.h"
#include "sv_common.h"
#include "sv_internal.h"

namespace {

constexpr size_t kAlign = SV_WORKSPACE_ALIGN;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// Chunks of a row of V elements (in 64 bits: V may be near INT_MAX).
int n_chunks_for(int V) { return (int)(((long long)V + sv::kChunk - 1) / sv::kChunk); }

// Workspace: [partials | gathered logits | chunk wave totals | per-row
// decision records], each aligned.  n_gath = logits gathered at draft tokens.
struct Layout {
  size_t part, gath, mass, rec, total;
};

Layout layout(long long n_rows, int B, int V, long long n_gath, bool linear) {
  const int nc = n_chunks_for(V);
  Layout l;
  l.part = 0;
  l.gath = align_up((size_t)n_rows * nc * sv::kPartsPerChunk * sizeof(sv::Partial));
  l.mass = l.gath + align_up((size_t)n_gath * sizeof(float));
  l.rec = l.mass + (linear ? align_up((size_t)B * nc * sv::kFinWaves * sizeof(double)) : 0);
  l.total = l.rec + (linear ? align_up((size_t)B * sizeof(sv::LinRecord)) : 0);
  if (l.total == 0) l.total = kAlign;
  return l;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// One-shot timing hook (spec_verify_profile_next), one per host thread: an
// armed pair is seen and consumed only by calls on the thread that armed it.
struct ProfHook {
  hipEvent_t begin, end;
};
thread_local ProfHook t_prof = {nullptr, nullptr};

ProfHook take_prof_hook() {
  const ProfHook h = t_prof;
  t_prof = ProfHook{nullptr, nullptr};
  return h;
}

hipError_t launch_stats_timed(int dtype, const sv::StatsArgs& s, hipStream_t stream) {
  const ProfHook h = take_prof_hook();
  return sv::launch_stats(dtype, s, stream, h.begin, h.end);
}

int check_workspace(void* ws, size_t bytes, size_t need) {
  if (!ws || ((uintptr_t)ws % kAlign) != 0 || bytes < need) return SV_ERR_WORKSPACE;
  return SV_OK;
}

// Workspace of the allocation-free linear verify: a static device array, one
// copy per GPU, held until the process ends.  Host code never uses the
// array's name as an address: each device's copy is found once, with that
// device current, through hipGetSymbolAddress.
static __device__ __align__(256) unsigned char scratch[SV_STATIC_SCRATCH_BYTES];
std::atomic<void*> g_scratch[sv::kMaxDevices];

// This device's copy of `scratch` (nullptr if its address cannot be had).
void* device_scratch() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= sv::kMaxDevices) return nullptr;
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (p) return p;
  void* q = nullptr;
  if (hipGetSymbolAddress(&q, HIP_SYMBOL(scratch)) != hipSuccess || !q) return nullptr;
  g_scratch[dev].store(q, std::memory_order_release);
  return q;
}

// Argument checks of the linear verify; SV_OK, with the workspace layout in
// *l, when the call has work to do (*empty false).
int linear_check(const void* target_logits, const void* draft_logits, int dtype, int B, int V,
                 int total_draft, const int32_t* draft_offsets, const int32_t* draft_tokens,
                 const float* temp_target, const float* temp_draft, const int32_t* num_accepted,
                 const int32_t* out_tokens, Layout* l, bool* empty) {
  *empty = false;
  if (dtype != SV_F32 && dtype != SV_BF16) return SV_ERR_INVALID_ARG;
  if (B < 0 || V < 1 || total_draft < 0) return SV_ERR_INVALID_ARG;
  if ((long long)total_draft > (long long)B * SV_MAX_GAMMA) return SV_ERR_INVALID_ARG;
  if (B == 0) {
    *empty = true;
    return SV_OK;
  }
  if (n_chunks_for(V) > sv::kMaxChunks) return SV_ERR_UNSUPPORTED;
  if (!target_logits || !draft_offsets || !temp_target || !temp_draft || !num_accepted ||
      !out_tokens)
    return SV_ERR_INVALID_ARG;
  if (total_draft > 0 && (!draft_logits || !draft_tokens)) return SV_ERR_INVALID_ARG;
  const long long n_rows = 2LL * total_draft + B;
  const int nc = n_chunks_for(V);
  if (sv::stats_items(n_rows, nc) >= (1LL << 31) || (long long)B * nc >= (1LL << 31))
    return SV_ERR_INVALID_ARG;
  *l = layout(n_rows, B, V, 2LL * total_draft, true);
  return SV_OK;
}

// The linear verify's launches on a checked call, with its workspace.
int linear_run(const void* target_logits, const void* draft_logits, int dtype, int B, int V,
               int total_draft, const int32_t* draft_offsets, const int32_t* draft_tokens,
               const float* temp_target, const float* temp_draft, uint64_t seed, uint64_t step,
               const uint32_t* row_ids, int32_t* num_accepted, int32_t* out_tokens,
               float* p_at_draft, float* q_at_draft, int32_t* row_status, const Layout& l,
               void* workspace, hipStream_t stream) {
  const long long n_t = (long long)total_draft + B;
  const long long n_rows = n_t + total_draft;
  const int nc = n_chunks_for(V);

  const int es = dtype == SV_BF16 ? 2 : 4;
  const int vec_ok = ((long long)V * es) % 16 == 0 && aligned16(target_logits) &&
                     (total_draft == 0 || aligned16(draft_logits));
  char* ws = (char*)workspace;

  sv::StatsArgs s{};
  s.rows_a = target_logits;
  s.rows_b = draft_logits;
  s.n_a = n_t;
  s.n_rows = n_rows;
  s.V = V;
  s.n_chunks = nc;
  s.tree = 0;
  s.offsets = draft_offsets;
  s.B = B;
  s.N = 0;
  s.n_nodes = nullptr;
  s.temp_a = temp_target;
  s.temp_b = temp_draft;
  s.part = (sv::Partial*)(ws + l.part);
  s.vec_ok = vec_ok;
  s.tokens = draft_tokens;
  s.parents = nullptr;
  s.total_draft = total_draft;
  s.gath = (float*)(ws + l.gath);
  if (launch_stats_timed(dtype, s, stream) != hipSuccess) return SV_ERR_HIP;

  sv::LinearArgs f{};
  f.target = target_logits;
  f.draft = draft_logits;
  f.V = V;
  f.n_chunks = nc;
  f.B = B;
  f.total_draft = total_draft;
  f.n_target_rows = n_t;
  f.off = draft_offsets;
  f.tokens = draft_tokens;
  f.temp_t = temp_target;
  f.temp_d = temp_draft;
  f.seed = seed;
  f.step = step;
  f.row_ids = row_ids;
  f.part = s.part;
  f.gath = s.gath;
  f.wsum = (double*)(ws + l.mass);
  f.rec = (sv::LinRecord*)(ws + l.rec);
  f.num_accepted = num_accepted;
  f.out_tokens = out_tokens;
  f.p_at = p_at_draft;
  f.q_at = q_at_draft;
  f.row_status = row_status;
  f.vec_ok = vec_ok;
  if (sv::launch_linear_finish(dtype, f, stream) != hipSuccess) return SV_ERR_HIP;
  return SV_OK;
}

}  // namespace

extern "C" {

int spec_verify_version(void) { return (0 << 16) | 1; }

const char* spec_verify_status_string(int status) {
  switch (status) {
    case SV_OK: return "ok";
    case SV_ERR_INVALID_ARG: return "invalid argument";
    case SV_ERR_UNSUPPORTED: return "unsupported request";
    case SV_ERR_WORKSPACE: return "workspace missing, too small or misaligned";
    case SV_ERR_HIP: return "HIP kernel launch failed";
    case SV_ERR_SCRATCH: return "request needs more than the built-in static scratch";
    default: return "unknown status";
  }
}

size_t spec_verify_linear_workspace_size(int B, int total_draft, int V, int dtype) {
  (void)dtype;
  if (B < 0 || total_draft < 0 || V < 1) return 0;
  return layout(2LL * total_draft + B, B, V, 2LL * total_draft, true).total;
}


int spec_verify_linear(const void* target_logits, const void* draft_logits, int dtype, int B,
                       int V, int total_draft, const int32_t* draft_offsets,
                       const int32_t* draft_tokens, const float* temp_target,
                       const float* temp_draft, uint64_t seed, uint64_t step,
                       const uint32_t* row_ids, int32_t* num_accepted, int32_t* out_tokens,
                       float* p_at_draft, float* q_at_draft, int32_t* row_status,
                       void* workspace, size_t workspace_bytes, hipStream_t stream) {
  Layout l;
  bool empty;
  int st = linear_check(target_logits, draft_logits, dtype, B, V, total_draft, draft_offsets,
                        draft_tokens, temp_target, temp_draft, num_accepted, out_tokens, &l,
                        &empty);
  if (st != SV_OK || empty) return st;
  st = check_workspace(workspace, workspace_bytes, l.total);
  if (st != SV_OK) return st;
  return linear_run(target_logits, draft_logits, dtype, B, V, total_draft, draft_offsets,
                    draft_tokens, temp_target, temp_draft, seed, step, row_ids, num_accepted,
                    out_tokens, p_at_draft, q_at_draft, row_status, l, workspace, stream);
}

int spec_verify_linear_noalloc(const void* target_logits, const void* draft_logits, int dtype,
                               int B, int V, int total_draft, const int32_t* draft_offsets,
                               const int32_t* draft_tokens, const float* temp_target,
                               const float* temp_draft, uint64_t seed, uint64_t step,
                               const uint32_t* row_ids, int32_t* num_accepted,
                               int32_t* out_tokens, float* p_at_draft, float* q_at_draft,
                               int32_t* row_status, hipStream_t stream) {
  Layout l;
  bool empty;
  const int st = linear_check(target_logits, draft_logits, dtype, B, V, total_draft,
                              draft_offsets, draft_tokens, temp_target, temp_draft, num_accepted,
                              out_tokens, &l, &empty);
  if (st != SV_OK || empty) return st;
  if (l.total > (size_t)SV_STATIC_SCRATCH_BYTES) return SV_ERR_SCRATCH;
  void* ws = device_scratch();
  if (!ws) return SV_ERR_HIP;
  return linear_run(target_logits, draft_logits, dtype, B, V, total_draft, draft_offsets,
                    draft_tokens, temp_target, temp_draft, seed, step, row_ids, num_accepted,
                    out_tokens, p_at_draft, q_at_draft, row_status, l, ws, stream);
}

// Sized for either candidate mode (SAMPLED_WOR keeps the draft rows' partials
// and gathers too).
size_t spec_verify_tree_workspace_size(int B, int N, int V, int dtype) {
  (void)dtype;
  if (B < 0 || N < 1 || V < 1) return 0;
  return layout(2LL * B * N, B, V, 2LL * B * N, false).total;
}

int spec_verify_tree(const void* target_logits, const void* draft_logits, int dtype, int B,
                     int N, int V, const int32_t* parents, const int32_t* node_tokens,
                     const int32_t* n_nodes, int cand_mode, const float* temp_target,
                     const float* temp_draft, uint64_t seed, uint64_t step,
                     const uint32_t* row_ids, int32_t* num_accepted, int32_t* path_nodes,
                     int32_t* out_tokens, float* p_at_node, int32_t* row_status,
                     void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (dtype != SV_F32 && dtype != SV_BF16) return SV_ERR_INVALID_ARG;
  if (B < 0 || N < 1 || N > SV_MAX_TREE_NODES || V < 1) return SV_ERR_INVALID_ARG;
  if (cand_mode != SV_TREE_TOPK && cand_mode != SV_TREE_SAMPLED_WOR) return SV_ERR_INVALID_ARG;
  const bool wor = cand_mode == SV_TREE_SAMPLED_WOR;
  if (B == 0) return SV_OK;
  if (n_chunks_for(V) > sv::kMaxChunks) return SV_ERR_UNSUPPORTED;
  if (!target_logits || !parents || !node_tokens || !temp_target || !num_accepted ||
      !path_nodes || !out_tokens)
    return SV_ERR_INVALID_ARG;
  if (wor && (!draft_logits || !temp_draft)) return SV_ERR_INVALID_ARG;
  const long long n_nodes_all = (long long)B * N;
  const long long n_rows = wor ? 2 * n_nodes_all : n_nodes_all;
  const int nc = n_chunks_for(V);
  if (sv::stats_items(n_rows, nc) >= (1LL << 31)) return SV_ERR_INVALID_ARG;
  const Layout l = layout(n_rows, B, V, n_rows, false);
  const int wst = check_workspace(workspace, workspace_bytes, l.total);
  if (wst != SV_OK) return wst;
  const int es = dtype == SV_BF16 ? 2 : 4;
  const int vec_ok = ((long long)V * es) % 16 == 0 && aligned16(target_logits) &&
                     (!wor || aligned16(draft_logits));
  char* ws = (char*)workspace;

  sv::StatsArgs s{};
  s.rows_a = target_logits;
  s.rows_b = wor ? draft_logits : nullptr;
  s.n_a = n_nodes_all;
  s.n_rows = n_rows;
  s.V = V;
  s.n_chunks = nc;
  s.tree = 1;
  s.offsets = nullptr;
  s.B = B;
  s.N = N;
  s.n_nodes = n_nodes;
  s.temp_a = temp_target;
  s.temp_b = wor ? temp_draft : temp_target;
  s.part = (sv::Partial*)(ws + l.part);
  s.vec_ok = vec_ok;
  s.tokens = node_tokens;
  s.parents = parents;
  s.total_draft = 0;
  s.gath = (float*)(ws + l.gath);
  if (launch_stats_timed(dtype, s, stream) != hipSuccess) return SV_ERR_HIP;

  sv::TreeArgs f{};
  f.target = target_logits;
  f.draft = wor ? draft_logits : nullptr;
  f.mode = wor ? 1 : 0;
  f.V = V;
  f.n_chunks = nc;
  f.B = B;
  f.N = N;
  f.parents = parents;
  f.tokens = node_tokens;
  f.n_nodes = n_nodes;
  f.temp = temp_target;
  f.temp_d = wor ? temp_draft : temp_target;
  f.seed = seed;
  f.step = step;
  f.row_ids = row_ids;
  f.part = s.part;
  f.gath = s.gath;
  f.num_accepted = num_accepted;
  f.path_nodes = path_nodes;
  f.out_tokens = out_tokens;
  f.p_at = p_at_node;
  f.row_status = row_status;
  f.vec_ok = vec_ok;
  if (sv::launch_tree_finish(dtype, f, stream) != hipSuccess) return SV_ERR_HIP;
  return SV_OK;
}

int spec_verify_attn(const void* q, const void* k_cache, const void* v_cache,
                     const int32_t* prefix_len, const int32_t* parents, int B, int H, int N,
                     int d, int S_max, float scale, void* out, float* lse, hipStream_t stream) {
  if (B < 0 || H < 1 || N < 1 || N > SV_MAX_TREE_NODES || S_max < N) return SV_ERR_INVALID_ARG;
  if (d != 128) return SV_ERR_UNSUPPORTED;
  if (!(scale > 0.0f) || !(scale < __builtin_huge_valf())) return SV_ERR_INVALID_ARG;
  if (B == 0) return SV_OK;
  if (!q || !k_cache || !v_cache || !prefix_len || !out) return SV_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(out))
    return SV_ERR_INVALID_ARG;
  if ((long long)B * H >= (1LL << 31)) return SV_ERR_INVALID_ARG;
  sv::AttnArgs a{};
  a.q = (const uint16_t*)q;
  a.k = (const uint16_t*)k_cache;
  a.v = (const uint16_t*)v_cache;
  a.prefix_len = prefix_len;
  a.parents = parents;
  a.B = B;
  a.H = H;
  a.N = N;
  a.S_max = S_max;
  a.scale_log2 = (float)((double)scale * sv::kLog2e);
  a.out = (uint16_t*)out;
  a.lse = lse;
  const ProfHook h = take_prof_hook();
  if (sv::launch_attn(a, stream, h.begin, h.end) != hipSuccess) return SV_ERR_HIP;
  return SV_OK;
}

int spec_verify_kv_commit(void* k_cache, void* v_cache, int layers, long long layer_stride,
                          const int32_t* prefix_len, const int32_t* num_accepted,
                          const int32_t* path_nodes, int path_stride, int B, int H, int N, int d,
                          int S_max, int32_t* new_len, hipStream_t stream) {
  if (layers < 1 || B < 0 || H < 1 || N < 1 || N > SV_MAX_TREE_NODES || S_max < N)
    return SV_ERR_INVALID_ARG;
  if (d < 8 || d > 256 || d % 8 != 0) return SV_ERR_INVALID_ARG;
  if (B == 0) return SV_OK;
  if (!k_cache || !v_cache || !prefix_len || !num_accepted || !new_len) return SV_ERR_INVALID_ARG;
  if (!aligned16(k_cache) || !aligned16(v_cache)) return SV_ERR_INVALID_ARG;
  // elements per layer and of the whole cache must fit a signed 64-bit index
  const long long kIdxMax = 1LL << 62;
  long long per_layer = 1;
  for (long long f : {(long long)B, (long long)H, (long long)S_max, (long long)d}) {
    if (per_layer > kIdxMax / f) return SV_ERR_INVALID_ARG;
    per_layer *= f;
  }
  if (layers > 1 && (layer_stride < per_layer || layer_stride % 8 != 0)) return SV_ERR_INVALID_ARG;
  if (layers > 1 && layer_stride > (kIdxMax - per_layer) / (layers - 1)) return SV_ERR_INVALID_ARG;
  if (path_nodes && path_stride < N - 1) return SV_ERR_INVALID_ARG;
  if ((long long)layers * B >= (1LL << 31)) return SV_ERR_INVALID_ARG;
  sv::KvArgs a{};
  a.k = (uint16_t*)k_cache;
  a.v = (uint16_t*)v_cache;
  a.layer_stride = layers > 1 ? layer_stride : per_layer;
  a.prefix_len = prefix_len;
  a.num_accepted = num_accepted;
  a.path = path_nodes;
  a.path_stride = path_stride;
  a.layers = layers;
  a.B = B;
  a.H = H;
  a.S_max = S_max;
  a.d = d;
  a.n_new = N;
  a.new_len = new_len;
  const ProfHook h = take_prof_hook();
  if (sv::launch_kv_commit(a, stream, h.begin, h.end) != hipSuccess) return SV_ERR_HIP;
  return SV_OK;
}

int spec_verify_telemetry_linear(const int32_t* num_accepted, const int32_t* draft_offsets,
                                 int B, sv_telemetry* acc, hipStream_t stream) {
  if (B < 0) return SV_ERR_INVALID_ARG;
  if (B == 0) return SV_OK;
  if (!num_accepted || !draft_offsets || !acc || ((uintptr_t)acc & 7u)) return SV_ERR_INVALID_ARG;
  if (sv::launch_telemetry_linear(num_accepted, draft_offsets, B, acc, stream) != hipSuccess)
    return SV_ERR_HIP;
  return SV_OK;
}

int spec_verify_telemetry_tree(const int32_t* num_accepted, const int32_t* path_nodes,
                               const int32_t* parents, const int32_t* n_nodes, int B, int N,
                               sv_telemetry* acc, hipStream_t stream) {
  if (B < 0 || N < 1 || N > SV_MAX_TREE_NODES) return SV_ERR_INVALID_ARG;
  if (B == 0) return SV_OK;
  if (!num_accepted || !parents || !acc || ((uintptr_t)acc & 7u)) return SV_ERR_INVALID_ARG;
  if (N > 1 && !path_nodes) return SV_ERR_INVALID_ARG;
  if (sv::launch_telemetry_tree(num_accepted, path_nodes, parents, n_nodes, B, N, acc, stream) !=
      hipSuccess)
    return SV_ERR_HIP;
  return SV_OK;
}

int spec_verify_telemetry_summary(const sv_telemetry* acc, double* out, hipStream_t stream) {
  if (!acc || !out || ((uintptr_t)acc & 7u) || ((uintptr_t)out & 7u)) return SV_ERR_INVALID_ARG;
  if (sv::launch_telemetry_summary(acc, out, stream) != hipSuccess) return SV_ERR_HIP;
  return SV_OK;
}

int spec_verify_draft_topk(const void* logits, int dtype, int R, int V, int k,
                           const float* temp, int32_t* tokens, float* logprob,
                           hipStream_t stream) {
  if (dtype != SV_F32 && dtype != SV_BF16) return SV_ERR_INVALID_ARG;
  if (R < 0 || V < 1 || k < 1 || k > SV_MAX_TOPK || k > V) return SV_ERR_INVALID_ARG;
  if (R == 0) return SV_OK;
  if (!logits || !tokens || !logprob) return SV_ERR_INVALID_ARG;
  if (sv::launch_draft_topk(dtype, logits, R, V, k, temp, tokens, logprob, stream) != hipSuccess)
    return SV_ERR_HIP;
  return SV_OK;
}

int spec_verify_tree_prune(const int32_t* cand_parent, const int32_t* cand_token,
                           const float* cand_logq, const int32_t* n_cand, int B, int C, int n_max,
                           double tau, int32_t* parents, int32_t* tokens, float* cum_logprob,
                           int32_t* n_nodes, int32_t* n_pass, hipStream_t stream) {
  if (B < 0 || C < 0 || C > SV_MAX_CANDIDATES || n_max < 1 || n_max > SV_MAX_TREE_NODES)
    return SV_ERR_INVALID_ARG;
  if (!(tau >= 0.0)) return SV_ERR_INVALID_ARG;
  if (B == 0) return SV_OK;
  if (!parents || !tokens || !cum_logprob || !n_nodes) return SV_ERR_INVALID_ARG;
  if (C > 0 && (!cand_parent || !cand_token || !cand_logq)) return SV_ERR_INVALID_ARG;
  sv::TreePruneArgs a{};
  a.cand_parent = cand_parent;
  a.cand_token = cand_token;
  a.cand_logq = cand_logq;
  a.n_cand = n_cand;
  a.B = B;
  a.C = C;
  a.n_max = n_max;
  a.tau = tau;
  a.parents = parents;
  a.tokens = tokens;
  a.cum_logprob = cum_logprob;
  a.n_nodes = n_nodes;
  a.n_pass = n_pass;
  if (sv::launch_tree_prune(a, stream) != hipSuccess) return SV_ERR_HIP;
  return SV_OK;
}

int spec_verify_gamma_update(uint32_t* history, const int32_t* num_accepted,
                             const int32_t* draft_offsets, const float* temp_target,
                             int couple_temperature, int B, int32_t* gamma_next,
                             int32_t* draft_offsets_next, hipStream_t stream) {
  if (B < 0) return SV_ERR_INVALID_ARG;
  if (B == 0) return SV_OK;
  if (!history || !num_accepted || !draft_offsets || !gamma_next) return SV_ERR_INVALID_ARG;
  if (couple_temperature && !temp_target) return SV_ERR_INVALID_ARG;
  if ((long long)B * 8 >= (1LL << 31)) return SV_ERR_INVALID_ARG;   // offsets stay in int32
  if (sv::launch_gamma_update(history, num_accepted, draft_offsets, temp_target,
                              couple_temperature ? 1 : 0, B, gamma_next, draft_offsets_next,
                              stream) != hipSuccess)
    return SV_ERR_HIP;
  return SV_OK;
}

int spec_verify_philox_words(uint64_t seed, uint64_t step, const uint32_t* row_ids, int n_rows,
                             int n_slots, uint32_t* out_words, hipStream_t stream) {
  if (n_rows < 0 || n_slots < 0) return SV_ERR_INVALID_ARG;
  if ((long long)n_rows * n_slots == 0) return SV_OK;
  if (!out_words || !aligned16(out_words)) return SV_ERR_INVALID_ARG;
  if ((long long)n_rows * n_slots >= (1LL << 31) * 256LL) return SV_ERR_INVALID_ARG;
  if (sv::launch_philox_words(seed, step, row_ids, n_rows, n_slots, out_words, stream) !=
      hipSuccess)
    return SV_ERR_HIP;
  return SV_OK;
}

int spec_verify_exp2(const float* x, float* y, int n, hipStream_t stream) {
  if (n < 0) return SV_ERR_INVALID_ARG;
  if (n == 0) return SV_OK;
  if (!x || !y) return SV_ERR_INVALID_ARG;
  if (sv::launch_exp2_words(x, y, n, stream) != hipSuccess) return SV_ERR_HIP;
  return SV_OK;
}

int spec_verify_profile_next(hipEvent_t begin, hipEvent_t end) {
  t_prof = ProfHook{begin, end};
  return SV_OK;
}

}  // extern "C"
