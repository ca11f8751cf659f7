/*
 * spec_verify.h -- C ABI of the speculative-decoding verify step on MI355X (gfx950).
 *
 * The verify step of speculative decoding: after a draft model proposes
 * gamma tokens (or a tree of tokens), the target model scores them in one
 * forward pass; each draft token d is accepted with probability
 * min(1, p(d)/q(d)), the first rejection ends the round, and the round
 * emits one more token drawn from the normalised residual max(0, p - q)
 * after a rejection, or from p after the last draft when every draft was
 * accepted.  Sources (page address, section):
 *   - kwkr.cn/news/620872 §2.1 (one target pass scores all positions under a
 *     causal mask), §2.3 and §4.1 (accept when p >= q, else with probability
 *     p/q; the result keeps the target law), §4.3 (greedy decoding turns the
 *     test into exact match; stop at the first rejection), §5.3 (tree
 *     verification);
 *   - cf-1.com/news/5632551 §2.2 (probability-ratio test), §2.3 (gamma,
 *     alpha, c; expected tokens per round), §3.3 (all-accept / all-reject
 *     cases and KV rollback), §5.4 (token trees and their mask matrix);
 *   - blog.lonae.com/posts/2026-draft-model-kv-jDwzYp ("推测解码的工程真相
 *     2026"), formal-definition paragraph (verify gamma drafts plus one
 *     bonus position; residual max(0, pi_t - pi_d)), tree-attention
 *     paragraphs (top-k or sampled children; per-tree causal mask).
 *
 * Conventions shared by every entry point
 *   - Every pointer is device memory unless stated otherwise, owned by the
 *     caller.  The library allocates nothing and keeps no state between
 *     calls (the one-shot timing hook below aside); scratch space is the
 *     caller's workspace.
 *   - Calls are asynchronous on `stream` and never synchronise the host.
 *     Argument checks that need no device data happen on the host before
 *     anything is enqueued; a non-zero return means nothing was enqueued,
 *     except SV_ERR_HIP, which reports a failed kernel launch.
 *   - Contract violations found in device data (a token outside [0, V), a
 *     bad offset or parent, a negative or non-finite temperature, a row whose
 *     logits have no finite maximum) are reported per batch row in
 *     `row_status` and do not stop the other rows.  An error row gets
 *     num_accepted = -1 and -1 in every output token slot it owns.  NaN
 *     logits are undefined behaviour (no fault, unspecified outputs).
 *   - Outputs are a pure function of (inputs, seed, step, row ids): the same
 *     call gives the same bits on every run and for any launch geometry.
 *   - Draft and target share one vocabulary of size V.
 *   - A workspace must not be shared by calls that may run concurrently.
 *
 * Randoms: Philox-4x32-10 (Salmon et al., SC'11), key = (seed low word,
 * seed high word), counter = (slot, row id, step low word, step high word).
 * u_acc = (x0 >> 8) * 2^-24 decides the acceptance of the token in `slot`;
 * u_smp = (x1 >> 8) * 2^-24 drives the inverse-CDF draw made after `slot`.
 * Slot 0 is the last committed token; draft d_i of the linear verify sits in
 * slot i + 1; a tree node's slot is its node index.  The row id is
 * row_ids[b] (or b when row_ids is NULL), never a packed index, so packing
 * does not change a row's randoms.
 */
#ifndef SPEC_VERIFY_H
#define SPEC_VERIFY_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Return codes. */
#define SV_OK 0
#define SV_ERR_INVALID_ARG (-1) /* null pointer, bad size, dtype, N > 64, ... */
#define SV_ERR_UNSUPPORTED (-2) /* valid request the library does not implement */
#define SV_ERR_WORKSPACE (-3)   /* workspace missing, too small or misaligned */
#define SV_ERR_HIP (-4)         /* a kernel launch failed */
#define SV_ERR_SCRATCH (-5)     /* needs more than the static scratch of a _noalloc call */

/* Logit element types. */
#define SV_F32 0
#define SV_BF16 1

/* Tree candidate modes. */
#define SV_TREE_TOPK 0        /* children are the draft's deterministic top-k */
#define SV_TREE_SAMPLED_WOR 1 /* children drawn from q without replacement */

/* Per-row status bits.  Bits 0-7 are errors, bits 8+ are warnings. */
#define SV_ROW_OK 0
#define SV_ROW_BAD_TOKEN 1      /* a draft / node token outside [0, V) */
#define SV_ROW_BAD_SHAPE 2      /* bad offsets (gamma_b < 0 or > 64) or parents / n_nodes */
#define SV_ROW_NONFINITE 4      /* a logit row without a finite maximum */
#define SV_ROW_BAD_TEMP 8       /* negative or non-finite temperature */
#define SV_ROW_WARN_QZERO 256   /* q(d) = 0 for a tested draft token (ratio taken as +inf or 0) */
#define SV_ROW_WARN_RZERO 512   /* rejection with zero residual mass: drew from p instead */

#define SV_MAX_GAMMA 64
#define SV_MAX_TREE_NODES 64
#define SV_MAX_TOPK 64
#define SV_MAX_CANDIDATES 1024
#define SV_WORKSPACE_ALIGN 256
#define SV_STATIC_SCRATCH_BYTES (4u << 20) /* per-GPU scratch of spec_verify_linear_noalloc */

/* Library version, (major << 16) | minor. */
int spec_verify_version(void);

/* Static, human-readable text for a return code. */
const char* spec_verify_status_string(int status);

/*
 * Linear verify (kwkr §2.3, §4.1, §4.3; cf-1 §2.2; lonae formal-definition
 * paragraph).  Batch row b has gamma_b = draft_offsets[b+1] - draft_offsets[b]
 * draft tokens (0 <= gamma_b <= 64).
 *
 *   target_logits  [sum_b (gamma_b + 1), V], row-major, `dtype` elements.
 *                  The gamma_b + 1 target rows of b start at row
 *                  draft_offsets[b] + b; row i is the target's distribution
 *                  for slot i + 1 (row gamma_b follows the last draft).
 *   draft_logits   [total_draft, V]; the draft rows of b start at row
 *                  draft_offsets[b]; row i is the distribution d_i was drawn
 *                  from.
 *   dtype          SV_F32 or SV_BF16.  Rows whose byte length is not a
 *                  multiple of 16 are handled, more slowly.
 *   B, V           batch rows (>= 0; 0 is a no-op) and vocabulary size (>= 1).
 *   total_draft    draft_offsets[B] (host copy, sizes the launch).
 *   draft_offsets  [B + 1] int32, non-decreasing, draft_offsets[0] = 0.
 *                  A row whose own offsets are out of range is flagged
 *                  SV_ROW_BAD_SHAPE; when the offsets are not
 *                  non-decreasing, the other rows' results are unspecified
 *                  (the packed row -> batch row mapping is then ambiguous).
 *   draft_tokens   [total_draft] int32 draft token ids.
 *   temp_target, temp_draft  [B] float temperatures; 0 means greedy (a
 *                  one-hot at the first maximum, kwkr §4.3).
 *   seed, step, row_ids  Philox key / counter words (row_ids may be NULL).
 * Outputs:
 *   num_accepted   [B] int32: accepted drafts, or -1 for an error row.
 *   out_tokens     [sum_b (gamma_b + 1)] int32, same packing as the target
 *                  rows: the accepted drafts, then the residual or bonus
 *                  token, then -1.
 *   p_at_draft, q_at_draft  [total_draft] float p_i(d_i), q_i(d_i); may be NULL.
 *   row_status     [B] int32 SV_ROW_* bits; may be NULL.
 *   workspace      device scratch of spec_verify_linear_workspace_size()
 *                  bytes, SV_WORKSPACE_ALIGN-aligned; contents need no
 *                  initialisation and are clobbered.
 * Returns SV_OK or a negative SV_ERR_* code.
 */
size_t spec_verify_linear_workspace_size(int B, int total_draft, int V, int dtype);
int spec_verify_linear(const void* target_logits, const void* draft_logits, int dtype,
                       int B, int V, int total_draft,
                       const int32_t* draft_offsets, const int32_t* draft_tokens,
                       const float* temp_target, const float* temp_draft,
                       uint64_t seed, uint64_t step, const uint32_t* row_ids,
                       int32_t* num_accepted, int32_t* out_tokens,
                       float* p_at_draft, float* q_at_draft, int32_t* row_status,
                       void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * For callers that cannot allocate device memory: code under HIP graph
 * capture that must not call hipMalloc, tight serving loops, and harnesses
 * that forbid allocation.  The same verify as spec_verify_linear (same
 * arguments, outputs, row statuses and results), without the workspace
 * arguments: the workspace is a static device array of
 * SV_STATIC_SCRATCH_BYTES (4 MiB) that the library keeps on each GPU it runs
 * on until the process ends.  The call allocates nothing; the caller still
 * passes inputs and outputs.  The GPU is the calling thread's current device.
 *
 * Returns SV_ERR_SCRATCH, before any launch, when
 * spec_verify_linear_workspace_size(B, total_draft, V, dtype) exceeds
 * SV_STATIC_SCRATCH_BYTES (B = 256 rows with 1130 drafts at V = 152064 need
 * about 1.4 MB); SV_ERR_HIP when the array's device address cannot be had;
 * otherwise what spec_verify_linear returns.  Nothing in the array has to
 * start at zero: a call reads only bytes it wrote earlier in the same call.
 * Every call on one GPU shares that GPU's array: calls that overlap in time
 * on one GPU (on two streams, or from two host threads without ordering)
 * race on it and give undefined results; calls ordered on one stream do not.
 */
int spec_verify_linear_noalloc(const void* target_logits, const void* draft_logits, int dtype,
                               int B, int V, int total_draft, const int32_t* draft_offsets,
                               const int32_t* draft_tokens, const float* temp_target,
                               const float* temp_draft, uint64_t seed, uint64_t step,
                               const uint32_t* row_ids, int32_t* num_accepted,
                               int32_t* out_tokens, float* p_at_draft, float* q_at_draft,
                               int32_t* row_status, hipStream_t stream);

/*
 * Tree verify (kwkr §5.3; cf-1 §5.4; lonae tree-attention paragraphs), TOPK
 * mode: the children of a node are tested in node-index order; child c_j is
 * accepted when u_acc(c_j) < p'(c_j), p' being the node's target
 * distribution with the tokens of the already-rejected siblings removed and
 * renormalised; on acceptance the walk descends; when every child is
 * rejected the emitted token is drawn from p with all of them removed; at a
 * leaf the bonus token is drawn from p (draws use u_smp of the stop node).
 *
 * SAMPLED_WOR mode (the tree-attention paragraph's temperature-sampled
 * children): the children of a node were drawn from its draft distribution
 * q without replacement.  Child c_j is accepted when
 * u_acc(c_j) < p_j(c_j) / q_j(c_j), where q_j is q with the tokens of
 * c_1..c_{j-1} removed and renormalised, p_1 = p, and each rejection sets
 * p_{j+1} = norm(max(0, p_j - q_j)) (left as p_j when that is empty,
 * SV_ROW_WARN_RZERO); when every child is rejected the token is drawn from
 * the last p_{k+1}; at a leaf the bonus is drawn from p.  A tested child
 * with q_j(c_j) = 0 sets SV_ROW_WARN_QZERO (ratio +inf, or 0 if p_j is 0 too).
 * Each rejected sibling costs one extra pass over its node's two rows.
 *
 *   target_logits  [B, N, V] `dtype`; row n is the target's distribution for
 *                  the token that follows node n (node 0 = root = the last
 *                  committed token).
 *   draft_logits   [B, N, V] `dtype`, SAMPLED_WOR only (else may be NULL):
 *                  row n is the draft distribution that n's children were
 *                  drawn from; rows of nodes without children are not read.
 *   N              nodes per tree including the root, 1..64.
 *   parents        [B, N] int32; parents[b][0] is ignored; for 0 < i <
 *                  n_nodes[b], 0 <= parents[b][i] < i.
 *   node_tokens    [B, N] int32; node 0's entry is ignored.
 *   n_nodes        [B] int32 in 1..N, or NULL for N everywhere.
 *   cand_mode      SV_TREE_TOPK or SV_TREE_SAMPLED_WOR; any other value is
 *                  SV_ERR_INVALID_ARG, as is SAMPLED_WOR without draft_logits
 *                  or temp_draft.
 *   temp_target    [B]; temp_draft [B] (SAMPLED_WOR; else may be NULL).
 *                  Every target row n < n_nodes[b], and the draft row of
 *                  every node with a child, needs a finite maximum
 *                  (SV_ROW_NONFINITE otherwise).
 * Outputs:
 *   num_accepted   [B] depth of the accepted path, -1 for an error row.
 *   path_nodes     [B, N-1] node ids of the accepted path, then -1.
 *   out_tokens     [B, N] tokens of the accepted path, then the drawn token, then -1.
 *   p_at_node      [B, N] p_parent(n)(token_n) for 0 < n < n_nodes, else 0; may be NULL.
 *   row_status     [B]; may be NULL.
 *   workspace      spec_verify_tree_workspace_size() bytes (enough for either
 *                  mode), as for the linear call.
 */
size_t spec_verify_tree_workspace_size(int B, int N, int V, int dtype);
int spec_verify_tree(const void* target_logits, const void* draft_logits, int dtype,
                     int B, int N, int V,
                     const int32_t* parents, const int32_t* node_tokens, const int32_t* n_nodes,
                     int cand_mode, const float* temp_target, const float* temp_draft,
                     uint64_t seed, uint64_t step, const uint32_t* row_ids,
                     int32_t* num_accepted, int32_t* path_nodes, int32_t* out_tokens,
                     float* p_at_node, int32_t* row_status,
                     void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Causal- or tree-masked verify attention (kwkr §2.1; cf-1 §5.4; lonae
 * tree-attention paragraphs).  For batch row b with prefix length
 * L = prefix_len[b] and N query tokens whose keys/values are already stored
 * at cache slots [L, L+N):
 *   O[b,h,i] = sum_j softmax_j(Q[b,h,i] . K[b,h,j] * scale + M_ij) V[b,h,j],
 * j over the prefix [0, L) and over L + t for every new token t that is i
 * itself or an ancestor of i in the tree given by `parents` (a chain, i.e. a
 * causal mask, when parents is NULL).  Every head has its own K/V.
 *
 *   q              [B, H, N, d] bf16 (after any positional encoding).
 *   k_cache, v_cache [B, H, S_max, d] bf16.
 *   prefix_len     [B] int32 with 0 <= L and L + N <= S_max (checked on the
 *                  device: a violating row gets zero output and NaN LSE).
 *   parents        [B, N] int32 or NULL; same rules as spec_verify_tree.
 *   N 1..64, d 128, H >= 1, scale usually 1/sqrt(d).
 *   out            [B, H, N, d] bf16.
 *   lse            [B, H, N] float natural-log sum of exp(scores); may be NULL.
 * Arithmetic: bf16 MFMA products, float32 accumulation and softmax; the
 * softmax weights are rounded to bf16 for the P.V product.
 */
int spec_verify_attn(const void* q, const void* k_cache, const void* v_cache,
                     const int32_t* prefix_len, const int32_t* parents,
                     int B, int H, int N, int d, int S_max, float scale,
                     void* out, float* lse, hipStream_t stream);

/*
 * KV-cache commit after a verify round (cf-1 §3.3: reuse the cached prefix,
 * keep the accepted positions, drop every entry after the accept point;
 * kwkr §5.1: one pre-allocated cache spliced by offsets).  The round's
 * forward pass stored the entries of its N new tokens (node 0 = the root,
 * the last committed token) at slots [L, L + N), L = prefix_len[b].  For
 * each batch row with n = num_accepted[b] >= 0 and a valid path, the entry
 * at slot L + path[i] moves to slot L + 1 + i (i < n) in every layer and
 * head of both caches, every source read before any write, and
 * new_len[b] = L + 1 + n.  A row with n < 0 (flagged by the verify call) is
 * left as it is with new_len[b] = L; a row whose L, n or path is malformed
 * (L < 0, L + N > S_max, n > N - 1, node ids not strictly increasing
 * within [1, N)) is left as it is with new_len[b] = -1.  Entries at slots
 * >= new_len[b] are unspecified afterwards.
 *
 *   k_cache, v_cache  [layers][B, H, S_max, d] bf16, 16-byte aligned; layer l
 *                  starts layer_stride elements after layer l - 1 (ignored
 *                  when layers == 1; else >= B H S_max d, a multiple of 8).
 *   prefix_len     [B] int32, the L of the round.
 *   num_accepted   [B] int32, as the verify call returned it.
 *   path_nodes     [B, path_stride] int32 accepted node ids (spec_verify_tree's
 *                  path_nodes, path_stride = N - 1), or NULL for a linear round
 *                  (a chain: nothing moves, only new_len is written).
 *   N 1..64, d 8..256 (a multiple of 8), S_max >= N.
 *   new_len        [B] int32 out.
 * Work items: one per (layer, b); each thread moves 16-byte columns of one head.
 */
int spec_verify_kv_commit(void* k_cache, void* v_cache, int layers, long long layer_stride,
                          const int32_t* prefix_len, const int32_t* num_accepted,
                          const int32_t* path_nodes, int path_stride, int B, int H, int N, int d,
                          int S_max, int32_t* new_len, hipStream_t stream);

/*
 * Round telemetry (blog.lonae.com/posts/2026-draft-model-kv-jDwzYp,
 * observability paragraphs: acceptance rate and its per-request histogram,
 * which must keep the low and the high peak apart; Speculative Efficiency;
 * Tree Width Effective).  Counters are added on the device into a caller-
 * owned sv_telemetry block (zero it to open a window); the summary call
 * derives the signals from a block.
 *
 * Per row of a verify call (rows with num_accepted < 0, or a malformed
 * shape, only add to error_rows): rounds += 1; drafted += the round's draft
 * steps (gamma_b for a linear row, the depth of the deepest node for a
 * tree); accepted += num_accepted; full_accepts += 1 when every step was
 * accepted (a tree walk that ended on a leaf); acc_rate_hist[k] for
 * accepted / drafted in [k/20, (k+1)/20) (1.0 in the last bin; rows with no
 * draft step not binned); accepted_hist[min(n, 64)]; trees also add their
 * root-to-leaf paths to tree_paths, those through the first accepted node
 * to tree_paths_hit, and the rank of every accepted node among its
 * siblings (0 = first child tested) to sibling_rank_hist.
 */
#define SV_TELEM_ACC_BINS 20
#define SV_TELEM_POS_BINS 65
#define SV_TELEM_RANK_BINS 64
typedef struct sv_telemetry {
  uint64_t rounds, error_rows, drafted, accepted, full_accepts, tree_paths, tree_paths_hit;
  uint64_t acc_rate_hist[SV_TELEM_ACC_BINS];
  uint64_t accepted_hist[SV_TELEM_POS_BINS];
  uint64_t sibling_rank_hist[SV_TELEM_RANK_BINS];
} sv_telemetry;

/* Linear rounds: num_accepted [B] and draft_offsets [B+1] as given to and
 * returned by spec_verify_linear. */
int spec_verify_telemetry_linear(const int32_t* num_accepted, const int32_t* draft_offsets,
                                 int B, sv_telemetry* acc, hipStream_t stream);

/* Tree rounds: num_accepted [B] and path_nodes [B, N-1] as returned by
 * spec_verify_tree for parents [B, N] and n_nodes [B] (NULL: N). */
int spec_verify_telemetry_tree(const int32_t* num_accepted, const int32_t* path_nodes,
                               const int32_t* parents, const int32_t* n_nodes, int B, int N,
                               sv_telemetry* acc, hipStream_t stream);

/* Derived signals of a block, out[8] float64 (device memory):
 *   [0] acceptance_rate = accepted / drafted
 *   [1] avg_accepted_tokens = accepted / rounds
 *   [2] draft_steps = drafted / rounds
 *   [3] Speculative Efficiency = [0] * [1] / [2] (with these readings it is
 *       (accepted / drafted)^2, at most 1)
 *   [4] Tree Width Effective = tree_paths_hit / tree_paths
 *   [5..7] bins of acc_rate_hist holding its P50, P95, P99 rows (-1 if empty)
 * NaN where a ratio has no rows. */
int spec_verify_telemetry_summary(const sv_telemetry* acc, double* out, hipStream_t stream);

/*
 * Draft candidates (blog.lonae.com/posts/2026-draft-model-kv-jDwzYp,
 * tree-attention paragraphs: every draft position branches into the
 * draft's top-k candidates).  For each of R draft rows [R, V] `dtype`, the
 * k tokens of largest logit, largest first (equal logits to the lower id;
 * -0 and +0 are equal), and their log-probabilities log softmax(x / T)[token]
 * at the row's temperature (temp [R], NULL for 1; T = 0: 0 for the first
 * token and -inf for the rest; a negative or non-finite T: tokens -1, NaN).
 * 1 <= k <= 64, k <= V.  NaN logits are undefined behaviour.  tokens,
 * logprob: [R, k].  One work item per row: the logits at or above a lower
 * bound of the k-th largest are ranked directly; when more than 1024 tie
 * there, a radix select over the row takes over.
 */
int spec_verify_draft_topk(const void* logits, int dtype, int R, int V, int k,
                           const float* temp, int32_t* tokens, float* logprob, hipStream_t stream);

/*
 * Tree pruning (same paragraphs: the production tree is pruned by
 * cumulative draft probability up to a node budget, not fully expanded).
 * Each batch row holds a forest of C <= 1024 drafted candidates: candidate
 * i has parent cand_parent[i] (-1: a child of the root, else an earlier
 * candidate), token cand_token[i] and cand_logq[i] = log q of the token
 * under its parent's draft row (<= 0).  The kept tree is the n_max - 1
 * candidates of largest cumulative log q (the sum along the path), ties to
 * the shallower, then the earlier parent, then the lower sibling rank, with
 * -inf never kept; it is closed under parents.  Its nodes are numbered
 * breadth first (depth, then the parent's new index, then sibling rank)
 * behind the root, node 0 (parent -1, token -1, cumulative 0): parents and
 * tokens [B, n_max] are spec_verify_tree's inputs, cum_logprob [B, n_max]
 * float, n_nodes [B] (0 for a forest whose parents are malformed), and
 * n_pass [B] (may be NULL) the kept nodes with cumulative probability
 * >= tau.  Slots past n_nodes hold -1 (cumulative -inf).  n_cand [B] may
 * be NULL (C everywhere).  n_max 1..64.
 */
int spec_verify_tree_prune(const int32_t* cand_parent, const int32_t* cand_token,
                           const float* cand_logq, const int32_t* n_cand, int B, int C, int n_max,
                           double tau, int32_t* parents, int32_t* tokens, float* cum_logprob,
                           int32_t* n_nodes, int32_t* n_pass, hipStream_t stream);

/*
 * Dynamic speculation length (blog.lonae.com/posts/2026-draft-model-kv-jDwzYp,
 * bimodal-acceptance paragraph): after a linear round, each request's
 * acceptance over its last 16 steps sets its next gamma: 8 above 60%, 4
 * from 30% to 60%, 2 below 30%; with couple_temperature, a request whose
 * temp_target is above 0.8 gets gamma 1.  A step is one tested draft
 * position: a round that accepted n of its gamma_b drafts adds n accepted
 * steps, then one rejected step if n < gamma_b; a flagged round (n < 0)
 * adds nothing.  The rate is taken over the last min(16, steps seen)
 * steps; a request with none yet gets 4.
 *
 *   history            [B] uint32 in/out: bits 0..15 the last steps (bit 0
 *                      the newest, 1 = accepted), bits 16..20 how many of
 *                      them are valid (0..16).  Zero for a new request.
 *   num_accepted       [B] as returned by spec_verify_linear.
 *   draft_offsets      [B+1] the offsets of that round.
 *   temp_target        [B] or NULL (required with couple_temperature).
 *   gamma_next         [B] int32 out.
 *   draft_offsets_next [B+1] int32 out (running sum of gamma_next), or NULL.
 */
int spec_verify_gamma_update(uint32_t* history, const int32_t* num_accepted,
                             const int32_t* draft_offsets, const float* temp_target,
                             int couple_temperature, int B, int32_t* gamma_next,
                             int32_t* draft_offsets_next, hipStream_t stream);

/*
 * Diagnostic: the raw Philox-4x32-10 words the verify calls draw, for
 * n_rows rows (row id row_ids[r], or r when NULL) and slots 0..n_slots-1:
 * out_words[(r * n_slots + s) * 4 + w] = word w of counter
 * (s, row id, step low, step high) under key (seed low, seed high).
 */
int spec_verify_philox_words(uint64_t seed, uint64_t step, const uint32_t* row_ids,
                             int n_rows, int n_slots, uint32_t* out_words, hipStream_t stream);

/*
 * Diagnostic: y[i] = the hardware base-2 exponential (one v_exp_f32) of the
 * float32 x[i], for i < n: the function every probability, stop weight and
 * row sum of the verify calls is formed with (2^(x k - c) with k = log2(e)/T
 * and an integer offset c).  Lets a caller pin its error, which sets how far
 * a draw's cumulative masses may sit from their exact values.  x and y are
 * device arrays of n floats (they may be the same array).  Errors:
 * SV_ERR_INVALID_ARG for n < 0 or a null pointer when n > 0.
 */
int spec_verify_exp2(const float* x, float* y, int n, hipStream_t stream);

/*
 * Diagnostic timing hook (for benchmarks): the calling thread's next
 * spec_verify_linear, spec_verify_tree, spec_verify_attn or
 * spec_verify_kv_commit call attaches `begin` and `end` to the dispatch of
 * its dominant kernel (the vocabulary pass, the attention kernel or the
 * commit kernel), so the events bracket that kernel alone, as a profiler
 * sees it; then the hook forgets both.  Either may be NULL to clear the
 * hook.  The hook is per host thread: a call made on another thread neither
 * sees nor consumes it, so the entry points stay reentrant and thread-safe.
 * Not for use under stream capture.  It changes no output and skips no work.
 */
int spec_verify_profile_next(hipEvent_t begin, hipEvent_t end);

#ifdef __cplusplus
}
#endif

#endif /* SPEC_VERIFY_H */
