"""Python binding of libspecverify.so, the MI355X verify step of speculative decoding.

Argument marshalling only: every step of the verify runs in the HIP kernels
behind the C ABI declared in include/spec_verify.h.  PyTorch supplies device
memory and the current stream.  There is no fallback: if the library is not
built, every call raises.
"""

import ctypes
import os

import torch

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libspecverify.so")

SV_OK = 0
SV_F32 = 0
SV_BF16 = 1
SV_TREE_TOPK = 0
SV_TREE_SAMPLED_WOR = 1
SV_WORKSPACE_ALIGN = 256
SV_STATIC_SCRATCH_BYTES = 4 << 20
SV_ERR_SCRATCH = -5

ROW_BAD_TOKEN = 1
ROW_BAD_SHAPE = 2
ROW_NONFINITE = 4
ROW_BAD_TEMP = 8
ROW_WARN_QZERO = 256
ROW_WARN_RZERO = 512

_lib = None


class SpecVerifyError(RuntimeError):
    def __init__(self, status, what):
        super().__init__("%s: %s (status %d)" % (what, status_string(status), status))
        self.status = status


def library():
    """Load libspecverify.so (raises when it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError("libspecverify.so is not built; run "
                           "`python -m rejection_sampling_verify_04_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, u64, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_uint64, ctypes.c_size_t
    L.spec_verify_version.restype = i32
    L.spec_verify_status_string.restype = ctypes.c_char_p
    L.spec_verify_status_string.argtypes = [i32]
    L.spec_verify_linear_workspace_size.restype = sz
    L.spec_verify_linear_workspace_size.argtypes = [i32, i32, i32, i32]
    L.spec_verify_linear.restype = i32
    L.spec_verify_linear.argtypes = [vp, vp, i32, i32, i32, i32, vp, vp, vp, vp, u64, u64, vp,
                                     vp, vp, vp, vp, vp, vp, sz, vp]
    L.spec_verify_linear_noalloc.restype = i32
    L.spec_verify_linear_noalloc.argtypes = [vp, vp, i32, i32, i32, i32, vp, vp, vp, vp, u64, u64,
                                             vp, vp, vp, vp, vp, vp, vp]
    L.spec_verify_tree_workspace_size.restype = sz
    L.spec_verify_tree_workspace_size.argtypes = [i32, i32, i32, i32]
    L.spec_verify_tree.restype = i32
    L.spec_verify_tree.argtypes = [vp, vp, i32, i32, i32, i32, vp, vp, vp, i32, vp, vp, u64, u64,
                                   vp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.spec_verify_attn.restype = i32
    L.spec_verify_attn.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, ctypes.c_float,
                                   vp, vp, vp]
    L.spec_verify_profile_next.restype = i32
    L.spec_verify_profile_next.argtypes = [vp, vp]
    L.spec_verify_exp2.restype = i32
    L.spec_verify_exp2.argtypes = [vp, vp, i32, vp]
    L.spec_verify_philox_words.restype = i32
    L.spec_verify_philox_words.argtypes = [u64, u64, vp, i32, i32, vp, vp]
    L.spec_verify_telemetry_linear.restype = i32
    L.spec_verify_telemetry_linear.argtypes = [vp, vp, i32, vp, vp]
    L.spec_verify_telemetry_tree.restype = i32
    L.spec_verify_telemetry_tree.argtypes = [vp, vp, vp, vp, i32, i32, vp, vp]
    L.spec_verify_telemetry_summary.restype = i32
    L.spec_verify_telemetry_summary.argtypes = [vp, vp, vp]
    L.spec_verify_draft_topk.restype = i32
    L.spec_verify_draft_topk.argtypes = [vp, i32, i32, i32, i32, vp, vp, vp, vp]
    L.spec_verify_tree_prune.restype = i32
    L.spec_verify_tree_prune.argtypes = [vp, vp, vp, vp, i32, i32, i32, ctypes.c_double, vp, vp,
                                         vp, vp, vp, vp]
    L.spec_verify_gamma_update.restype = i32
    L.spec_verify_gamma_update.argtypes = [vp, vp, vp, vp, i32, i32, vp, vp, vp]
    L.spec_verify_kv_commit.restype = i32
    L.spec_verify_kv_commit.argtypes = [vp, vp, i32, ctypes.c_longlong, vp, vp, vp, i32, i32, i32,
                                        i32, i32, i32, vp, vp]
    _lib = L
    return L


def status_string(status):
    return library().spec_verify_status_string(int(status)).decode()


def version():
    return library().spec_verify_version()


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _dev(t, name, dtype=None):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError("%s must be a CUDA tensor" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if dtype is not None and t.dtype != dtype:
        raise ValueError("%s must have dtype %s, got %s" % (name, dtype, t.dtype))
    return t


def _logit_code(t, name):
    if t.dtype == torch.bfloat16:
        return SV_BF16
    if t.dtype == torch.float32:
        return SV_F32
    raise ValueError("%s must be bfloat16 or float32" % name)


def _workspace(nbytes, device, workspace):
    if workspace is None:
        return torch.empty(max(int(nbytes), SV_WORKSPACE_ALIGN), dtype=torch.uint8, device=device)
    _dev(workspace, "workspace", torch.uint8)
    return workspace


def linear_workspace_size(B, total_draft, V, dtype_code=SV_BF16):
    return library().spec_verify_linear_workspace_size(B, total_draft, V, dtype_code)


def tree_workspace_size(B, N, V, dtype_code=SV_BF16):
    return library().spec_verify_tree_workspace_size(B, N, V, dtype_code)


def verify_linear(target_logits, draft_logits, draft_offsets, draft_tokens, temp_target,
                  temp_draft, seed=0, step=0, row_ids=None, want_probs=True, workspace=None,
                  outputs=None, stream=None):
    """Linear verify (see spec_verify_linear).  Returns a dict of output tensors.

    target_logits [sum(gamma_b + 1), V] and draft_logits [sum(gamma_b), V]
    (bf16 or fp32, same dtype); draft_offsets [B+1], draft_tokens
    [sum(gamma_b)] int32; temp_target, temp_draft [B] float32; row_ids [B]
    int32 (reinterpreted as uint32) or None.
    """
    L = library()
    _dev(target_logits, "target_logits")
    _dev(draft_logits, "draft_logits", target_logits.dtype)
    dt = _logit_code(target_logits, "target_logits")
    _dev(draft_offsets, "draft_offsets", torch.int32)
    _dev(draft_tokens, "draft_tokens", torch.int32)
    _dev(temp_target, "temp_target", torch.float32)
    _dev(temp_draft, "temp_draft", torch.float32)
    if row_ids is not None:
        _dev(row_ids, "row_ids", torch.int32)
    B = draft_offsets.numel() - 1
    total = draft_tokens.numel()
    V = target_logits.shape[-1]
    dev = target_logits.device
    if outputs is None:
        outputs = dict(
            num_accepted=torch.empty(B, dtype=torch.int32, device=dev),
            out_tokens=torch.empty(total + B, dtype=torch.int32, device=dev),
            row_status=torch.empty(B, dtype=torch.int32, device=dev))
        if want_probs:
            outputs["p_at_draft"] = torch.empty(total, dtype=torch.float32, device=dev)
            outputs["q_at_draft"] = torch.empty(total, dtype=torch.float32, device=dev)
    need = L.spec_verify_linear_workspace_size(B, total, V, dt)
    ws = _workspace(need, dev, workspace)
    st = L.spec_verify_linear(
        _ptr(target_logits), _ptr(draft_logits), dt, B, V, total, _ptr(draft_offsets),
        _ptr(draft_tokens), _ptr(temp_target), _ptr(temp_draft), int(seed), int(step),
        _ptr(row_ids), _ptr(outputs["num_accepted"]), _ptr(outputs["out_tokens"]),
        _ptr(outputs.get("p_at_draft")), _ptr(outputs.get("q_at_draft")),
        _ptr(outputs.get("row_status")), _ptr(ws), ws.numel(), _stream(stream))
    if st != SV_OK:
        raise SpecVerifyError(st, "spec_verify_linear")
    return outputs


def verify_linear_noalloc(target_logits, draft_logits, draft_offsets, draft_tokens, temp_target,
                          temp_draft, seed=0, step=0, row_ids=None, outputs=None, stream=None):
    """Linear verify with the library's static per-GPU scratch as its workspace
    (see spec_verify_linear_noalloc): nothing is allocated when `outputs`
    (the dict verify_linear returns) is passed in."""
    L = library()
    _dev(target_logits, "target_logits")
    _dev(draft_logits, "draft_logits", target_logits.dtype)
    dt = _logit_code(target_logits, "target_logits")
    _dev(draft_offsets, "draft_offsets", torch.int32)
    _dev(draft_tokens, "draft_tokens", torch.int32)
    _dev(temp_target, "temp_target", torch.float32)
    _dev(temp_draft, "temp_draft", torch.float32)
    if row_ids is not None:
        _dev(row_ids, "row_ids", torch.int32)
    B = draft_offsets.numel() - 1
    total = draft_tokens.numel()
    V = target_logits.shape[-1]
    dev = target_logits.device
    if outputs is None:
        outputs = dict(
            num_accepted=torch.empty(B, dtype=torch.int32, device=dev),
            out_tokens=torch.empty(total + B, dtype=torch.int32, device=dev),
            row_status=torch.empty(B, dtype=torch.int32, device=dev),
            p_at_draft=torch.empty(total, dtype=torch.float32, device=dev),
            q_at_draft=torch.empty(total, dtype=torch.float32, device=dev))
    st = L.spec_verify_linear_noalloc(
        _ptr(target_logits), _ptr(draft_logits), dt, B, V, total, _ptr(draft_offsets),
        _ptr(draft_tokens), _ptr(temp_target), _ptr(temp_draft), int(seed), int(step),
        _ptr(row_ids), _ptr(outputs["num_accepted"]), _ptr(outputs["out_tokens"]),
        _ptr(outputs.get("p_at_draft")), _ptr(outputs.get("q_at_draft")),
        _ptr(outputs.get("row_status")), _stream(stream))
    if st != SV_OK:
        raise SpecVerifyError(st, "spec_verify_linear_noalloc")
    return outputs


def verify_tree(target_logits, parents, node_tokens, temp_target, n_nodes=None, seed=0, step=0,
                row_ids=None, cand_mode=SV_TREE_TOPK, draft_logits=None, temp_draft=None,
                want_probs=True, workspace=None, outputs=None, stream=None):
    """Tree verify (see spec_verify_tree).  target_logits [B, N, V]; parents,
    node_tokens [B, N] int32; n_nodes [B] int32 or None.  SV_TREE_SAMPLED_WOR
    also takes draft_logits (same shape and dtype) and temp_draft [B]."""
    L = library()
    _dev(target_logits, "target_logits")
    dt = _logit_code(target_logits, "target_logits")
    if target_logits.dim() != 3:
        raise ValueError("target_logits must be [B, N, V]")
    B, N, V = target_logits.shape
    if cand_mode == SV_TREE_SAMPLED_WOR:
        if draft_logits is None or temp_draft is None:
            raise ValueError("SV_TREE_SAMPLED_WOR needs draft_logits and temp_draft")
        _dev(draft_logits, "draft_logits")
        if draft_logits.dtype != target_logits.dtype or draft_logits.shape != target_logits.shape:
            raise ValueError("draft_logits must match target_logits in shape and dtype")
        _dev(temp_draft, "temp_draft", torch.float32)
    _dev(parents, "parents", torch.int32)
    _dev(node_tokens, "node_tokens", torch.int32)
    _dev(temp_target, "temp_target", torch.float32)
    if n_nodes is not None:
        _dev(n_nodes, "n_nodes", torch.int32)
    if row_ids is not None:
        _dev(row_ids, "row_ids", torch.int32)
    dev = target_logits.device
    if outputs is None:
        outputs = dict(
            num_accepted=torch.empty(B, dtype=torch.int32, device=dev),
            path_nodes=torch.empty((B, max(N - 1, 1)), dtype=torch.int32, device=dev),
            out_tokens=torch.empty((B, N), dtype=torch.int32, device=dev),
            row_status=torch.empty(B, dtype=torch.int32, device=dev))
        if want_probs:
            outputs["p_at_node"] = torch.empty((B, N), dtype=torch.float32, device=dev)
    need = L.spec_verify_tree_workspace_size(B, N, V, dt)
    ws = _workspace(need, dev, workspace)
    st = L.spec_verify_tree(
        _ptr(target_logits), _ptr(draft_logits), dt, B, N, V, _ptr(parents), _ptr(node_tokens),
        _ptr(n_nodes), int(cand_mode), _ptr(temp_target), _ptr(temp_draft), int(seed), int(step),
        _ptr(row_ids), _ptr(outputs["num_accepted"]), _ptr(outputs["path_nodes"]),
        _ptr(outputs["out_tokens"]), _ptr(outputs.get("p_at_node")),
        _ptr(outputs.get("row_status")), _ptr(ws), ws.numel(), _stream(stream))
    if st != SV_OK:
        raise SpecVerifyError(st, "spec_verify_tree")
    return outputs


def verify_attn(q, k_cache, v_cache, prefix_len, parents=None, scale=None, want_lse=True,
                outputs=None, stream=None):
    """Verify attention (see spec_verify_attn).  q [B,H,N,d], k/v [B,H,S_max,d] bf16."""
    L = library()
    _dev(q, "q", torch.bfloat16)
    _dev(k_cache, "k_cache", torch.bfloat16)
    _dev(v_cache, "v_cache", torch.bfloat16)
    _dev(prefix_len, "prefix_len", torch.int32)
    if parents is not None:
        _dev(parents, "parents", torch.int32)
    B, H, N, d = q.shape
    S_max = k_cache.shape[2]
    if tuple(k_cache.shape) != (B, H, S_max, d) or tuple(v_cache.shape) != (B, H, S_max, d):
        raise ValueError("k_cache / v_cache must be [B, H, S_max, d] matching q")
    if scale is None:
        scale = d ** -0.5
    dev = q.device
    if outputs is None:
        outputs = dict(out=torch.empty_like(q))
        if want_lse:
            outputs["lse"] = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    st = L.spec_verify_attn(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(prefix_len),
                            _ptr(parents), B, H, N, d, S_max, float(scale),
                            _ptr(outputs["out"]), _ptr(outputs.get("lse")), _stream(stream))
    if st != SV_OK:
        raise SpecVerifyError(st, "spec_verify_attn")
    return outputs


def kv_commit(k_cache, v_cache, prefix_len, num_accepted, path_nodes=None, n_new=None,
              new_len=None, stream=None):
    """KV-cache commit after a verify round (see spec_verify_kv_commit), in place.

    k_cache, v_cache: [B, H, S_max, d] or [layers, B, H, S_max, d] bf16;
    prefix_len, num_accepted: [B] int32; path_nodes: [B, N-1] int32 from
    verify_tree, or None for a linear round (then n_new = gamma + 1 must be
    given).  Returns new_len [B] int32.
    """
    L = library()
    for t, name in ((k_cache, "k_cache"), (v_cache, "v_cache")):
        _dev(t, name, torch.bfloat16)
    if k_cache.shape != v_cache.shape:
        raise ValueError("k_cache and v_cache must have the same shape")
    if k_cache.dim() == 4:
        layers, (B, H, S_max, d) = 1, k_cache.shape
    elif k_cache.dim() == 5:
        layers, B, H, S_max, d = k_cache.shape
    else:
        raise ValueError("k_cache must be [B, H, S_max, d] or [layers, B, H, S_max, d]")
    _dev(prefix_len, "prefix_len", torch.int32)
    _dev(num_accepted, "num_accepted", torch.int32)
    if path_nodes is not None:
        _dev(path_nodes, "path_nodes", torch.int32)
        if n_new is None:
            n_new = path_nodes.shape[1] + 1
        stride = path_nodes.shape[1]
    else:
        stride = 0
    if n_new is None:
        raise ValueError("n_new is needed for a linear round")
    if new_len is None:
        new_len = torch.empty(B, dtype=torch.int32, device=k_cache.device)
    st = L.spec_verify_kv_commit(
        _ptr(k_cache), _ptr(v_cache), layers, B * H * S_max * d, _ptr(prefix_len),
        _ptr(num_accepted), _ptr(path_nodes), stride, B, H, int(n_new), d, S_max, _ptr(new_len),
        _stream(stream))
    if st != SV_OK:
        raise SpecVerifyError(st, "spec_verify_kv_commit")
    return new_len


def draft_topk(logits, k, temp=None, stream=None):
    """Top-k candidates of draft rows (see spec_verify_draft_topk).

    logits: [R, V] bf16 or fp32; temp: [R] float32 or None (1).
    Returns (tokens [R, k] int32, logprob [R, k] float32).
    """
    L = library()
    _dev(logits, "logits")
    dt = _logit_code(logits, "logits")
    R, V = logits.shape
    if temp is not None:
        _dev(temp, "temp", torch.float32)
    tokens = torch.empty((R, k), dtype=torch.int32, device=logits.device)
    logprob = torch.empty((R, k), dtype=torch.float32, device=logits.device)
    st = L.spec_verify_draft_topk(_ptr(logits), dt, R, V, int(k), _ptr(temp), _ptr(tokens),
                                  _ptr(logprob), _stream(stream))
    if st != SV_OK:
        raise SpecVerifyError(st, "spec_verify_draft_topk")
    return tokens, logprob


def tree_prune(cand_parent, cand_token, cand_logq, n_max, tau=0.1, n_cand=None, stream=None):
    """Prune drafted candidate forests into verify trees (see spec_verify_tree_prune).

    cand_*: [B, C] (int32, int32, float32).  Returns dict with parents, tokens
    [B, n_max] int32, cum_logprob [B, n_max] float32, n_nodes [B], n_pass [B].
    """
    L = library()
    _dev(cand_parent, "cand_parent", torch.int32)
    _dev(cand_token, "cand_token", torch.int32)
    _dev(cand_logq, "cand_logq", torch.float32)
    if n_cand is not None:
        _dev(n_cand, "n_cand", torch.int32)
    B, C = cand_parent.shape
    dev = cand_parent.device
    out = dict(parents=torch.empty((B, n_max), dtype=torch.int32, device=dev),
               tokens=torch.empty((B, n_max), dtype=torch.int32, device=dev),
               cum_logprob=torch.empty((B, n_max), dtype=torch.float32, device=dev),
               n_nodes=torch.empty(B, dtype=torch.int32, device=dev),
               n_pass=torch.empty(B, dtype=torch.int32, device=dev))
    st = L.spec_verify_tree_prune(_ptr(cand_parent), _ptr(cand_token), _ptr(cand_logq),
                                  _ptr(n_cand), B, C, int(n_max), float(tau),
                                  _ptr(out["parents"]), _ptr(out["tokens"]),
                                  _ptr(out["cum_logprob"]), _ptr(out["n_nodes"]),
                                  _ptr(out["n_pass"]), _stream(stream))
    if st != SV_OK:
        raise SpecVerifyError(st, "spec_verify_tree_prune")
    return out


def gamma_update(history, num_accepted, draft_offsets, temp_target=None,
                 couple_temperature=False, gamma_next=None, draft_offsets_next=None,
                 stream=None):
    """Dynamic speculation length after a linear round (see spec_verify_gamma_update).

    history: [B] int32 words updated in place (zeros for new requests).
    Returns (gamma_next [B], draft_offsets_next [B+1]) int32 on the device.
    """
    L = library()
    _dev(history, "history", torch.int32)
    _dev(num_accepted, "num_accepted", torch.int32)
    _dev(draft_offsets, "draft_offsets", torch.int32)
    if temp_target is not None:
        _dev(temp_target, "temp_target", torch.float32)
    B = history.shape[0]
    dev = history.device
    if gamma_next is None:
        gamma_next = torch.empty(B, dtype=torch.int32, device=dev)
    if draft_offsets_next is None:
        draft_offsets_next = torch.empty(B + 1, dtype=torch.int32, device=dev)
    st = L.spec_verify_gamma_update(_ptr(history), _ptr(num_accepted), _ptr(draft_offsets),
                                    _ptr(temp_target), int(bool(couple_temperature)), B,
                                    _ptr(gamma_next), _ptr(draft_offsets_next), _stream(stream))
    if st != SV_OK:
        raise SpecVerifyError(st, "spec_verify_gamma_update")
    return gamma_next, draft_offsets_next


TELEMETRY_FIELDS = ["rounds", "error_rows", "drafted", "accepted", "full_accepts", "tree_paths",
                    "tree_paths_hit"]
TELEMETRY_BINS = [("acc_rate_hist", 20), ("accepted_hist", 65), ("sibling_rank_hist", 64)]
TELEMETRY_WORDS = len(TELEMETRY_FIELDS) + sum(n for _, n in TELEMETRY_BINS)
SUMMARY_FIELDS = ["acceptance_rate", "avg_accepted_tokens", "draft_steps",
                  "speculative_efficiency", "tree_width_effective", "acc_rate_p50_bin",
                  "acc_rate_p95_bin", "acc_rate_p99_bin"]


def telemetry_block(device="cuda"):
    """A zeroed sv_telemetry block (int64 words) that opens a window."""
    return torch.zeros(TELEMETRY_WORDS, dtype=torch.int64, device=device)


def telemetry_linear(num_accepted, draft_offsets, acc, stream=None):
    """Add the rows of a linear verify call to `acc` (see spec_verify_telemetry_linear)."""
    L = library()
    _dev(num_accepted, "num_accepted", torch.int32)
    _dev(draft_offsets, "draft_offsets", torch.int32)
    _dev(acc, "acc", torch.int64)
    st = L.spec_verify_telemetry_linear(_ptr(num_accepted), _ptr(draft_offsets),
                                        num_accepted.shape[0], _ptr(acc), _stream(stream))
    if st != SV_OK:
        raise SpecVerifyError(st, "spec_verify_telemetry_linear")
    return acc


def telemetry_tree(num_accepted, path_nodes, parents, acc, n_nodes=None, stream=None):
    """Add the rows of a tree verify call to `acc` (see spec_verify_telemetry_tree)."""
    L = library()
    _dev(num_accepted, "num_accepted", torch.int32)
    _dev(path_nodes, "path_nodes", torch.int32)
    _dev(parents, "parents", torch.int32)
    _dev(acc, "acc", torch.int64)
    if n_nodes is not None:
        _dev(n_nodes, "n_nodes", torch.int32)
    B, N = parents.shape
    st = L.spec_verify_telemetry_tree(_ptr(num_accepted), _ptr(path_nodes), _ptr(parents),
                                      _ptr(n_nodes), B, N, _ptr(acc), _stream(stream))
    if st != SV_OK:
        raise SpecVerifyError(st, "spec_verify_telemetry_tree")
    return acc


def telemetry_summary(acc, stream=None):
    """The derived signals of a block, [8] float64 on the device (SUMMARY_FIELDS order)."""
    L = library()
    _dev(acc, "acc", torch.int64)
    out = torch.empty(8, dtype=torch.float64, device=acc.device)
    st = L.spec_verify_telemetry_summary(_ptr(acc), _ptr(out), _stream(stream))
    if st != SV_OK:
        raise SpecVerifyError(st, "spec_verify_telemetry_summary")
    return out


def telemetry_fields(acc):
    """Name the words of a block (host copy; no arithmetic)."""
    words = acc.cpu().tolist()
    out = dict(zip(TELEMETRY_FIELDS, words[:len(TELEMETRY_FIELDS)]))
    i = len(TELEMETRY_FIELDS)
    for name, n in TELEMETRY_BINS:
        out[name] = words[i:i + n]
        i += n
    return out


def profile_next(begin_event, end_event, ensure_created=True):
    """Have the next linear/tree call record two torch.cuda.Events around its vocabulary pass.

    The events must exist as HIP events; with ensure_created they are recorded
    once here first (do that outside any graph capture).
    """
    if ensure_created:
        begin_event.record()
        end_event.record()
    library().spec_verify_profile_next(ctypes.c_void_p(begin_event.cuda_event),
                                       ctypes.c_void_p(end_event.cuda_event))


def exp2_hw(x, stream=None):
    """The hardware 2^x the verify kernels use, elementwise over a float32 device tensor."""
    L = library()
    _dev(x, "x", torch.float32)
    y = torch.empty_like(x)
    st = L.spec_verify_exp2(_ptr(x), _ptr(y), int(x.numel()), _stream(stream))
    if st != SV_OK:
        raise SpecVerifyError(st, "spec_verify_exp2")
    return y


def philox_words(seed, step, n_rows, n_slots, row_ids=None, stream=None):
    """Raw Philox words [n_rows, n_slots, 4] (uint32 stored in int32)."""
    L = library()
    dev = torch.device("cuda", torch.cuda.current_device())
    if row_ids is not None:
        _dev(row_ids, "row_ids", torch.int32)
    out = torch.empty((n_rows, n_slots, 4), dtype=torch.int32, device=dev)
    st = L.spec_verify_philox_words(int(seed), int(step), _ptr(row_ids), n_rows, n_slots,
                                    _ptr(out), _stream(stream))
    if st != SV_OK:
        raise SpecVerifyError(st, "spec_verify_philox_words")
    return out
