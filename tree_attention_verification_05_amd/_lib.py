"""ctypes binding of libtv.so: the calls include/tv.h declares, argument marshalling only.

Every function takes torch tensors that live on an AMD GPU, checks dtype,
shape, contiguity and device, and passes raw device pointers plus the current
HIP stream of that device to the library.  All computation happens in the
library's kernels; there is no fallback of any kind: if libtv.so is missing
or a tensor is on the CPU, the call raises.
"""
from __future__ import annotations

import ctypes
import os
import re
from typing import Dict, Optional, Tuple

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libtv.so")
HEADER = os.path.join(os.path.dirname(_HERE), "include", "tv.h")

TV_OK = 0
TV_ERR_TOO_LARGE = 8
TV_ACCEPT_NOALLOC_SCRATCH_BYTES = 4 << 20
TV_F32, TV_BF16 = 0, 1
TV_KV_TOKEN_MAJOR = 0x100  # dtype flag: caches [num_blocks, 16, Hkv, D] instead of [num_blocks, Hkv, 16, D]
TV_DEV_BAD_TREE, TV_DEV_BAD_CACHE, TV_DEV_BAD_TOKEN = 1, 2, 4
TV_DEV_BAD_RANDOM, TV_DEV_UNSUPPORTED = 8, 16
TV_MAX_NODES = 256
BLOCK_SIZE = 16

_c_i32 = ctypes.c_int32
_c_ptr = ctypes.c_void_p
_c_size = ctypes.c_size_t


class TVError(RuntimeError):
    """A libtv call returned a status other than TV_OK."""

    def __init__(self, fn: str, status: int, text: str):
        super().__init__(f"{fn}: {text} (status {status})")
        self.status = status


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python -m tree_attention_verification_05_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    sig = {
        "tv_status_string": (ctypes.c_char_p, [_c_i32]),
        "tv_version": (ctypes.c_int, []),
        "tv_build_tree_mask": (_c_i32, [_c_ptr, _c_i32, _c_i32, _c_ptr, _c_ptr, _c_ptr, _c_ptr]),
        "tv_tree_attention_workspace_size": (_c_size, [_c_i32] * 6),
        "tv_tree_attention": (_c_i32, [_c_ptr, _c_ptr, _c_ptr, _c_i32, _c_ptr, _c_i32, _c_i32,
                                       _c_ptr, _c_i32, _c_ptr, _c_ptr, _c_i32, _c_i32, _c_i32,
                                       _c_i32, _c_i32, ctypes.c_float, _c_i32, _c_ptr, _c_size,
                                       _c_ptr, _c_ptr]),
        "tv_tree_attention_parents": (_c_i32, [_c_ptr, _c_ptr, _c_ptr, _c_i32, _c_ptr, _c_i32, _c_i32,
                                               _c_ptr, _c_i32, _c_ptr, _c_ptr, _c_i32, _c_i32, _c_i32,
                                               _c_i32, _c_i32, ctypes.c_float, _c_i32, _c_ptr, _c_size,
                                               _c_ptr, _c_ptr]),
        "tv_accept_greedy_workspace_size": (_c_size, [_c_i32] * 3),
        "tv_accept_greedy_compact": (_c_i32, [_c_ptr, _c_ptr, _c_ptr, _c_i32, _c_i32, _c_i32, _c_ptr, _c_ptr,
                                              _c_ptr, _c_ptr, _c_ptr, _c_size, _c_ptr, _c_ptr, _c_i32, _c_ptr,
                                              _c_i32, _c_i32, _c_ptr, _c_i32, _c_i32, _c_i32, _c_ptr, _c_ptr,
                                              _c_ptr]),
        "tv_accept_greedy": (_c_i32, [_c_ptr, _c_ptr, _c_ptr, _c_i32, _c_i32, _c_i32, _c_ptr,
                                      _c_ptr, _c_ptr, _c_ptr, _c_ptr, _c_size, _c_ptr, _c_ptr]),
        "tv_accept_greedy_noalloc": (_c_i32, [_c_ptr, _c_ptr, _c_ptr, _c_i32, _c_i32, _c_i32, _c_ptr,
                                              _c_ptr, _c_ptr, _c_ptr, _c_ptr, _c_ptr]),
        "tv_accept_stochastic_workspace_size": (_c_size, [_c_i32] * 3),
        "tv_accept_stochastic": (_c_i32, [_c_ptr, _c_ptr, _c_ptr, _c_ptr, _c_ptr, _c_ptr, _c_i32,
                                          _c_i32, _c_i32, ctypes.c_float, _c_ptr, _c_ptr, _c_ptr,
                                          _c_ptr, _c_size, _c_ptr, _c_ptr]),
        "tv_lm_head_argmax_workspace_size": (_c_size, [_c_i32] * 3),
        "tv_lm_head_argmax": (_c_i32, [_c_ptr, _c_ptr, _c_i32, _c_i32, _c_i32, _c_i32, _c_ptr, _c_ptr,
                                       _c_ptr, _c_size, _c_ptr]),
        "tv_build_draft_tree_workspace_size": (_c_size, [_c_i32] * 4),
        "tv_build_draft_tree": (_c_i32, [_c_ptr, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_ptr, _c_ptr,
                                         _c_ptr, _c_ptr, _c_ptr, _c_size, _c_ptr]),
        "tv_kv_compact": (_c_i32, [_c_ptr, _c_ptr, _c_i32, _c_ptr, _c_i32, _c_i32, _c_ptr, _c_ptr,
                                   _c_ptr, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_ptr, _c_ptr,
                                   _c_ptr]),
        "tv_tree_kv_write": (_c_i32, [_c_ptr, _c_ptr, _c_ptr, _c_ptr, _c_ptr, _c_ptr, _c_ptr, _c_i32,
                                      _c_ptr, _c_i32, _c_i32, _c_ptr, _c_i32, _c_i32, _c_i32, _c_i32,
                                      _c_i32, ctypes.c_float, _c_i32, _c_ptr, _c_ptr]),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    return lib


lib = _load()


def header_functions() -> list:
    """Names of the functions tv.h declares."""
    with open(HEADER) as f:
        text = f.read()
    return sorted(set(re.findall(r"TV_API\s+[\w\s\*]*?\b(tv_\w+)\s*\(", text)))


# ------------------------------------------------------------------ helpers

def _check(fn: str, st: int) -> None:
    if st != TV_OK:
        raise TVError(fn, st, lib.tv_status_string(st).decode())


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _dev(t: torch.Tensor, name: str, dtype=None, shape=None) -> torch.Tensor:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on the GPU (got {t.device})")
    if dtype is not None and t.dtype not in (dtype if isinstance(dtype, tuple) else (dtype,)):
        raise TypeError(f"{name}: dtype {t.dtype} not allowed")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)} != {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _stream(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


def _tv_dtype(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return TV_BF16
    if t.dtype == torch.float32:
        return TV_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


_cached_ws: Dict[Tuple[int, int, int], torch.Tensor] = {}


def cached_workspace(device: torch.device, nbytes: int, kind: int = 0) -> torch.Tensor:
    """A workspace for tv_accept_greedy (kind 0), tv_accept_stochastic
    (kind 1), tv_lm_head_argmax (kind 2), tv_build_draft_tree (kind 3) or
    tv_tree_attention (kind 4), kept per device, current stream and kind, and
    grown when a call needs more.  A new buffer is zero-filled: the attention
    workspace's arrival counters must start at zero (each call leaves them
    so); the other calls need no initial contents.

    One buffer per stream: calls on one stream run in order, so they may
    share it; calls on different streams get different buffers, and a buffer
    is only ever used on the stream that allocated it, which is the stream the
    caching allocator orders its reuse against when a grown buffer replaces
    it.  Callers that pass their own workspace to calls running concurrently
    on several streams must pass one per stream."""
    idx = device.index if device.index is not None else torch.cuda.current_device()
    key = (idx, torch.cuda.current_stream(idx).cuda_stream, kind)
    ws = _cached_ws.get(key)
    if ws is None or ws.numel() < nbytes:
        ws = torch.zeros(max(nbytes, 4096), dtype=torch.uint8, device=device)
        _cached_ws[key] = ws
    return ws


# ------------------------------------------------------------------ calls

def tv_build_tree_mask(parents: torch.Tensor, mask: Optional[torch.Tensor] = None,
                       depth: Optional[torch.Tensor] = None,
                       dev_status: Optional[torch.Tensor] = None):
    """parents int32 [B, N] -> (mask int64 [B, N, W] holding the uint64 words,
    depth int32 [B, N])."""
    _dev(parents, "parents", torch.int32)
    B, N = parents.shape
    W = (N + 63) // 64
    if mask is None:
        mask = torch.empty((B, N, W), dtype=torch.int64, device=parents.device)
    _dev(mask, "mask", (torch.int64, torch.uint64), (B, N, W))
    if depth is None:
        depth = torch.empty((B, N), dtype=torch.int32, device=parents.device)
    _dev(depth, "depth", torch.int32, (B, N))
    if dev_status is not None:
        _dev(dev_status, "dev_status", torch.int32)
    _check("tv_build_tree_mask", lib.tv_build_tree_mask(
        _ptr(parents), B, N, _ptr(mask), _ptr(depth), _ptr(dev_status), _stream(parents)))
    return mask, depth


def tv_tree_attention_workspace_size(B, N, Hq, Hkv, D, max_prefix_len) -> int:
    return int(lib.tv_tree_attention_workspace_size(B, N, Hq, Hkv, D, max_prefix_len))


def _cache_dims(k_cache: torch.Tensor, token_major: bool):
    """(num_blocks, Hkv, block_size, D) of a cache in either layout."""
    if k_cache.dim() != 4:
        raise ValueError("caches must be 4-d")
    if token_major:
        nb, bs, Hkv, D = k_cache.shape  # [num_blocks, block_size, Hkv, D]
    else:
        nb, Hkv, bs, D = k_cache.shape  # [num_blocks, Hkv, block_size, D]
    return nb, Hkv, bs, D


def tv_tree_attention(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                      block_table: torch.Tensor, prefix_lens: torch.Tensor, max_prefix_len: int,
                      mask: torch.Tensor, out: Optional[torch.Tensor] = None, scale: float = 0.0,
                      workspace: Optional[torch.Tensor] = None,
                      dev_status: Optional[torch.Tensor] = None,
                      token_major: bool = False) -> torch.Tensor:
    """q [B, N, Hq, D]; caches [num_blocks, Hkv, 16, D] (token_major:
    [num_blocks, 16, Hkv, D]; bf16 or fp32, same as q); block_table int32
    [B, max_blocks]; prefix_lens int32 [B]; mask from tv_build_tree_mask.
    Returns out [B, N, Hq, D] in q's dtype."""
    return _tree_attention(q, k_cache, v_cache, block_table, prefix_lens, max_prefix_len, mask, None, out,
                           scale, workspace, dev_status, token_major)


def tv_tree_attention_parents(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                              block_table: torch.Tensor, prefix_lens: torch.Tensor, max_prefix_len: int,
                              parents: torch.Tensor, out: Optional[torch.Tensor] = None, scale: float = 0.0,
                              workspace: Optional[torch.Tensor] = None,
                              dev_status: Optional[torch.Tensor] = None,
                              token_major: bool = False) -> torch.Tensor:
    """tv_tree_attention with the tree's parents (int32 [B, N], N <= 64) in
    place of the masks, which the attention kernels build themselves."""
    return _tree_attention(q, k_cache, v_cache, block_table, prefix_lens, max_prefix_len, None, parents, out,
                           scale, workspace, dev_status, token_major)


def _tree_attention(q, k_cache, v_cache, block_table, prefix_lens, max_prefix_len, mask, parents, out, scale,
                    workspace, dev_status, token_major):
    dt = _tv_dtype(q)
    _dev(q, "q", q.dtype)
    B, N, Hq, D = q.shape
    nb, Hkv, bs, _ = _cache_dims(k_cache, token_major)
    _dev(k_cache, "k_cache", q.dtype, k_cache.shape)
    _dev(v_cache, "v_cache", q.dtype, k_cache.shape)
    if k_cache.shape[3] != D:
        raise ValueError("cache rows must have q's head dim")
    _dev(block_table, "block_table", torch.int32)
    if block_table.dim() != 2 or block_table.shape[0] != B:
        raise ValueError("block_table must be [B, max_blocks]")
    _dev(prefix_lens, "prefix_lens", torch.int32, (B,))
    if mask is not None:
        _dev(mask, "mask", (torch.int64, torch.uint64), (B, N, (N + 63) // 64))
    else:
        _dev(parents, "parents", torch.int32, (B, N))
    if out is None:
        out = torch.empty_like(q)
    _dev(out, "out", q.dtype, q.shape)
    need = tv_tree_attention_workspace_size(B, N, Hq, Hkv, D, max_prefix_len) if dt == TV_BF16 else 0
    if need and (workspace is None or workspace.numel() * workspace.element_size() < need):
        workspace = cached_workspace(q.device, need, kind=4)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if dev_status is not None:
        _dev(dev_status, "dev_status", torch.int32)
    name = "tv_tree_attention" if mask is not None else "tv_tree_attention_parents"
    _check(name, getattr(lib, name)(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), nb, _ptr(block_table), block_table.shape[1], bs,
        _ptr(prefix_lens), int(max_prefix_len), _ptr(mask if mask is not None else parents), _ptr(out), B, N, Hq,
        Hkv, D, float(scale), dt | (TV_KV_TOKEN_MAJOR if token_major else 0), _ptr(workspace), ws_bytes,
        _ptr(dev_status), _stream(q)))
    return out


def _accept_outputs(logits, draft_tokens, parents, accept_len, accepted_nodes, bonus_token, target_argmax,
                    want_argmax):
    """Checks of the greedy acceptance inputs; the outputs, allocated when
    not given."""
    _dev(logits, "logits", torch.float32)
    B, N, V = logits.shape
    _dev(draft_tokens, "draft_tokens", torch.int32, (B, N))
    _dev(parents, "parents", torch.int32, (B, N))
    dev = logits.device
    if accept_len is None:
        accept_len = torch.empty(B, dtype=torch.int32, device=dev)
    if accepted_nodes is None:
        accepted_nodes = torch.empty((B, N), dtype=torch.int32, device=dev)
    if bonus_token is None:
        bonus_token = torch.empty(B, dtype=torch.int32, device=dev)
    if target_argmax is None and want_argmax:
        target_argmax = torch.empty((B, N), dtype=torch.int32, device=dev)
    _dev(accept_len, "accept_len", torch.int32, (B,))
    _dev(accepted_nodes, "accepted_nodes", torch.int32, (B, N))
    _dev(bonus_token, "bonus_token", torch.int32, (B,))
    if target_argmax is not None:
        _dev(target_argmax, "target_argmax", torch.int32, (B, N))
    return B, N, V, accept_len, accepted_nodes, bonus_token, target_argmax


def tv_accept_greedy(logits: torch.Tensor, draft_tokens: torch.Tensor, parents: torch.Tensor,
                     accept_len: Optional[torch.Tensor] = None,
                     accepted_nodes: Optional[torch.Tensor] = None,
                     bonus_token: Optional[torch.Tensor] = None,
                     target_argmax: Optional[torch.Tensor] = None, want_argmax: bool = True,
                     workspace: Optional[torch.Tensor] = None,
                     dev_status: Optional[torch.Tensor] = None):
    """logits fp32 [B, N, V]; draft_tokens, parents int32 [B, N].  Returns
    (accept_len [B], accepted_nodes [B, N], bonus_token [B], target_argmax
    [B, N] or None), all int32."""
    B, N, V, accept_len, accepted_nodes, bonus_token, target_argmax = _accept_outputs(
        logits, draft_tokens, parents, accept_len, accepted_nodes, bonus_token, target_argmax, want_argmax)
    dev = logits.device
    need = int(lib.tv_accept_greedy_workspace_size(B, N, V))
    if workspace is None:
        workspace = cached_workspace(dev, need)
    if dev_status is not None:
        _dev(dev_status, "dev_status", torch.int32)
    _check("tv_accept_greedy", lib.tv_accept_greedy(
        _ptr(logits), _ptr(draft_tokens), _ptr(parents), B, N, V, _ptr(accept_len),
        _ptr(accepted_nodes), _ptr(bonus_token), _ptr(target_argmax), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _ptr(dev_status), _stream(logits)))
    return accept_len, accepted_nodes, bonus_token, target_argmax


def tv_accept_greedy_noalloc(logits: torch.Tensor, draft_tokens: torch.Tensor, parents: torch.Tensor,
                             accept_len: torch.Tensor, accepted_nodes: torch.Tensor,
                             bonus_token: torch.Tensor, target_argmax: Optional[torch.Tensor] = None,
                             dev_status: Optional[torch.Tensor] = None) -> None:
    """tv_accept_greedy without a workspace (the library's static scratch
    serves instead) and without allocating: every output is the caller's.
    logits fp32 [B, N, V]; draft_tokens, parents, accepted_nodes (and
    target_argmax, if given) int32 [B, N]; accept_len, bonus_token int32 [B]."""
    _dev(logits, "logits", torch.float32)
    B, N, V = logits.shape
    _dev(draft_tokens, "draft_tokens", torch.int32, (B, N))
    _dev(parents, "parents", torch.int32, (B, N))
    _dev(accept_len, "accept_len", torch.int32, (B,))
    _dev(accepted_nodes, "accepted_nodes", torch.int32, (B, N))
    _dev(bonus_token, "bonus_token", torch.int32, (B,))
    if target_argmax is not None:
        _dev(target_argmax, "target_argmax", torch.int32, (B, N))
    if dev_status is not None:
        _dev(dev_status, "dev_status", torch.int32)
    _check("tv_accept_greedy_noalloc", lib.tv_accept_greedy_noalloc(
        _ptr(logits), _ptr(draft_tokens), _ptr(parents), B, N, V, _ptr(accept_len),
        _ptr(accepted_nodes), _ptr(bonus_token), _ptr(target_argmax), _ptr(dev_status), _stream(logits)))


def tv_accept_stochastic(logits: torch.Tensor, draft_tokens: torch.Tensor, parents: torch.Tensor,
                         temperature: float, uniforms: torch.Tensor, exponentials: torch.Tensor,
                         draft_probs: Optional[torch.Tensor] = None,
                         accept_len: Optional[torch.Tensor] = None,
                         accepted_nodes: Optional[torch.Tensor] = None,
                         bonus_token: Optional[torch.Tensor] = None,
                         workspace: Optional[torch.Tensor] = None,
                         dev_status: Optional[torch.Tensor] = None):
    """logits fp32 [B, N, V]; draft_tokens, parents int32 [B, N]; uniforms fp32
    [B, N]; exponentials fp32 [B, V]; draft_probs fp32 [B, N, V] or None
    (point-mass proposals).  Returns (accept_len [B], accepted_nodes [B, N],
    bonus_token [B]), all int32."""
    _dev(logits, "logits", torch.float32)
    B, N, V = logits.shape
    _dev(draft_tokens, "draft_tokens", torch.int32, (B, N))
    _dev(parents, "parents", torch.int32, (B, N))
    _dev(uniforms, "uniforms", torch.float32, (B, N))
    _dev(exponentials, "exponentials", torch.float32, (B, V))
    if draft_probs is not None:
        _dev(draft_probs, "draft_probs", torch.float32, (B, N, V))
    dev = logits.device
    if accept_len is None:
        accept_len = torch.empty(B, dtype=torch.int32, device=dev)
    if accepted_nodes is None:
        accepted_nodes = torch.empty((B, N), dtype=torch.int32, device=dev)
    if bonus_token is None:
        bonus_token = torch.empty(B, dtype=torch.int32, device=dev)
    _dev(accept_len, "accept_len", torch.int32, (B,))
    _dev(accepted_nodes, "accepted_nodes", torch.int32, (B, N))
    _dev(bonus_token, "bonus_token", torch.int32, (B,))
    need = int(lib.tv_accept_stochastic_workspace_size(B, N, V))
    if workspace is None:
        workspace = cached_workspace(dev, need, kind=1)
    if dev_status is not None:
        _dev(dev_status, "dev_status", torch.int32)
    _check("tv_accept_stochastic", lib.tv_accept_stochastic(
        _ptr(logits), _ptr(draft_probs), _ptr(draft_tokens), _ptr(parents), _ptr(uniforms),
        _ptr(exponentials), B, N, V, float(temperature), _ptr(accept_len), _ptr(accepted_nodes),
        _ptr(bonus_token), _ptr(workspace), workspace.numel() * workspace.element_size(),
        _ptr(dev_status), _stream(logits)))
    return accept_len, accepted_nodes, bonus_token


def tv_lm_head_argmax(hidden: torch.Tensor, weight: torch.Tensor,
                      argmax: Optional[torch.Tensor] = None,
                      max_score: Optional[torch.Tensor] = None, want_max: bool = True,
                      workspace: Optional[torch.Tensor] = None):
    """hidden bf16 [..., H] (rows = all leading dims), weight bf16 [V, H].
    Returns (argmax int32 [...], max_score fp32 [...] or None)."""
    _dev(hidden, "hidden", torch.bfloat16)
    _dev(weight, "weight", torch.bfloat16)
    H = hidden.shape[-1]
    V = weight.shape[0]
    if weight.dim() != 2 or weight.shape[1] != H:
        raise ValueError("weight must be [V, H] with the hidden width of `hidden`")
    lead = tuple(hidden.shape[:-1])
    M = 1
    for d in lead:
        M *= int(d)
    dev = hidden.device
    if argmax is None:
        argmax = torch.empty(lead, dtype=torch.int32, device=dev)
    if max_score is None and want_max:
        max_score = torch.empty(lead, dtype=torch.float32, device=dev)
    _dev(argmax, "argmax", torch.int32, lead)
    if max_score is not None:
        _dev(max_score, "max_score", torch.float32, lead)
    need = int(lib.tv_lm_head_argmax_workspace_size(M, H, V))
    if workspace is None:
        workspace = cached_workspace(dev, need, kind=2)
    _check("tv_lm_head_argmax", lib.tv_lm_head_argmax(
        _ptr(hidden), _ptr(weight), M, H, V, TV_BF16, _ptr(argmax), _ptr(max_score), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(hidden)))
    return argmax, max_score


def tv_build_draft_tree(draft_logits: torch.Tensor, N: int,
                        root_tokens: Optional[torch.Tensor] = None,
                        parents: Optional[torch.Tensor] = None,
                        tokens: Optional[torch.Tensor] = None,
                        scores: Optional[torch.Tensor] = None, want_scores: bool = True,
                        workspace: Optional[torch.Tensor] = None):
    """draft_logits fp32 [B, depth, topk, V] (row (l, j): the drafter's scores
    at the j-th best node of level l - 1; row (0, 0) at the root).
    Returns (parents int32 [B, N], tokens int32 [B, N], scores fp32 [B, N] or None)."""
    _dev(draft_logits, "draft_logits", torch.float32)
    if draft_logits.dim() != 4:
        raise ValueError("draft_logits must be [B, depth, topk, V]")
    B, depth, topk, V = (int(x) for x in draft_logits.shape)
    dev = draft_logits.device
    if root_tokens is not None:
        _dev(root_tokens, "root_tokens", torch.int32, (B,))
    if parents is None:
        parents = torch.empty((B, N), dtype=torch.int32, device=dev)
    if tokens is None:
        tokens = torch.empty((B, N), dtype=torch.int32, device=dev)
    if scores is None and want_scores:
        scores = torch.empty((B, N), dtype=torch.float32, device=dev)
    _dev(parents, "parents", torch.int32, (B, N))
    _dev(tokens, "tokens", torch.int32, (B, N))
    if scores is not None:
        _dev(scores, "scores", torch.float32, (B, N))
    need = int(lib.tv_build_draft_tree_workspace_size(B, depth, topk, V))
    if workspace is None:
        workspace = cached_workspace(dev, need, kind=3)
    _check("tv_build_draft_tree", lib.tv_build_draft_tree(
        _ptr(draft_logits), B, depth, topk, V, N, _ptr(root_tokens), _ptr(parents), _ptr(tokens),
        _ptr(scores), _ptr(workspace), workspace.numel() * workspace.element_size(),
        _stream(draft_logits)))
    return parents, tokens, scores


def tv_kv_compact(k_cache: torch.Tensor, v_cache: torch.Tensor, block_table: torch.Tensor,
                  prefix_lens: torch.Tensor, accepted_nodes: torch.Tensor,
                  accept_len: torch.Tensor, new_lens: Optional[torch.Tensor] = None,
                  dev_status: Optional[torch.Tensor] = None, token_major: bool = False) -> torch.Tensor:
    """Compacts the accepted path's K/V in place (caches [num_blocks, Hkv, 16,
    D], or [num_blocks, 16, Hkv, D] with token_major); returns new_lens int32
    [B]."""
    dt = _tv_dtype(k_cache)
    nb, Hkv, bs, D = _cache_dims(k_cache, token_major)
    _dev(k_cache, "k_cache", k_cache.dtype)
    _dev(v_cache, "v_cache", k_cache.dtype, k_cache.shape)
    _dev(accepted_nodes, "accepted_nodes", torch.int32)
    B, N = accepted_nodes.shape
    _dev(block_table, "block_table", torch.int32)
    if block_table.dim() != 2 or block_table.shape[0] != B:
        raise ValueError("block_table must be [B, max_blocks]")
    _dev(prefix_lens, "prefix_lens", torch.int32, (B,))
    _dev(accept_len, "accept_len", torch.int32, (B,))
    if new_lens is None:
        new_lens = torch.empty(B, dtype=torch.int32, device=k_cache.device)
    _dev(new_lens, "new_lens", torch.int32, (B,))
    if dev_status is not None:
        _dev(dev_status, "dev_status", torch.int32)
    _check("tv_kv_compact", lib.tv_kv_compact(
        _ptr(k_cache), _ptr(v_cache), nb, _ptr(block_table), block_table.shape[1], bs,
        _ptr(prefix_lens), _ptr(accepted_nodes), _ptr(accept_len), B, N, Hkv, D,
        dt | (TV_KV_TOKEN_MAJOR if token_major else 0), _ptr(new_lens), _ptr(dev_status), _stream(k_cache)))
    return new_lens


def tv_accept_greedy_compact(logits: torch.Tensor, draft_tokens: torch.Tensor, parents: torch.Tensor,
                             k_cache: torch.Tensor, v_cache: torch.Tensor, block_table: torch.Tensor,
                             prefix_lens: torch.Tensor, accept_len: Optional[torch.Tensor] = None,
                             accepted_nodes: Optional[torch.Tensor] = None,
                             bonus_token: Optional[torch.Tensor] = None,
                             target_argmax: Optional[torch.Tensor] = None, want_argmax: bool = True,
                             new_lens: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                             dev_status: Optional[torch.Tensor] = None, token_major: bool = False):
    """tv_accept_greedy, then tv_kv_compact of the accepted paths, in one
    call.  Returns (accept_len, accepted_nodes, bonus_token, target_argmax or
    None, new_lens)."""
    B, N, V, accept_len, accepted_nodes, bonus_token, target_argmax = _accept_outputs(
        logits, draft_tokens, parents, accept_len, accepted_nodes, bonus_token, target_argmax, want_argmax)
    dev = logits.device
    dt = _tv_dtype(k_cache)
    nb, Hkv, bs, D = _cache_dims(k_cache, token_major)
    _dev(k_cache, "k_cache", k_cache.dtype)
    _dev(v_cache, "v_cache", k_cache.dtype, k_cache.shape)
    _dev(block_table, "block_table", torch.int32)
    if block_table.dim() != 2 or block_table.shape[0] != B:
        raise ValueError("block_table must be [B, max_blocks]")
    _dev(prefix_lens, "prefix_lens", torch.int32, (B,))
    if new_lens is None:
        new_lens = torch.empty(B, dtype=torch.int32, device=dev)
    _dev(new_lens, "new_lens", torch.int32, (B,))
    need = int(lib.tv_accept_greedy_workspace_size(B, N, V))
    if workspace is None:
        workspace = cached_workspace(dev, need)
    if dev_status is not None:
        _dev(dev_status, "dev_status", torch.int32)
    _check("tv_accept_greedy_compact", lib.tv_accept_greedy_compact(
        _ptr(logits), _ptr(draft_tokens), _ptr(parents), B, N, V, _ptr(accept_len), _ptr(accepted_nodes),
        _ptr(bonus_token), _ptr(target_argmax), _ptr(workspace), workspace.numel() * workspace.element_size(),
        _ptr(k_cache), _ptr(v_cache), nb, _ptr(block_table), block_table.shape[1], bs, _ptr(prefix_lens), Hkv, D,
        dt | (TV_KV_TOKEN_MAJOR if token_major else 0), _ptr(new_lens), _ptr(dev_status), _stream(logits)))
    return accept_len, accepted_nodes, bonus_token, target_argmax, new_lens


def tv_tree_kv_write(q: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor, depth: torch.Tensor,
                     k_cache: torch.Tensor, v_cache: torch.Tensor, block_table: torch.Tensor,
                     prefix_lens: torch.Tensor, rope_theta: float, q_out: Optional[torch.Tensor] = None,
                     dev_status: Optional[torch.Tensor] = None, token_major: bool = False) -> torch.Tensor:
    """q [B, N, Hq, D]; k_new, v_new [B, N, Hkv, D]; depth int32 [B, N] (from
    tv_build_tree_mask); caches [num_blocks, Hkv, 16, D] (token_major:
    [num_blocks, 16, Hkv, D]) updated in place at positions P_b + i.  Returns
    the rotated queries (q_out, may be q)."""
    dt = _tv_dtype(q)
    _dev(q, "q", q.dtype)
    B, N, Hq, D = q.shape
    nb, Hkv, bs, D2 = _cache_dims(k_cache, token_major)
    _dev(k_new, "k_new", q.dtype, (B, N, Hkv, D))
    _dev(v_new, "v_new", q.dtype, (B, N, Hkv, D))
    _dev(depth, "depth", torch.int32, (B, N))
    _dev(k_cache, "k_cache", q.dtype, k_cache.shape)
    _dev(v_cache, "v_cache", q.dtype, k_cache.shape)
    if D2 != D:
        raise ValueError("cache rows must have q's head dim")
    _dev(block_table, "block_table", torch.int32)
    if block_table.dim() != 2 or block_table.shape[0] != B:
        raise ValueError("block_table must be [B, max_blocks]")
    _dev(prefix_lens, "prefix_lens", torch.int32, (B,))
    if q_out is None:
        q_out = torch.empty_like(q)
    _dev(q_out, "q_out", q.dtype, q.shape)
    if dev_status is not None:
        _dev(dev_status, "dev_status", torch.int32)
    _check("tv_tree_kv_write", lib.tv_tree_kv_write(
        _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(depth), _ptr(q_out), _ptr(k_cache), _ptr(v_cache), nb,
        _ptr(block_table), block_table.shape[1], bs, _ptr(prefix_lens), B, N, Hq, Hkv, D,
        float(rope_theta), dt | (TV_KV_TOKEN_MAJOR if token_major else 0), _ptr(dev_status), _stream(q)))
    return q_out
