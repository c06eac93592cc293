"""Seeded synthetic inputs for single-pass verification of a draft token tree.

This module draws inputs only.  It holds none of the verification arithmetic
(no attention, no argmax over target scores, no acceptance walk, no cache
compaction); both the CPU oracle's tests and the GPU path's tests, benchmark
and smoke check take their inputs from here.

What the inputs stand for (all synthetic; no model, weight or data set is
read):

* A draft token tree per sequence: a parent-index array with node 0 the root
  (the last verified token, parent -1) and ``parent[i] < i`` for every other
  node, plus one draft token id per node.  The tree shapes follow the pages'
  draft families: random trees, EAGLE-2 style dynamic trees built by top-k
  expansion and global rerank of cumulative draft scores ("EAGLE代码实现原理",
  section 树结构缓冲: branch prediction, level pruning), depth-biased trees, and
  the P-EAGLE linear chain ("P-EAGLE：vLLM集成并行推测解码加速LLM推理",
  section 技术原理和实现方式).
* A paged K/V cache ``[num_blocks, Hkv, block_size, D]`` (within a block, the
  slots of one KV head after another) with one block table row per sequence
  ("vLLM-TreeEagle" README, architecture graph: PagedAttention under the
  tree-attention layer).  Prefix position ``t`` of sequence ``b`` lives in
  block ``block_table[b, t // block_size]`` at slot ``t % block_size``; tree
  node ``i`` sits at position ``prefix_len[b] + i``.
* Query rows ``[B, N, Hq, D]`` for every tree node.
* Target logits ``[B, N, V]`` in fp32, with the draft token of some children
  planted as the unique maximum of their parent's row so that a controlled
  share of drafts matches the target ("P-EAGLE" page, section 技术原理和实现方式:
  the target scores every proposed token in one pass; acceptance guidance of
  60-80% in its best-practice section).

Randomness: every component of every configuration has its own numpy
``default_rng`` stream keyed by ``(seed, config_tag, component[, chunk])``, so
skipping or resizing one component never changes another.  Large dense
tensors are drawn in fixed-size chunks, each with its own stream, so values do
not depend on the number of threads used to draw them.
"""
from __future__ import annotations

import dataclasses
from concurrent.futures import ThreadPoolExecutor
from typing import Optional, Sequence, Tuple, Union

import numpy as np
import torch

BLOCK_SIZE = 16
_CHUNK = 1 << 22  # elements per independently seeded chunk of a dense tensor

# component tags of the random streams
_C_PREFIX, _C_TREE, _C_MATCH, _C_BLOCKS, _C_Q, _C_K, _C_V, _C_LOGITS, _C_PLANT = range(1, 10)
_C_KNEW, _C_VNEW = 10, 11
_C_UNIF, _C_EXPO, _C_QNOISE, _C_QDRAW = 12, 13, 14, 15
_C_HID, _C_WLM = 16, 17
_C_DLOGITS, _C_DROOT = 18, 19

# Sampling temperature of the stochastic-verification inputs: the top of the
# 0.0-0.7 range that the P-EAGLE page's practical notes recommend for speedup.
SAMPLING_TEMPERATURE = 0.7

# Rotary base of the model family each workload is shaped after: Qwen2
# 1000000; the Llama-3-shaped layers (8B, the batched 32/8-head layer, the
# 70B share) 500000; the tiny case the classic 10000.
def rope_theta(spec) -> float:
    if "qwen2" in spec.name:
        return 1000000.0
    if "tiny" in spec.name:
        return 10000.0
    return 500000.0


def hidden_size(spec) -> int:
    """Width of the final hidden state that the target's LM head projects
    (Llama-3-8B 4096, Qwen2-7B 3584, Llama-3-70B 8192; 256 for the tiny case)."""
    if "tiny" in spec.name:
        return 256
    if "qwen2" in spec.name:
        return 3584
    if "70b" in spec.name or "chain" in spec.name:
        return 8192
    return 4096


@dataclasses.dataclass(frozen=True)
class Spec:
    """Shape and distribution of one synthetic verification workload."""

    name: str
    tag: int                      # distinguishes random streams of different specs
    B: int
    Hq: int
    Hkv: int
    D: int
    V: int
    dtype: str                    # "f32" or "bf16": element type of q and the K/V cache
    prefix: Union[int, Tuple[int, int]]   # fixed length, or inclusive integer range per sequence
    tree: Tuple                   # ("uniform", N, depth) | ("eagle2", N, depth, topk)
                                  # | ("geometric", N, depth, p) | ("chain", N)
    logit_std: float
    match: Union[float, Tuple[float, float]]  # per-node plant probability, or a range per sequence
    block_size: int = BLOCK_SIZE
    prefix_lengths: Optional[Tuple[int, ...]] = None  # explicit per-sequence lengths (B of them);
                                                      # when given, ``prefix`` is not used

    @property
    def N(self) -> int:
        return int(self.tree[1])


@dataclasses.dataclass
class Workload:
    """One batch of verification inputs (host tensors)."""

    spec: Spec
    seed: int
    prefix_lens: np.ndarray       # int32 [B]
    parents: np.ndarray           # int32 [B, N]; parents[b, 0] == -1
    draft_tokens: np.ndarray      # int32 [B, N]; entry 0 (the root) is never compared
    block_table: np.ndarray       # int32 [B, max_blocks]; -1 in unused entries
    num_blocks: int
    planted: np.ndarray           # bool [B, N]: node i's token was planted as its parent row's max
    match_rate: np.ndarray        # float64 [B]
    q: Optional[torch.Tensor]     # [B, N, Hq, D] bf16 or f32
    k_cache: Optional[torch.Tensor]  # [num_blocks, Hkv, block_size, D]
    v_cache: Optional[torch.Tensor]
    logits: Optional[torch.Tensor]   # [B, N, V] f32

    @property
    def B(self) -> int:
        return self.spec.B

    @property
    def N(self) -> int:
        return self.spec.N

    @property
    def max_blocks(self) -> int:
        return int(self.block_table.shape[1])

    @property
    def max_prefix_len(self) -> int:
        return int(self.prefix_lens.max())


# --------------------------------------------------------------------------
# random streams
# --------------------------------------------------------------------------

def _rng(seed: int, tag: int, comp: int, *extra: int) -> np.random.Generator:
    return np.random.default_rng([seed, tag, comp, *extra])


def _normal(shape: Sequence[int], std: float, seed: int, tag: int, comp: int) -> np.ndarray:
    """N(0, std^2) float32 array drawn in fixed chunks, each its own stream."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.float32)
    nchunks = (n + _CHUNK - 1) // _CHUNK

    def fill(c: int) -> None:
        lo, hi = c * _CHUNK, min(n, (c + 1) * _CHUNK)
        _rng(seed, tag, comp, c).standard_normal(hi - lo, dtype=np.float32, out=out[lo:hi])

    if nchunks <= 1:
        for c in range(nchunks):
            fill(c)
    else:
        with ThreadPoolExecutor(max_workers=min(16, nchunks)) as ex:
            list(ex.map(fill, range(nchunks)))
    if std != 1.0:
        out *= np.float32(std)
    return out.reshape(shape)


def _to_dtype(a: np.ndarray, dtype: str) -> torch.Tensor:
    t = torch.from_numpy(a)
    if dtype == "bf16":
        return t.to(torch.bfloat16)          # round to nearest even
    if dtype == "f32":
        return t
    raise ValueError(dtype)


# --------------------------------------------------------------------------
# draft trees
# --------------------------------------------------------------------------

def _depths(parents: np.ndarray) -> np.ndarray:
    d = np.zeros(len(parents), dtype=np.int64)
    for i in range(1, len(parents)):
        d[i] = d[parents[i]] + 1
    return d


def _sibling_distinct_tokens(parents: np.ndarray, V: int, rng: np.random.Generator) -> np.ndarray:
    """One token per node; the children of any node carry distinct tokens."""
    N = len(parents)
    tok = np.zeros(N, dtype=np.int64)
    tok[0] = rng.integers(0, V)
    for p in range(N):
        kids = np.nonzero(parents == p)[0]
        if len(kids):
            tok[kids] = rng.choice(V, size=len(kids), replace=False)
    return tok


def tree_uniform(N: int, depth: int, V: int, rng: np.random.Generator, max_tries: int = 100000):
    """Each node's parent uniform among earlier nodes; resampled until the
    maximum depth (edges from the root) equals ``depth`` exactly."""
    for _ in range(max_tries):
        par = np.full(N, -1, dtype=np.int64)
        for i in range(1, N):
            par[i] = rng.integers(0, i)
        if N == 1 or _depths(par).max() == depth:
            return par, _sibling_distinct_tokens(par, V, rng)
    raise RuntimeError(f"no uniform tree with N={N} and depth {depth}")


def tree_chain(N: int, V: int, rng: np.random.Generator):
    par = np.arange(-1, N - 1, dtype=np.int64)
    return par, _sibling_distinct_tokens(par, V, rng)


def tree_geometric(N: int, depth: int, p: float, V: int, rng: np.random.Generator,
                   max_tries: int = 10000):
    """Depth-biased tree: node i's parent is the k-th ancestor of node i-1 with
    k ~ Geometric(p) counted from 0 (so a share p of nodes extends the previous
    node), clipped at the root, then moved up until its depth is below
    ``depth``.  Resampled until the maximum depth equals ``depth``."""
    for _ in range(max_tries):
        par = np.full(N, -1, dtype=np.int64)
        dep = np.zeros(N, dtype=np.int64)
        for i in range(1, N):
            a = i - 1
            k = int(rng.geometric(p)) - 1
            while k > 0 and a != 0:
                a = int(par[a])
                k -= 1
            while dep[a] >= depth:
                a = int(par[a])
            par[i] = a
            dep[i] = dep[a] + 1
        if N == 1 or dep.max() == depth:
            return par, _sibling_distinct_tokens(par, V, rng)
    raise RuntimeError(f"no geometric tree with N={N} and depth {depth}")


def tree_eagle2(N: int, depth: int, topk: int, V: int, rng: np.random.Generator):
    """EAGLE-2 style dynamic tree from synthetic draft scores.

    Level 1 expands the root; every later level expands the ``topk`` nodes of
    the previous level with the highest cumulative score.  Each expansion
    creates ``topk`` children with distinct uniform token ids and
    log-probabilities from a softmax over ``topk`` N(0,1) draft logits; a
    child's cumulative score is its parent's plus its own log-probability.
    The tree keeps the root and the ``N-1`` best generated nodes by cumulative
    score (ties: shallower first, then earlier generated), which is closed
    under ancestors because every log-probability is negative.  Nodes are
    relabelled by (depth, descending score)."""
    # generated node records: (score, depth, gen_id, parent_gen_id, token)
    score = [0.0]
    dep = [0]
    parent = [-1]
    token = [int(rng.integers(0, V))]
    prev_level = [0]
    for level in range(1, depth + 1):
        order = sorted(prev_level, key=lambda g: (-score[g], g))[:topk]
        cur = []
        for g in order:
            z = rng.standard_normal(topk)
            logp = z - (np.log(np.sum(np.exp(z - z.max()))) + z.max())
            toks = rng.choice(V, size=topk, replace=False)
            for c in range(topk):
                score.append(score[g] + float(logp[c]))
                dep.append(level)
                parent.append(g)
                token.append(int(toks[c]))
                cur.append(len(score) - 1)
        prev_level = cur
    gen = list(range(1, len(score)))
    keep = sorted(gen, key=lambda g: (-score[g], dep[g], g))[: N - 1]
    keep_set = set(keep)
    for g in keep:
        assert parent[g] == 0 or parent[g] in keep_set
    nodes = [0] + sorted(keep, key=lambda g: (dep[g], -score[g], g))
    new_id = {g: i for i, g in enumerate(nodes)}
    par = np.array([-1] + [new_id[parent[g]] for g in nodes[1:]], dtype=np.int64)
    tok = np.array([token[g] for g in nodes], dtype=np.int64)
    return par, tok


def make_tree(tree: Tuple, V: int, rng: np.random.Generator):
    kind = tree[0]
    if kind == "uniform":
        return tree_uniform(tree[1], tree[2], V, rng)
    if kind == "chain":
        return tree_chain(tree[1], V, rng)
    if kind == "geometric":
        return tree_geometric(tree[1], tree[2], tree[3], V, rng)
    if kind == "eagle2":
        return tree_eagle2(tree[1], tree[2], tree[3], V, rng)
    raise ValueError(kind)


# --------------------------------------------------------------------------
# full workloads
# --------------------------------------------------------------------------

def build(spec: Spec, seed: int = 0, dense: bool = True, logits: bool = True) -> Workload:
    """Draw one workload.  ``dense=False`` skips q and the K/V cache and
    ``logits=False`` skips the target logits (structure only)."""
    B, N, V = spec.B, spec.N, spec.V
    bs = spec.block_size

    r = _rng(seed, spec.tag, _C_PREFIX)
    if spec.prefix_lengths is not None:
        if len(spec.prefix_lengths) != B:
            raise ValueError("prefix_lengths needs one length per sequence")
        prefix_lens = np.asarray(spec.prefix_lengths, dtype=np.int32)
    elif isinstance(spec.prefix, tuple):
        lo, hi = spec.prefix
        prefix_lens = r.integers(lo, hi + 1, size=B).astype(np.int32)
    else:
        prefix_lens = np.full(B, int(spec.prefix), dtype=np.int32)

    parents = np.zeros((B, N), dtype=np.int32)
    draft = np.zeros((B, N), dtype=np.int32)
    for b in range(B):
        par, tok = make_tree(spec.tree, V, _rng(seed, spec.tag, _C_TREE, b))
        parents[b] = par
        draft[b] = tok

    r = _rng(seed, spec.tag, _C_MATCH)
    if isinstance(spec.match, tuple):
        match_rate = r.uniform(spec.match[0], spec.match[1], size=B)
    else:
        match_rate = np.full(B, float(spec.match))

    # which children get their token planted as the parent row's unique max
    planted = np.zeros((B, N), dtype=bool)
    r = _rng(seed, spec.tag, _C_PLANT)
    u = r.random((B, N))
    chain = spec.tree[0] == "chain"
    for b in range(B):
        has_planted_child = np.zeros(N, dtype=bool)
        for i in range(1, N):
            p = parents[b, i]
            if chain:
                ok = (i == 1 or planted[b, i - 1]) and u[b, i] < match_rate[b]
            else:
                ok = (not has_planted_child[p]) and u[b, i] < match_rate[b]
            if ok:
                planted[b, i] = True
                has_planted_child[p] = True

    # paged cache: one random permutation of physical block ids
    nblk = (prefix_lens.astype(np.int64) + N + bs - 1) // bs
    num_blocks = int(nblk.sum())
    perm = _rng(seed, spec.tag, _C_BLOCKS).permutation(num_blocks).astype(np.int32)
    max_blocks = int(nblk.max())
    block_table = np.full((B, max_blocks), -1, dtype=np.int32)
    off = 0
    for b in range(B):
        block_table[b, : nblk[b]] = perm[off: off + nblk[b]]
        off += int(nblk[b])

    q = k = v = None
    if dense:
        q = _to_dtype(_normal((B, N, spec.Hq, spec.D), 1.0, seed, spec.tag, _C_Q), spec.dtype)
        cshape = (num_blocks, spec.Hkv, bs, spec.D)
        k = _to_dtype(_normal(cshape, 1.0, seed, spec.tag, _C_K), spec.dtype)
        v = _to_dtype(_normal(cshape, 1.0, seed, spec.tag, _C_V), spec.dtype)

    lg = None
    if logits:
        lg_np = _normal((B, N, V), spec.logit_std, seed, spec.tag, _C_LOGITS)
        for b in range(B):
            for i in np.nonzero(planted[b])[0]:
                row = lg_np[b, parents[b, i]]
                row[draft[b, i]] = row.max() + np.float32(1.0)
        lg = torch.from_numpy(lg_np)

    return Workload(spec=spec, seed=seed, prefix_lens=prefix_lens, parents=parents,
                    draft_tokens=draft, block_table=block_table, num_blocks=num_blocks,
                    planted=planted, match_rate=match_rate, q=q, k_cache=k, v_cache=v,
                    logits=lg)


# The five workloads, numbered 1..5.
CONFIGS = {
    1: Spec("tiny-f32-h4kv2-d64-prefix128-tree8", 1, B=1, Hq=4, Hkv=2, D=64, V=1000, dtype="f32",
            prefix=128, tree=("uniform", 8, 3), logit_std=1.0, match=0.7),
    2: Spec("llama3-8b-layer-bf16-prefix2048-eagle2-tree60", 2, B=1, Hq=32, Hkv=8, D=128, V=128256,
            dtype="bf16", prefix=2048, tree=("eagle2", 60, 6, 10), logit_std=2.0, match=0.7),
    3: Spec("batched-serving-bf16-b32-prefix512-8192-tree26", 3, B=32, Hq=32, Hkv=8, D=128, V=128256,
            dtype="bf16", prefix=(512, 8192), tree=("uniform", 26, 5), logit_std=2.0,
            match=(0.4, 0.9)),
    4: Spec("qwen2-7b-layer-bf16-b4-prefix32768-tree64", 4, B=4, Hq=28, Hkv=4, D=128, V=152064,
            dtype="bf16", prefix=32768, tree=("geometric", 64, 8, 0.5), logit_std=2.0, match=0.6),
    5: Spec("chain-70b-layer-bf16-b128-prefix1024-4096-k8", 5, B=128, Hq=64, Hkv=8, D=128, V=128256,
            dtype="bf16", prefix=(1024, 4096), tree=("chain", 9), logit_std=2.0, match=0.7),
}

# Reduced versions of each workload: same head layout, tree family and value
# distributions, with fewer sequences, shorter prefixes and a smaller vocab so
# that the CPU oracle finishes in seconds.  Prefixes still span several
# 64-key tiles and end mid-block.
SMALL = {
    1: CONFIGS[1],
    2: dataclasses.replace(CONFIGS[2], name="small-llama3-8b-eagle2-tree60", tag=12,
                           prefix=1000, V=5003),
    3: dataclasses.replace(CONFIGS[3], name="small-batched-b5-tree26", tag=13, B=5,
                           prefix=(40, 700), V=4099),
    4: dataclasses.replace(CONFIGS[4], name="small-qwen2-7b-tree64", tag=14, B=2,
                           prefix=(1500, 2600), V=3001),
    5: dataclasses.replace(CONFIGS[5], name="small-chain-b9-k8", tag=15, B=9,
                           prefix=(1, 600), V=2048),
}


def make_config(i: int, seed: int = 0, **kw) -> Workload:
    return build(CONFIGS[i], seed, **kw)


def make_small(i: int, seed: int = 0, **kw) -> Workload:
    return build(SMALL[i], seed, **kw)


def tree_kv_inputs(spec, seed: int = 0):
    """The step's new key and value rows of every tree node, [B, N, Hkv, D]
    in the workload's element type, N(0, 1), for the tree K/V write; they
    are drawn from streams of their own, so the rest of the workload is
    unchanged."""
    shape = (spec.B, spec.N, spec.Hkv, spec.D)
    k = _to_dtype(_normal(shape, 1.0, seed, spec.tag, _C_KNEW), spec.dtype)
    v = _to_dtype(_normal(shape, 1.0, seed, spec.tag, _C_VNEW), spec.dtype)
    return k, v


def stochastic_inputs(spec, seed: int = 0, logits=None, proposals: bool = False):
    """Random inputs of stochastic verification, each from its own stream.

    Returns a dict with ``uniforms`` [B, N] float32 in [0, 1) (entry c decides
    node c), ``expo`` [B, V] float32 Exp(1) variates (an exact zero, which
    float64 draws with probability about 2^-53, is replaced by 2^-53), and
    ``temperature``.  With ``proposals`` (chain trees only) it also returns
    ``draft_probs`` [B, N, V] float32 and ``draft_tokens`` [B, N] int32: the
    drafter stand-in's distribution for node c is a softmax at the sampling
    temperature of the target row of node c - 1 plus N(0, 1) noise, and node
    c's token is drawn from it by inverse CDF (row 0 is uniform and unused).
    ``logits`` [B, N, V] (the workload's target logits) is needed then.
    """
    B, N, V = spec.B, spec.N, spec.V
    u = _rng(seed, spec.tag, _C_UNIF).random((B, N), dtype=np.float32)
    e = _rng(seed, spec.tag, _C_EXPO).standard_exponential((B, V))
    e[e == 0] = 2.0 ** -53
    out = {"uniforms": torch.from_numpy(u), "expo": torch.from_numpy(e.astype(np.float32)),
           "temperature": SAMPLING_TEMPERATURE}
    if proposals:
        if spec.tree[0] != "chain":
            raise ValueError("proposal distributions are generated for chain trees only")
        lg = logits.numpy() if isinstance(logits, torch.Tensor) else np.asarray(logits)
        noise = _normal((B, N, V), 1.0, seed, spec.tag, _C_QNOISE)
        probs = np.empty((B, N, V), dtype=np.float32)
        probs[:, 0, :] = np.float32(1.0 / V)
        draw = _rng(seed, spec.tag, _C_QDRAW).random((B, N))
        tok = np.zeros((B, N), dtype=np.int32)
        for b in range(B):
            z = (lg[b, :N - 1].astype(np.float64) + noise[b, 1:]) / SAMPLING_TEMPERATURE
            z -= z.max(axis=-1, keepdims=True)
            q = np.exp(z)
            q /= q.sum(axis=-1, keepdims=True)
            probs[b, 1:] = q
            cdf = np.cumsum(q, axis=-1)
            for c in range(1, N):
                tok[b, c] = min(int(np.searchsorted(cdf[c - 1], draw[b, c] * cdf[c - 1, -1], side="right")), V - 1)
        out["draft_probs"] = torch.from_numpy(probs)
        out["draft_tokens"] = torch.from_numpy(tok)
    return out


def lm_head_inputs(spec, seed: int = 0):
    """Final hidden states [B, N, H] and the LM-head weight [V, H], both bf16:
    hidden N(0, 1), weight N(0, (logit_std / sqrt(H))^2), so that the scores
    have the workload's logit spread."""
    H = hidden_size(spec)
    hid = _to_dtype(_normal((spec.B, spec.N, H), 1.0, seed, spec.tag, _C_HID), "bf16")
    w = _to_dtype(_normal((spec.V, H), spec.logit_std / float(np.sqrt(H)), seed, spec.tag, _C_WLM), "bf16")
    return hid, w


def draft_tree_shape(spec) -> Tuple[int, int]:
    """(depth, topk) of the draft-tree construction that yields the
    workload's tree size: the EAGLE-2 tree keeps its own; the random trees
    expand their depth with topk 10 (4 in the tiny case, whose vocab is
    1000); the chain is topk 1 over N - 1 levels (the greedy chain)."""
    kind = spec.tree[0]
    if kind == "eagle2":
        return int(spec.tree[2]), int(spec.tree[3])
    if kind == "chain":
        return spec.N - 1, 1
    return int(spec.tree[2]), (4 if "tiny" in spec.name else 10)


def draft_tree_inputs(spec, seed: int = 0, depth: Optional[int] = None, topk: Optional[int] = None):
    """The drafter's next-token scores for draft-tree construction.

    Returns a dict with ``draft_logits`` [B, depth, topk, V] float32,
    N(0, logit_std^2) (row (l, j): the scores at the j-th best node of
    level l - 1; row (0, 0) at the root), ``root_tokens`` [B] int32 uniform
    in [0, V), and ``depth``, ``topk``, ``N``.  Each from its own stream.
    """
    d0, k0 = draft_tree_shape(spec)
    depth = d0 if depth is None else depth
    topk = k0 if topk is None else topk
    B, V = spec.B, spec.V
    lg = _normal((B, depth, topk, V), spec.logit_std, seed, spec.tag, _C_DLOGITS)
    root = _rng(seed, spec.tag, _C_DROOT).integers(0, V, size=B, dtype=np.int64).astype(np.int32)
    return {"draft_logits": torch.from_numpy(lg.reshape(B, depth, topk, V)),
            "root_tokens": torch.from_numpy(root), "depth": depth, "topk": topk, "N": spec.N}
