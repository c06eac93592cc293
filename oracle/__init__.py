"""CPU oracle for single-pass verification of a draft token tree.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg import this package.  It shares no code, header,
table or helper with the GPU library and imports nothing from it; the two meet
only in the seeded input generators of the ``workloads`` package.

Everything here is the plain definition of what the verification step
computes, written out in NumPy in float64 (inputs are bf16 or fp32 values,
which float64 holds exactly).  There is no blocking, no split of the key
range, no online softmax and no reordering beyond what the definitions state.

Sources (web pages; cited by title and section):

* "vLLM-TreeEagle: Tree Attention优化的EAGLE3推测解码框架" (README) -- section
  核心组件, item 1 TreeAttentionLayer: every candidate path is verified in one
  forward pass under a tree attention mask built at run time; section
  技术创新点 1: the mask supports irregular candidate trees; architecture
  graph: the tree-attention layer sits on PagedAttention.
* "EAGLE代码实现原理：从树结构缓冲到KV缓存优化的技术细节" -- section
  KV缓存优化: ``KVCache.copy(indices, prev_length)`` gathers the cache rows
  named by ``indices`` and writes them contiguously starting at
  ``prev_length``; section 树结构缓冲: candidate paths share the computation
  of their common prefix.
* "P-EAGLE：vLLM集成并行推测解码加速LLM推理" -- section 技术原理和实现方式,
  steps 3 and 4: the target scores all proposed tokens in one pass (with a
  tree attention mask), and the sequence is truncated at the first rejected
  token; section 技术难点和解决方案: the block manager rolls the cache back or
  appends to it.
* "vLLM EAGLE 投机解码实战：EAGLE/EAGLE3 草稿模型配置、源码实现与接受率评测" --
  section 无损性保障: greedy speculative decoding must produce exactly what
  greedy decoding produces, and sampled speculative decoding must keep the
  target distribution (its rejection sampler is tested for convergence to
  it).

Readings taken where the pages are silent (each is also listed with the
design notes):

* Node 0 of every tree is the root, the last verified token; its K/V is
  written by this pass like every other node's, and its draft token is never
  compared.  ``parents[0] == -1`` and ``0 <= parents[i] < i`` for i >= 1.
* Node i's key and value sit in the paged cache at logical position
  ``prefix_len + i`` (the in-cache layout that ``KVCache.copy`` implies).
* Query head h reads KV head ``h // (Hq // Hkv)``; scale defaults to
  ``1/sqrt(D)``; there is no positional term inside attention.
* Greedy acceptance: the target's choice at a node is the lowest vocabulary
  index among the row's maxima (``np.argmax``).  The accepted path is the
  longest path from the root whose every child carries its parent's choice;
  equally long paths are ordered as sequences of node indices and the
  smallest is taken (this only matters when siblings share a token).
* ``accept_len`` counts accepted draft tokens (root and bonus excluded);
  ``accepted_nodes`` lists the path from the root, padded with -1; the bonus
  token is the target's choice at the last accepted node.  Compaction moves
  ``accept_len + 1`` cache rows (root plus accepted drafts) and the new
  length is ``prefix_len + accept_len + 1``.
* Stochastic acceptance: the speculative-sampling rule (accept a proposal x
  from q with probability min(1, r(x)/q(x)), else continue from the
  normalised positive part of r - q), applied to the children of a node in
  index order; a deterministic proposal is the point mass on its token.  The
  random numbers are inputs: one uniform per node and one Exp(1) variate per
  vocabulary entry for the final draw (largest r[v] / E[v]).

Parity pins for every function here live in the CPU test suite (brute force,
closed forms, textbook special cases, invariants).
"""
from __future__ import annotations

import numpy as np

# status bits reported for malformed inputs
ST_BAD_TREE = 1      # parents[0] != -1 or parents[i] outside [0, i)
ST_BAD_CACHE = 2     # a block id outside [0, num_blocks) or prefix_len > max_prefix_len
ST_BAD_TOKEN = 4     # a draft token (nodes >= 1) outside [0, V)
ST_BAD_RANDOM = 8    # a uniform outside [0, 1) or an exponential variate not in (0, inf)
ST_UNSUPPORTED = 16  # proposal distributions given for a tree that is not a chain


# --------------------------------------------------------------------------
# tree structure
# --------------------------------------------------------------------------

def tree_valid(parents) -> bool:
    """A parent array is a valid tree iff the root has parent -1 and every
    other node's parent comes before it ("vLLM-TreeEagle" README, 技术创新点 1:
    the candidate tree is built dynamically, any shape allowed)."""
    p = np.asarray(parents)
    if len(p) == 0 or p[0] != -1:
        return False
    return all(0 <= int(p[i]) < i for i in range(1, len(p)))


def tree_structure(parents):
    """Ancestor-or-self sets and depths of a draft tree.

    anc[i, j] is True iff node j lies on the path from the root to node i
    (j == i included): ``anc*(i) = {i} U anc*(parent(i))``.  This is the tree
    attention mask of the "vLLM-TreeEagle" README (核心组件, TreeAttentionLayer):
    node i may attend to tree node j iff j is an ancestor of i or i itself.
    depth[0] = 0 and depth[i] = depth[parent(i)] + 1.
    """
    p = np.asarray(parents, dtype=np.int64)
    if not tree_valid(p):
        raise ValueError("invalid parent array")
    n = len(p)
    anc = np.zeros((n, n), dtype=bool)
    depth = np.zeros(n, dtype=np.int64)
    for i in range(n):
        if i > 0:
            anc[i] = anc[p[i]]
            depth[i] = depth[p[i]] + 1
        anc[i, i] = True
    return anc, depth


def mask_words(anc) -> np.ndarray:
    """Pack ancestor rows into little-endian 64-bit words: bit (j % 64) of word
    (j // 64) of row i is set iff anc[i, j]."""
    anc = np.asarray(anc, dtype=bool)
    n = anc.shape[0]
    w = (n + 63) // 64
    out = np.zeros((n, w), dtype=np.uint64)
    for i in range(n):
        for j in np.nonzero(anc[i])[0]:
            out[i, j // 64] |= np.uint64(1) << np.uint64(j % 64)
    return out


def build_tree_mask(parents):
    """Batched mask and depth: parents [B, N] -> (mask uint64 [B, N, W],
    depth int32 [B, N]).  Rows of invalid trees are left zero."""
    parents = np.asarray(parents)
    B, N = parents.shape
    W = (N + 63) // 64
    mask = np.zeros((B, N, W), dtype=np.uint64)
    depth = np.zeros((B, N), dtype=np.int32)
    for b in range(B):
        if tree_valid(parents[b]):
            anc, d = tree_structure(parents[b])
            mask[b] = mask_words(anc)
            depth[b] = d
    return mask, depth


# --------------------------------------------------------------------------
# paged addressing
# --------------------------------------------------------------------------

def cache_rows(block_table_row, positions, block_size: int) -> np.ndarray:
    """Flat token row of logical positions: block ``table[t // bs]``, slot
    ``t % bs`` (paged KV layout under the tree-attention layer, "vLLM-TreeEagle"
    README architecture graph; block-manager paging in the "P-EAGLE" page,
    技术难点和解决方案).  Rows index the token-major view of ``token_rows``."""
    t = np.asarray(positions, dtype=np.int64)
    blk = np.asarray(block_table_row, dtype=np.int64)[t // block_size]
    return blk * block_size + t % block_size


def token_rows(cache) -> np.ndarray:
    """The paged cache ``[num_blocks, Hkv, block_size, D]`` (each block holds
    the slots of one head after another) as one row per token slot:
    ``[num_blocks * block_size, Hkv, D]`` (a copy)."""
    c = np.asarray(cache)
    nb, Hkv, bs, D = c.shape
    return np.ascontiguousarray(c.transpose(0, 2, 1, 3)).reshape(nb * bs, Hkv, D)


def from_token_rows(rows, nb: int, bs: int) -> np.ndarray:
    """Inverse of ``token_rows``."""
    rows = np.asarray(rows)
    Hkv, D = rows.shape[1:]
    return np.ascontiguousarray(rows.reshape(nb, bs, Hkv, D).transpose(0, 2, 1, 3))


# --------------------------------------------------------------------------
# tree attention
# --------------------------------------------------------------------------

def tree_attention(q, k_cache, v_cache, block_table, prefix_lens, parents, scale=None,
                   seqs=None, return_weights=False):
    """Tree-masked attention of every draft node over the prefix and its own
    ancestors.

    Source: "vLLM-TreeEagle" README, 核心组件 item 1 and 技术创新点 1 (one
    forward pass verifies every candidate path under a tree attention mask);
    "EAGLE代码实现原理", 树结构缓冲 (paths share the common prefix); "P-EAGLE"
    page, 技术原理和实现方式 step 3 (the target scores all proposed tokens in one
    pass).

    For sequence b, node i, query head h (KV head kh = h // g, g = Hq // Hkv)
    the visible keys are the prefix positions ``[0, P_b)`` and the tree
    positions ``P_b + j`` for every j in anc*(i).  With
    ``s_t = scale * <q[b,i,h], k[t, kh]>`` over visible t:

        out[b,i,h] = sum_t exp(s_t - max s) v[t, kh] / sum_t exp(s_t - max s)

    q: [B, N, Hq, D]; caches: [num_blocks, Hkv, block_size, D] (any float
    dtype; computed in float64).  Returns float64 [B, N, Hq, D]; sequences not
    in ``seqs`` (default: all) are NaN.  With ``return_weights`` it also
    returns {(b, kh): (weights [N*g, P_b+N], visible [N*g, P_b+N])} with rows
    ordered node-major (row = i*g + h % g).
    """
    q = np.asarray(q, dtype=np.float64)
    B, N, Hq, D = q.shape
    nb, Hkv, bs, D2 = k_cache.shape
    assert D2 == D and Hq % Hkv == 0
    g = Hq // Hkv
    if scale is None or scale <= 0:
        scale = 1.0 / np.sqrt(D)
    kf = token_rows(k_cache)
    vf = token_rows(v_cache)
    out = np.full((B, N, Hq, D), np.nan)
    weights = {}
    for b in (range(B) if seqs is None else seqs):
        P = int(prefix_lens[b])
        anc, _ = tree_structure(parents[b])
        rows = cache_rows(block_table[b], np.arange(P + N), bs)
        K = kf[rows].astype(np.float64)          # [P+N, Hkv, D]
        V = vf[rows].astype(np.float64)
        # visible[i, t]: key position t is visible to node i
        visible = np.zeros((N, P + N), dtype=bool)
        visible[:, :P] = True
        visible[:, P:] = anc
        for kh in range(Hkv):
            Qg = q[b, :, kh * g:(kh + 1) * g, :].reshape(N * g, D)     # row = i*g + hh
            vis = np.repeat(visible, g, axis=0)
            s = scale * (Qg @ K[:, kh, :].T)                             # [N*g, P+N]
            s = np.where(vis, s, -np.inf)
            m = s.max(axis=1, keepdims=True)
            w = np.exp(s - m)                                            # 0 where invisible
            w = w / w.sum(axis=1, keepdims=True)
            o = w @ V[:, kh, :]
            out[b, :, kh * g:(kh + 1) * g, :] = o.reshape(N, g, D)
            if return_weights:
                weights[(b, kh)] = (w, vis)
    if return_weights:
        return out, weights
    return out


# --------------------------------------------------------------------------
# greedy acceptance
# --------------------------------------------------------------------------

def target_argmax(logits) -> np.ndarray:
    """The target's greedy choice per tree node: the lowest index among the
    row's maxima (``np.argmax`` returns the first occurrence).  -0.0 and +0.0
    compare equal.  Rows are the target's next-token scores at each node
    ("P-EAGLE" page, 技术原理和实现方式 step 3)."""
    return np.argmax(np.asarray(logits), axis=-1).astype(np.int64)


def greedy_walk(am, draft_tokens, parents):
    """Longest accepted path of one tree under greedy verification.

    Source: "P-EAGLE" page, 技术原理和实现方式 step 4 (draft tokens are accepted
    while they agree with the target and the sequence is cut at the first
    rejection); "vLLM EAGLE 投机解码实战", 无损性保障 (greedy speculative
    decoding emits exactly the greedy tokens).

    An edge parent(c) -> c is accepted iff ``draft_tokens[c] == am[parent(c)]``
    (the child's draft token is the target's greedy choice after its parent).
    The accepted path is the longest root-started path whose edges are all
    accepted; if several are equally long, the lexicographically smallest
    sequence of node indices.  Written as the plain recursion: from a node,
    follow the accepted child with the longest accepted continuation, the
    lowest child index among equals.  Returns (path, bonus), bonus being the
    target's choice at the path's last node.
    """
    parents = np.asarray(parents)
    draft_tokens = np.asarray(draft_tokens)
    n = len(parents)

    def longest_from(cur):
        best = [cur]
        for c in range(cur + 1, n):       # ascending: the first of equals is kept
            if parents[c] == cur and draft_tokens[c] == am[cur]:
                cand = [cur] + longest_from(c)
                if len(cand) > len(best):
                    best = cand
        return best

    path = longest_from(0)
    return path, int(am[path[-1]])


def accept_greedy(logits, draft_tokens, parents):
    """Batched greedy acceptance: logits [B, N, V], draft_tokens [B, N],
    parents [B, N] -> dict with accept_len [B], accepted_nodes [B, N] (path from
    the root, -1 padded), bonus [B], argmax [B, N]."""
    logits = np.asarray(logits)
    B, N, _ = logits.shape
    am = target_argmax(logits)
    accept_len = np.zeros(B, dtype=np.int32)
    nodes = np.full((B, N), -1, dtype=np.int32)
    bonus = np.zeros(B, dtype=np.int32)
    for b in range(B):
        path, bon = greedy_walk(am[b], draft_tokens[b], parents[b])
        accept_len[b] = len(path) - 1
        nodes[b, :len(path)] = path
        bonus[b] = bon
    return {"accept_len": accept_len, "accepted_nodes": nodes, "bonus": bonus,
            "argmax": am.astype(np.int32)}


# --------------------------------------------------------------------------
# target LM head fused with the greedy choice
# --------------------------------------------------------------------------

def lm_head_logits(hidden, weight) -> np.ndarray:
    """The target's scores of every vocabulary entry at every tree node:
    logits[m, v] = sum_h hidden[m, h] * weight[v, h], in float64 (the output
    projection of the final hidden state onto the vocabulary, no bias, as in
    the Llama- and Qwen-family targets the pages run).  Source: "P-EAGLE"
    page, 技术原理和实现方式 step 3 (one target pass scores every proposed
    token).  hidden [M, H], weight [V, H] -> [M, V]."""
    h = np.asarray(hidden, dtype=np.float64)
    w = np.asarray(weight, dtype=np.float64)
    return h @ w.T


def lm_head_argmax(hidden, weight):
    """Greedy choice and its score per row, without keeping the scores:
    returns (argmax [M] int64, lowest index among the row's maxima; max [M]
    float64).  Source: "vLLM EAGLE 投机解码实战", 无损性保障 (greedy
    verification compares drafts with the target's greedy choice)."""
    lg = lm_head_logits(hidden, weight)
    am = target_argmax(lg)
    return am, lg[np.arange(lg.shape[0]), am]


# --------------------------------------------------------------------------
# stochastic acceptance (temperature > 0)
# --------------------------------------------------------------------------

def target_probs(logits_row, temperature: float) -> np.ndarray:
    """The target's sampling distribution at a node: softmax(logits / T)
    over the vocabulary ("P-EAGLE" page, 技术原理和实现方式 step 3: the target
    scores every proposed token in one pass; 需要注意的问题: the temperature
    sets how random the target's choice is)."""
    z = np.asarray(logits_row, dtype=np.float64) / float(temperature)
    e = np.exp(z - z.max())
    return e / e.sum()


def residual(r, q) -> np.ndarray:
    """What is left of the distribution r after a proposal drawn from q was
    rejected: the positive part of r - q, normalised.  If that part has no
    mass (only possible through rounding, since a rejection needs
    r(x) < q(x)), r is kept."""
    d = np.maximum(np.asarray(r, dtype=np.float64) - q, 0.0)
    m = d.sum()
    return d / m if m > 0 else np.asarray(r, dtype=np.float64)


def race_draw(r, expo):
    """One draw from the distribution proportional to r, given one Exp(1)
    variate per vocabulary entry: the index with the largest r[v] / E[v]
    (the first of equals).  Returns (index, relative gap between the best and
    the runner-up ratio)."""
    t = np.asarray(r, dtype=np.float64) / np.asarray(expo, dtype=np.float64)
    i = int(np.argmax(t))
    if len(t) > 1 and t[i] > 0:
        second = np.max(np.delete(t, i))
        gap = (t[i] - second) / t[i]
    else:
        gap = 1.0
    return i, float(gap)


def stochastic_walk(logits, draft_tokens, parents, temperature: float, uniforms, expo,
                    draft_probs=None, with_residual: bool = False):
    """Stochastic verification of one draft tree.

    Source: "P-EAGLE" page, 技术原理和实现方式 steps 3-4 (the target's
    probabilities of the proposed tokens are compared with the drafter's,
    the sampling rule decides acceptance, the sequence is cut at the first
    rejection); "vLLM EAGLE 投机解码实战", 无损性保障 (sampling stays
    lossless up to floating-point precision, and the rejection sampler is
    tested for convergence to the target distribution).  The rule that does
    both is the speculative-sampling rule: a token x proposed from q is
    accepted with probability min(1, r(x) / q(x)) where r is the target
    distribution, and after a rejection the remaining choice is drawn from
    the normalised positive part of r - q.  On a tree it is applied to the
    children of the current node in index order, each child tested against
    the residual that the rejections of its earlier siblings left.

    Inputs of one sequence: logits [N, V] (row i = target scores after node
    i), draft_tokens [N], parents [N], temperature T > 0, uniforms [N]
    (uniforms[c] in [0, 1) decides child c; entry 0 is unused), expo [V]
    (Exp(1) variates for the final draw), draft_probs [N, V] or None (row c
    = the distribution node c's token was drawn from; None means every token
    was proposed deterministically, a point mass on it, as the top-k
    expansion of an EAGLE-2 tree does).

    From node u (start at the root) with r = softmax(logits[u] / T): for
    each child c of u in increasing index, x = draft_tokens[c], q = the
    proposal of c; c is accepted iff uniforms[c] * q(x) < r(x), and then the
    walk moves to c.  A rejection replaces r by residual(r, q).  When every
    child is rejected (or u is a leaf) the bonus token is drawn from r by
    the exponential race.

    Returns (path, bonus, margin): the accepted nodes from the root, the
    bonus token, and the smallest relative margin of any decision taken (an
    acceptance test |u q(x) - r(x)| / max(u q(x), r(x)), or the gap of the
    final draw), which tells how close a run came to a different result.
    With ``with_residual`` the distribution r of the final draw is appended.
    """
    logits = np.asarray(logits)
    parents = np.asarray(parents)
    draft_tokens = np.asarray(draft_tokens)
    N, V = logits.shape
    path = [0]
    margin = 1.0
    cur = 0
    while True:
        r = target_probs(logits[cur], temperature)
        moved = False
        for c in range(cur + 1, N):
            if parents[c] != cur:
                continue
            x = int(draft_tokens[c])
            if draft_probs is None:
                q = np.zeros(V)
                q[x] = 1.0
            else:
                q = np.asarray(draft_probs[c], dtype=np.float64)
            lhs = float(uniforms[c]) * q[x]
            top = max(lhs, r[x])
            if top > 0:
                margin = min(margin, abs(lhs - r[x]) / top)
            if lhs < r[x]:
                path.append(c)
                cur = c
                moved = True
                break
            r = residual(r, q)
        if not moved:
            bonus, gap = race_draw(r, expo)
            if with_residual:
                return path, bonus, min(margin, gap), r
            return path, bonus, min(margin, gap)


def accept_stochastic(logits, draft_tokens, parents, temperature: float, uniforms, expo,
                      draft_probs=None):
    """Batched stochastic acceptance: logits [B, N, V], draft_tokens [B, N],
    parents [B, N], uniforms [B, N], expo [B, V], draft_probs [B, N, V] or
    None -> dict with accept_len [B], accepted_nodes [B, N] (path from the
    root, -1 padded), bonus [B] and margin [B] (see ``stochastic_walk``).
    A sequence whose tree or draft tokens are invalid gets path [0] and a
    bonus drawn from the root's distribution, as if nothing was proposed."""
    logits = np.asarray(logits)
    B, N, V = logits.shape
    accept_len = np.zeros(B, dtype=np.int32)
    nodes = np.full((B, N), -1, dtype=np.int32)
    bonus = np.zeros(B, dtype=np.int32)
    margin = np.ones(B)
    for b in range(B):
        tok = np.asarray(draft_tokens[b])
        if not tree_valid(parents[b]) or np.any(tok[1:] < 0) or np.any(tok[1:] >= V):
            path = [0]
            bon, mg = race_draw(target_probs(logits[b, 0], temperature), expo[b])
        else:
            path, bon, mg = stochastic_walk(logits[b], tok, parents[b], temperature, uniforms[b],
                                            expo[b], None if draft_probs is None else draft_probs[b])
        accept_len[b] = len(path) - 1
        nodes[b, :len(path)] = path
        bonus[b] = bon
        margin[b] = mg
    return {"accept_len": accept_len, "accepted_nodes": nodes, "bonus": bonus, "margin": margin}


# --------------------------------------------------------------------------
# draft-tree construction (EAGLE-2 style expansion and pruning)
# --------------------------------------------------------------------------

def log_softmax(row) -> np.ndarray:
    """log softmax of one score row, float64."""
    z = np.asarray(row, dtype=np.float64)
    m = z.max()
    return z - m - np.log(np.exp(z - m).sum())


def top_tokens(logp, k: int) -> np.ndarray:
    """The k most probable tokens of a row, most probable first, the lower
    index first among equals."""
    return np.argsort(-np.asarray(logp), kind="stable")[:k]


def build_draft_tree(draft_logits, N: int, topk: int, root_token: int = 0,
                     return_generated: bool = False):
    """Draft tree of N nodes grown level by level from the drafter's scores.

    Source: "EAGLE代码实现原理" page, 树结构缓冲 (branch prediction: likely
    continuations are proposed ahead; level pruning: high-probability paths
    are kept and low-probability branches cut); "vLLM-TreeEagle" README,
    核心组件 item 3 (multi-level candidate generation with path pruning).

    draft_logits [depth, topk, V]: row (l, j) is the drafter's next-token
    scores at the j-th kept node of level l (level 0 keeps the root alone,
    row (0, 0)).  A node's score is the sum of the log-probabilities
    (log softmax of its row) of the tokens on its path; the root's is 0.
    Level l: each kept node proposes its topk most probable tokens (the
    candidates, in order (j, rank)); the topk best candidates (score, then
    candidate order) are kept for level l + 1.  All candidates of all levels
    are the generated nodes; the tree is the root plus the N - 1 best of
    them (score, then level, then candidate order), which is ancestor-closed
    since a child never scores above its parent.  Nodes are numbered by
    (level, rank in that order), so parents come first.

    Returns (parents [N], tokens [N], scores [N]) and, with
    ``return_generated``, the generated nodes as (score, level, j, rank,
    token, parent generated index or -1 for the root).
    """
    lg = np.asarray(draft_logits)
    depth, K, V = lg.shape
    assert K == topk and 1 <= N
    gen = []                                  # generated nodes
    frontier = [(0.0, -1)]                    # (score, generated index); -1 = root
    for lev in range(depth):
        cands = []
        for j, (fs, fid) in enumerate(frontier):
            lp = log_softmax(lg[lev, j])
            for r, t in enumerate(top_tokens(lp, topk)):
                cands.append((fs + lp[t], lev, j, r, int(t), fid))
        first = len(gen)
        gen.extend(cands)
        order = sorted(range(len(cands)), key=lambda i: (-cands[i][0], i))
        frontier = [(cands[i][0], first + i) for i in order[:topk]]
    assert N - 1 <= len(gen), "not enough generated nodes"
    keep = sorted(range(len(gen)), key=lambda g: (-gen[g][0], gen[g][1], gen[g][2], gen[g][3]))[:N - 1]
    keep = sorted(keep, key=lambda g: (gen[g][1], -gen[g][0], gen[g][2], gen[g][3]))
    label = {g: i + 1 for i, g in enumerate(keep)}
    parents = np.full(N, -1, dtype=np.int64)
    tokens = np.zeros(N, dtype=np.int64)
    scores = np.zeros(N)
    tokens[0] = root_token
    for g, i in label.items():
        pg = gen[g][5]
        parents[i] = 0 if pg < 0 else label[pg]   # KeyError would mean not ancestor-closed
        tokens[i] = gen[g][4]
        scores[i] = gen[g][0]
    if return_generated:
        return parents, tokens, scores, gen
    return parents, tokens, scores


# --------------------------------------------------------------------------
# tree K/V write with rotary positions
# --------------------------------------------------------------------------

def rope(x, pos, theta: float) -> np.ndarray:
    """Rotary position embedding along the last axis (D even), rotate-half
    pairing: the pair (x[j], x[j + D/2]), j < D/2, turns by the angle
    ``pos * theta ** (-2 j / D)``:

        x'[j]       = x[j] cos(a_j) - x[j + D/2] sin(a_j)
        x'[j + D/2] = x[j + D/2] cos(a_j) + x[j] sin(a_j)

    The pages do not define the positional encoding; this is the textbook
    rotary embedding in the layout of the Llama-family target models the
    pages run (Llama 3, Qwen2).  x: [..., D]; pos: integers broadcastable to
    x.shape[:-1].  Float64."""
    x = np.asarray(x, dtype=np.float64)
    D = x.shape[-1]
    h = D // 2
    inv = float(theta) ** (-2.0 * np.arange(h, dtype=np.float64) / D)
    ang = np.asarray(pos, dtype=np.float64)[..., None] * inv
    c, s = np.cos(ang), np.sin(ang)
    x1, x2 = x[..., :h], x[..., h:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def tree_positions(parents, prefix_lens) -> np.ndarray:
    """Rotary position of every tree node: ``P_b + depth(i)``.  Siblings are
    alternative continuations of the same prefix, so they share a position;
    along a root-to-leaf path positions are consecutive, as in ordinary
    decoding of that path (reading of the tree attention layer, "vLLM-TreeEagle"
    README, 核心组件 item 1: every path is verified as if decoded alone)."""
    parents = np.asarray(parents)
    B, N = parents.shape
    pos = np.zeros((B, N), dtype=np.int64)
    for b in range(B):
        _, depth = tree_structure(parents[b])
        pos[b] = int(prefix_lens[b]) + depth
    return pos


def tree_kv_write(q, k_new, parents, prefix_lens, theta: float):
    """The tree step's queries and keys at their tree positions, and where
    the new K/V rows go.

    Source: "EAGLE代码实现原理", KV缓存优化 (``cat()`` appends the new rows
    after the current length inside the preallocated cache); "P-EAGLE" page,
    技术难点和解决方案 (the block manager appends the proposed tokens to the
    paged cache); tree positions as in ``tree_positions``.

    Returns (q_rot [B, N, Hq, D], k_rot [B, N, Hkv, D], positions [B, N]),
    float64.  Node i's rotated key and its value (unchanged) are stored at
    logical position ``P_b + i`` (``cache_rows``); no other cache row
    changes."""
    pos = tree_positions(parents, prefix_lens)
    q_rot = rope(q, pos[:, :, None], theta)
    k_rot = rope(k_new, pos[:, :, None], theta)
    return q_rot, k_rot, pos


# --------------------------------------------------------------------------
# KV compaction
# --------------------------------------------------------------------------

def kv_compact(k_cache, v_cache, block_table, prefix_lens, accepted_nodes, accept_len):
    """Move the accepted path's K/V into contiguous slots after the prefix.

    Source: "EAGLE代码实现原理", KV缓存优化 (``copy(indices, prev_length)``:
    select the rows named by ``indices`` into a new tensor, then copy it into
    the rows starting at ``prev_length``); "P-EAGLE" page, 技术难点和解决方案
    (roll the cache back to the accepted tokens).  With L = accept_len + 1 and
    path = accepted_nodes[:L], the rows at logical positions ``P + path`` are
    gathered first and then written to positions ``P + 0 .. P + L - 1``; every
    other row keeps its bytes.  Works on copies of the caches (any dtype, bytes
    preserved); returns (k_new, v_new, new_lens = P + L).
    """
    nb, _, bs, _ = np.asarray(k_cache).shape
    kf = token_rows(k_cache)
    vf = token_rows(v_cache)
    B = len(prefix_lens)
    new_lens = np.zeros(B, dtype=np.int32)
    for b in range(B):
        P = int(prefix_lens[b])
        L = int(accept_len[b]) + 1
        path = np.asarray(accepted_nodes[b][:L], dtype=np.int64)
        src = cache_rows(block_table[b], P + path, bs)
        dst = cache_rows(block_table[b], P + np.arange(L), bs)
        ks = kf[src].copy()
        vs = vf[src].copy()
        kf[dst] = ks
        vf[dst] = vs
        new_lens[b] = P + L
    return from_token_rows(kf, nb, bs), from_token_rows(vf, nb, bs), new_lens


# --------------------------------------------------------------------------
# input validation
# --------------------------------------------------------------------------

def input_status(parents, block_table=None, prefix_lens=None, num_blocks=None,
                 max_prefix_len=None, block_size=16, draft_tokens=None, V=None,
                 uniforms=None, expo=None, proposal_rows=False) -> int:
    """Status bits a verification call should report for these inputs:
    ST_BAD_TREE for an invalid parent array, ST_BAD_CACHE for a block id
    outside [0, num_blocks) among the blocks a sequence uses (prefix plus
    tree) or a prefix longer than ``max_prefix_len``, ST_BAD_TOKEN for a draft
    token of a non-root node outside [0, V), ST_BAD_RANDOM for a uniform of
    a non-root node outside [0, 1) or an exponential variate outside
    (0, inf), ST_UNSUPPORTED when proposal rows come with a valid tree that
    is not a chain (the library takes proposal distributions on chains
    only; the oracle's walk itself has no such limit)."""
    st = 0
    parents = np.asarray(parents)
    B, N = parents.shape
    for b in range(B):
        if not tree_valid(parents[b]):
            st |= ST_BAD_TREE
    if block_table is not None:
        for b in range(B):
            P = int(prefix_lens[b])
            if P > max_prefix_len or P < 0:
                st |= ST_BAD_CACHE
                continue
            used = (P + N + block_size - 1) // block_size
            blk = np.asarray(block_table[b][:used])
            if np.any(blk < 0) or np.any(blk >= num_blocks):
                st |= ST_BAD_CACHE
    if draft_tokens is not None:
        d = np.asarray(draft_tokens)[:, 1:]
        if np.any(d < 0) or np.any(d >= V):
            st |= ST_BAD_TOKEN
    if uniforms is not None:
        u = np.asarray(uniforms)[:, 1:]
        if not np.all((u >= 0) & (u < 1)):
            st |= ST_BAD_RANDOM
    if expo is not None:
        e = np.asarray(expo)
        if not np.all((e > 0) & np.isfinite(e)):
            st |= ST_BAD_RANDOM
    if proposal_rows:
        for b in range(B):
            if tree_valid(parents[b]) and np.any(parents[b][1:] != np.arange(N - 1)):
                st |= ST_UNSUPPORTED
    return st
