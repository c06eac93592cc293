"""Draft-tree construction (tv_build_draft_tree) against the oracle's
build_draft_tree.

Parents and tokens must match the oracle exactly wherever every decision the
construction takes is clear by more than DECISION_TOL: the frontier of each
level, the order of each level's best nodes, and the boundary of the global
top N - 1.  The library scores in fp32 (row log-sum-exp in a chunked order)
and the oracle in float64, so scores differ by up to about 2e-5 at these
depths; closer decisions may go either way, and such sequences are checked for
validity instead (a tree of the right shape whose every node is one of its
parent row's topk tokens, scored as its parent plus that token's
log-probability, in descending score order within each level).  Node scores
must match within SCORE_ATOL.
"""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as W

DECISION_TOL = 5e-5
SCORE_ATOL = 1e-4


# ---------------------------------------------------------------- host side

def test_draft_tree_host_checks():
    import tree_attention_verification_05_amd as T
    lib = T.lib
    P16 = 0x10000
    f = lib.tv_build_draft_tree
    need = lib.tv_build_draft_tree_workspace_size(2, 6, 10, 128256)
    # 51 rows of 16 chunks: one (max, sum) pair and ten keys each; per row
    # ten keys and a log-sum-exp
    assert need == 2 * 51 * 16 * (8 + 10 * 8) + 2 * 51 * (10 * 8 + 4)
    assert lib.tv_build_draft_tree_workspace_size(2, 17, 10, 1000) == 0
    assert lib.tv_build_draft_tree_workspace_size(2, 6, 17, 1000) == 0
    assert lib.tv_build_draft_tree_workspace_size(2, 6, 10, 262145) == 0
    assert lib.tv_build_draft_tree_workspace_size(2, 6, 10, 9) == 0

    def call(**kw):
        a = dict(lg=P16, B=2, d=6, k=10, V=128256, N=60, root=None, par=P16, tok=P16, sc=None,
                 ws=P16, wsb=need, s=None)
        a.update(kw)
        return f(a["lg"], a["B"], a["d"], a["k"], a["V"], a["N"], a["root"], a["par"], a["tok"],
                 a["sc"], a["ws"], a["wsb"], a["s"])
    assert call(lg=None) == 1 and call(par=None) == 1 and call(tok=None) == 1
    assert call(B=0) == 2 and call(d=0) == 2 and call(d=17) == 2 and call(k=0) == 2
    assert call(k=17) == 2 and call(V=262145) == 2 and call(N=0) == 2 and call(N=257) == 2
    assert call(k=4, V=3) == 2
    # topk 1 over 6 levels generates 6 nodes: a tree of 7 at most
    assert call(k=1, N=8) == 2
    assert call(lg=P16 + 4) == 5
    assert call(ws=None) == 6 and call(wsb=need - 1) == 6
    assert call(ws=P16 + 8) == 5


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_workload_shapes_generate_enough_nodes(cfg):
    spec = W.CONFIGS[cfg]
    depth, topk = W.draft_tree_shape(spec)
    assert topk + (depth - 1) * topk * topk >= spec.N - 1
    assert topk <= spec.V and depth <= 16 and topk <= 16


def test_chain_workload_is_the_greedy_chain():
    spec = W.SMALL[5]
    x = W.draft_tree_inputs(spec, 0)
    lg = x["draft_logits"].numpy()
    parents, tokens, _ = O.build_draft_tree(lg[0], spec.N, 1, root_token=int(x["root_tokens"][0]))
    assert parents.tolist() == [-1] + list(range(spec.N - 1))
    assert tokens[1:].tolist() == [int(np.argmax(lg[0, l, 0])) for l in range(spec.N - 1)]


# ---------------------------------------------------------------- checkers

def node_levels(parents) -> np.ndarray:
    lev = np.zeros(len(parents), dtype=np.int64)
    for i in range(1, len(parents)):
        lev[i] = lev[parents[i]] + 1
    return lev


def decision_margin(gen, parents, topk: int, depth: int, ignore_exact_ties: bool = False) -> float:
    """Smallest score gap at any decision of the construction, from the
    oracle's generated nodes (score, level, j, rank, token, parent) and its
    tree: the order of each level's topk best (the next level's rows) and of
    its kept nodes (their labels), each level's boundaries, and the boundary
    of the global top N - 1."""
    N = len(parents)
    margin = np.inf
    scores = np.array([g[0] for g in gen])
    levels = np.array([g[1] for g in gen])
    kept = np.bincount(node_levels(parents)[1:] - 1, minlength=depth) if N > 1 else np.zeros(depth, int)
    for l in range(depth):
        s = np.sort(scores[levels == l])[::-1]
        m = min(len(s), max(topk, int(kept[l])) + 1)
        gaps = s[:m - 1] - s[1:m]
        if ignore_exact_ties:
            gaps = gaps[gaps > 0]
        if len(gaps):
            margin = min(margin, float(gaps.min()))
    s = np.sort(scores)[::-1]
    if len(s) > N - 1 >= 1:
        gap = float(s[N - 2] - s[N - 1])
        if not (ignore_exact_ties and gap == 0):
            margin = min(margin, gap)
    return margin


def check_valid(rows, parents, tokens, scores, N: int, topk: int, root_token: int):
    """Validity of a construction result whose decisions may differ from the
    oracle's at near ties.

    Shape: a tree in level order whose every node is one of its parent row's
    topk tokens, scored as its parent plus that token's log-probability, in
    descending score order within each level.  Selection: every candidate is
    regenerated from the tree's own frontiers (the first topk nodes of each
    level, whose ranks name the drafter rows of the next level), and up to
    SCORE_ATOL + DECISION_TOL
      * no candidate left out of the tree scores above the lowest kept node
        (the kept set is the best N - 1 of all generated nodes), and
      * no candidate of a level outside that level's first topk nodes scores
        above the topk-th of them (each frontier is its level's top-k)."""
    depth = rows.shape[0]
    tol = SCORE_ATOL + DECISION_TOL
    assert parents[0] == -1 and tokens[0] == root_token and scores[0] == 0
    level = np.zeros(N, dtype=np.int64)
    for i in range(1, N):
        p = int(parents[i])
        assert 0 <= p < i
        level[i] = level[p] + 1
        assert level[i] >= level[i - 1] and level[i] <= depth
    by_level = {l: [i for i in range(N) if level[i] == l] for l in range(depth + 1)}
    lps = {}

    def row_logp(l, j):
        if (l, j) not in lps:
            lps[l, j] = O.log_softmax(rows[l, j])
        return lps[l, j]

    seen = set()
    for i in range(1, N):
        l, p = int(level[i]), int(parents[i])
        j = 0 if l == 1 else by_level[l - 1].index(p)       # the parent's rank within its level
        assert 0 <= j < topk
        lp = row_logp(l - 1, j)
        assert tokens[i] in set(O.top_tokens(lp, topk).tolist())
        assert abs(scores[i] - (scores[p] + lp[tokens[i]])) <= SCORE_ATOL
        assert (p, int(tokens[i])) not in seen
        seen.add((p, int(tokens[i])))
        if i > 1 and level[i - 1] == l:
            assert scores[i] <= scores[i - 1] + SCORE_ATOL
    if N == 1:
        return
    s_min = float(scores[1:].min())
    for l in range(1, depth + 1):
        frontier = [0] if l == 1 else by_level[l - 1][:topk]
        cands = []
        for j, p in enumerate(frontier):
            lp = row_logp(l - 1, j)
            for t in O.top_tokens(lp, topk):
                cands.append((float(scores[p] + lp[t]), p, int(t)))
        for sc, p, t in cands:
            assert (p, t) in seen or sc <= s_min + tol, (
                f"level {l}: candidate (parent {p}, token {t}) scores {sc:.6f}, left out of a tree "
                f"whose lowest kept score is {s_min:.6f}")
        nodes = by_level[l]
        if len(nodes) >= topk:
            kth = float(scores[nodes[topk - 1]])
            top = {(int(parents[i]), int(tokens[i])) for i in nodes[:topk]}
            for sc, p, t in cands:
                assert (p, t) in top or sc <= kth + tol, (
                    f"level {l}: candidate (parent {p}, token {t}) scores {sc:.6f} above the "
                    f"frontier's lowest {kth:.6f}")


def compare_sequence(rows, N, topk, root_token, gp, gt, gs, ignore_exact_ties=False) -> bool:
    """True if compared exactly; False if only checked for validity."""
    parents, tokens, scores, gen = O.build_draft_tree(rows, N, topk, root_token=root_token,
                                                      return_generated=True)
    margin = decision_margin(gen, parents, topk, rows.shape[0], ignore_exact_ties)
    if margin >= DECISION_TOL:
        assert np.array_equal(gp, parents), (gp, parents)
        assert np.array_equal(gt, tokens), (gt, tokens)
        assert np.abs(gs - scores).max() <= SCORE_ATOL
        return True
    check_valid(rows, gp, gt, gs, N, topk, root_token)
    return False


def run_gpu(lg: np.ndarray, N: int, root: np.ndarray):
    import tree_attention_verification_05_amd as T
    x = torch.from_numpy(np.ascontiguousarray(lg, dtype=np.float32)).cuda()
    r = torch.from_numpy(root.astype(np.int32)).cuda()
    p, t, s = T.tv_build_draft_tree(x, N, root_tokens=r)
    torch.cuda.synchronize()
    return p.cpu().numpy(), t.cpu().numpy(), s.cpu().numpy()


def clear_inputs(B, depth, topk, V, N, seed0, std=2.0):
    """Random draft scores whose every decision is clear by DECISION_TOL in
    the oracle (the first seed from seed0 on that gives one)."""
    for seed in range(seed0, seed0 + 50):
        rng = np.random.default_rng([seed, B, depth, topk, V, N])
        lg = (rng.standard_normal((B, depth, topk, V), dtype=np.float32) * np.float32(std))
        root = rng.integers(0, V, size=B).astype(np.int32)
        ok = True
        for b in range(B):
            parents, _, _, gen = O.build_draft_tree(lg[b], N, topk, return_generated=True)
            if decision_margin(gen, parents, topk, depth) < DECISION_TOL:
                ok = False
                break
        if ok:
            return lg, root
    raise AssertionError("no input with clear decisions")


# ---------------------------------------------------------------- GPU parity

CASES = [
    # B, depth, topk, V, N
    (3, 3, 4, 1000, 8),          # the tiny workload's shape
    (2, 4, 5, 17384, 40),        # three chunks, ragged tail
    (2, 3, 3, 5003, 20),         # V not a multiple of 4
    (1, 1, 7, 300, 8),           # one level: a star of the root's top tokens
    (2, 6, 1, 2048, 7),          # topk 1: the greedy chain
    (1, 16, 16, 1024, 256),      # the largest depth, topk and tree
    (2, 5, 10, 4000, 1),         # the root alone
    (1, 2, 16, 3 * 8192 + 4, 100),   # last chunk shorter than topk
    (1, 3, 4, 262144, 30),       # the largest vocab
    (4, 2, 3, 700, 12),          # every generated node kept (3 + 9 = 12 > 11)
    (1, 2, 3, 700, 13),          # exactly every generated node
]


@pytest.mark.gpu
@pytest.mark.parametrize("case", CASES, ids=[f"B{c[0]}-d{c[1]}-k{c[2]}-V{c[3]}-N{c[4]}" for c in CASES])
def test_draft_tree_parity_small(case):
    B, depth, topk, V, N = case
    print(f"draft tree B={B} depth={depth} topk={topk} V={V} N={N}", flush=True)
    lg, root = clear_inputs(B, depth, topk, V, N, seed0=7)
    gp, gt, gs = run_gpu(lg, N, root)
    for b in range(B):
        assert compare_sequence(lg[b], N, topk, int(root[b]), gp[b], gt[b], gs[b])


@pytest.mark.gpu
def test_draft_tree_exact_ties():
    """Every row constant: all tokens of a row tie (lowest ids first) and all
    candidates of a level tie (generation order decides); both sides compute
    bit-identical scores within a level, so the result is exact."""
    B, depth, topk, V, N = 2, 4, 5, 9000, 60
    lg = np.zeros((B, depth, topk, V), dtype=np.float32)
    lg[1] = 0.25
    root = np.array([5, 6], dtype=np.int32)
    gp, gt, gs = run_gpu(lg, N, root)
    for b in range(B):
        parents, tokens, scores = O.build_draft_tree(lg[b], N, topk, root_token=int(root[b]))
        assert np.array_equal(gp[b], parents) and np.array_equal(gt[b], tokens)
        assert np.abs(gs[b] - scores).max() <= SCORE_ATOL


@pytest.mark.gpu
def test_draft_tree_repeated_top_values():
    """Rows whose best values repeat at several ids (lower id first) and whose
    large entries are spread over many lanes, so that far more entries than
    topk pass a chunk's first cut."""
    B, depth, topk, V, N = 2, 3, 16, 2 * 8192, 80
    rng = np.random.default_rng(11)
    lg = rng.standard_normal((B, depth, topk, V), dtype=np.float32)
    e = np.arange(8192)
    group = ((e // 4) % 256) // 8            # an 8-lane group of 256-thread, 16-byte-load chunks
    spread = np.where(group < 16, np.float32(10) - np.float32(0.25) * group, np.float32(0))
    lg[0, 0, 0, :8192] = spread              # more than 512 entries at or above the cut
    lg[1, 1, 2, 8192:] = spread
    for b in range(B):                       # repeated maxima at scattered ids
        lg[b, 2, 1, [17, 900, 8191, 8192, 16000]] = 9.5
    root = np.array([1, 2], dtype=np.int32)
    gp, gt, gs = run_gpu(lg, N, root)
    for b in range(B):
        compare_sequence(lg[b], N, topk, int(root[b]), gp[b], gt[b], gs[b], ignore_exact_ties=True)


@pytest.mark.gpu
@pytest.mark.parametrize("cfg", [2, 3, 4, 5])
def test_draft_tree_parity_full_size(cfg):
    """The workloads at full size, in the launch the benchmark times; every
    sequence is compared exactly where all its decisions are clear, and
    checked for validity and selection (check_valid) where one is not."""
    spec = W.CONFIGS[cfg]
    x = W.draft_tree_inputs(spec, 0)
    lg = x["draft_logits"].numpy()
    root = x["root_tokens"].numpy()
    print(f"draft tree {spec.name}: shape {tuple(lg.shape)}", flush=True)
    gp, gt, gs = run_gpu(lg, spec.N, root)
    exact = [compare_sequence(lg[b], spec.N, x["topk"], int(root[b]), gp[b], gt[b], gs[b])
             for b in range(spec.B)]
    print(f"exactly compared {sum(exact)} of {len(exact)} sequences; the rest hold near ties and "
          f"passed the validity and selection checks", flush=True)
    from gpu_util import record
    record(f"draft_tree full{cfg}", seqs=len(exact), exact=sum(exact))


@pytest.mark.gpu
@pytest.mark.parametrize("cfg", [2, 3])
def test_built_tree_drives_the_verification_step(cfg):
    """The tree built on the GPU (parents and tokens) drives the verification
    step on the GPU (mask, attention, greedy acceptance, compaction); the
    oracle builds its own tree from the same drafter scores and runs its own
    step.  Some drafted tokens are planted as the target's choice at their
    parent, so that paths of several nodes are accepted."""
    import dataclasses
    import tree_attention_verification_05_amd as T
    from gpu_util import check_accept, check_attention, oracle_attention, raw_bits, run_step, upload
    w = W.make_small(cfg)
    spec = w.spec
    depth, topk = W.draft_tree_shape(spec)
    for seed in range(20):       # drafter scores whose every decision is clear
        x = W.draft_tree_inputs(spec, seed)
        lg = x["draft_logits"].numpy()
        root = x["root_tokens"].numpy()
        built = [O.build_draft_tree(lg[b], spec.N, topk, root_token=int(root[b]), return_generated=True)
                 for b in range(spec.B)]
        if all(decision_margin(g[3], g[0], topk, depth) >= DECISION_TOL for g in built):
            break
    else:
        raise AssertionError("no drafter scores with clear decisions")
    print(f"draft tree -> step on {spec.name}, drafter seed {seed}", flush=True)
    gp, gt, _ = run_gpu(lg, spec.N, root)
    parents = np.stack([g[0] for g in built]).astype(np.int32)
    tokens = np.stack([g[1] for g in built]).astype(np.int32)
    assert np.array_equal(gp, parents) and np.array_equal(gt, tokens)

    # the target agrees with the drafter at 70 % of the nodes (one child per parent)
    logits = w.logits.numpy().copy()
    rng = np.random.default_rng(cfg)
    for b in range(spec.B):
        planted_parent = set()
        for i in range(1, spec.N):
            p = int(parents[b, i])
            if p not in planted_parent and rng.random() < 0.7:
                logits[b, p, tokens[b, i]] = logits[b, p].max() + np.float32(1.0)
                planted_parent.add(p)
    w2 = dataclasses.replace(w, parents=gp.astype(np.int32), draft_tokens=gt.astype(np.int32),
                             logits=torch.from_numpy(logits))
    d = upload(w2)
    k0, v0 = raw_bits(w2.k_cache), raw_bits(w2.v_cache)
    res = run_step(T, d, w2.max_prefix_len)
    assert int(d["status"].item()) == 0
    mref, dref = O.build_tree_mask(parents)
    assert np.array_equal(res["mask"].cpu().numpy().view(np.uint64), mref)
    seqs = list(range(spec.B))
    check_attention(res["out"], oracle_attention(w2, seqs), seqs, w2.q.dtype)
    aref = O.accept_greedy(logits, tokens, parents)
    check_accept(res, aref)
    assert aref["accept_len"].max() >= 2
    kref, vref, nl = O.kv_compact(k0, v0, w2.block_table, w2.prefix_lens, aref["accepted_nodes"],
                                  aref["accept_len"])
    assert np.array_equal(res["new_lens"].cpu().numpy(), nl)
    assert np.array_equal(raw_bits(d["k"]), kref) and np.array_equal(raw_bits(d["v"]), vref)


def test_binding_rejects_host_tensors_and_bad_shapes():
    """Argument marshalling only: host tensors, wrong dtypes and ranks are
    refused before anything reaches the library (no GPU needed)."""
    import tree_attention_verification_05_amd as T
    with pytest.raises(ValueError, match="GPU"):
        T.tv_build_draft_tree(torch.zeros(1, 2, 3, 8), 4)
    with pytest.raises((TypeError, ValueError)):
        T.tv_build_draft_tree(torch.zeros(1, 2, 3, 8, dtype=torch.float64), 4)
    with pytest.raises(TypeError):
        T.tv_build_draft_tree(np.zeros((1, 2, 3, 8), dtype=np.float32), 4)


@pytest.mark.gpu
def test_optional_root_tokens_and_scores():
    """root_tokens NULL gives root token 0; scores NULL leaves the scores
    unwritten while parents and tokens are unchanged."""
    import tree_attention_verification_05_amd as T
    B, depth, topk, V, N = 3, 4, 5, 6000, 30
    lg, root = clear_inputs(B, depth, topk, V, N, seed0=21)
    x = torch.from_numpy(lg).cuda()
    p0, t0, s0 = T.tv_build_draft_tree(x, N, root_tokens=torch.from_numpy(root).cuda())
    p1, t1, s1 = T.tv_build_draft_tree(x, N, want_scores=False)
    torch.cuda.synchronize()
    assert s1 is None
    assert torch.equal(p0, p1)
    assert torch.equal(t0[:, 1:], t1[:, 1:]) and (t1[:, 0] == 0).all()
    assert (t0[:, 0].cpu().numpy() == root).all()
    for b in range(B):
        parents, tokens, scores = O.build_draft_tree(lg[b], N, topk)
        assert np.array_equal(p1[b].cpu().numpy(), parents) and np.array_equal(t1[b].cpu().numpy(), tokens)
        assert np.abs(s0[b].cpu().numpy() - scores).max() <= SCORE_ATOL
