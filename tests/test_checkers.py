"""The GPU tests' own checkers, pinned on the CPU: each accepts the oracle's
result and rejects a planted mistake, so that a checker that passes
everything cannot hide a wrong GPU result."""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from test_draft_tree import DECISION_TOL, SCORE_ATOL, check_valid
from test_lm_head import accumulation_tol
from test_stochastic import divergence_margin


# ---------------------------------------------------------------- draft tree

def tree_from_keep(gen, keep, N, root_token):
    """Parents, tokens and scores of the tree that keeps the generated nodes
    ``keep``, labelled as the construction labels them (level, then score
    descending, then candidate order)."""
    keep = sorted(keep, key=lambda g: (gen[g][1], -gen[g][0], gen[g][2], gen[g][3]))
    label = {g: i + 1 for i, g in enumerate(keep)}
    parents = np.full(N, -1, dtype=np.int64)
    tokens = np.zeros(N, dtype=np.int64)
    scores = np.zeros(N)
    tokens[0] = root_token
    for g, i in label.items():
        pg = gen[g][5]
        parents[i] = 0 if pg < 0 else label[pg]
        tokens[i] = gen[g][4]
        scores[i] = gen[g][0]
    return parents, tokens, scores


def draft_case(seed=3, depth=4, topk=5, V=3000, N=40):
    rng = np.random.default_rng(seed)
    rows = rng.standard_normal((depth, topk, V)).astype(np.float32) * 2
    parents, tokens, scores, gen = O.build_draft_tree(rows, N, topk, root_token=7, return_generated=True)
    return rows, parents, tokens, scores, gen


def test_check_valid_accepts_the_oracle_tree():
    for seed in range(5):
        rows, p, t, s, _ = draft_case(seed)
        check_valid(rows, p, t, s, len(p), rows.shape[1], 7)


def test_check_valid_rejects_a_tree_that_drops_a_better_node():
    """Swap the best kept leaf for the best candidate left out whose parent
    is kept: still a well-formed tree of the right size, but not the best
    N - 1 nodes."""
    rows, p, t, s, gen = draft_case(4)
    N, topk = len(p), rows.shape[1]
    ids = {(gen[g][1], gen[g][2], gen[g][3]) for g in range(len(gen))}
    assert len(ids) == len(gen)
    keep = sorted(range(len(gen)), key=lambda g: (-gen[g][0], gen[g][1], gen[g][2], gen[g][3]))[:N - 1]
    kept = set(keep)
    parents_of_kept = {gen[g][5] for g in kept}
    leaves = [g for g in kept if g not in parents_of_kept]
    best_leaf = max(leaves, key=lambda g: gen[g][0])
    outside = [g for g in range(len(gen)) if g not in kept and (gen[g][5] < 0 or gen[g][5] in kept)
               and gen[g][5] != best_leaf]
    worst_in = max(outside, key=lambda g: gen[g][0])
    assert gen[best_leaf][0] > gen[worst_in][0] + SCORE_ATOL + DECISION_TOL
    bad = (kept - {best_leaf}) | {worst_in}
    bp, bt, bs = tree_from_keep(gen, bad, N, 7)
    with pytest.raises(AssertionError):
        check_valid(rows, bp, bt, bs, N, topk, 7)


def test_check_valid_rejects_a_wrong_frontier():
    """A construction that expands a level's candidates in candidate order
    instead of by score: its tree is well formed, every node is a top-k
    token of its parent's row, but a frontier is not its level's top-k."""
    rows, _, _, _, _ = draft_case(5, depth=3, topk=4, N=30)
    depth, topk, V = rows.shape
    N = 30
    gen, frontier = [], [(0.0, -1)]
    for lev in range(depth):
        cands = []
        for j, (fs, fid) in enumerate(frontier):
            lp = O.log_softmax(rows[lev, j])
            for r, tk in enumerate(O.top_tokens(lp, topk)):
                cands.append((fs + lp[tk], lev, j, r, int(tk), fid))
        first = len(gen)
        gen.extend(cands)
        frontier = [(cands[i][0], first + i) for i in range(topk)]   # the mistake
    order = sorted(range(len(gen)), key=lambda g: (-gen[g][0], gen[g][1], gen[g][2], gen[g][3]))
    kept, keep = set(), []
    for g in order:                   # best N - 1, closed under ancestors
        if len(keep) == N - 1:
            break
        if gen[g][5] < 0 or gen[g][5] in kept:
            kept.add(g)
            keep.append(g)
    bp, bt, bs = tree_from_keep(gen, keep, N, 7)
    with pytest.raises(AssertionError):
        check_valid(rows, bp, bt, bs, N, topk, 7)


# ---------------------------------------------------------------- stochastic

def stoch_case(seed=0):
    w = W.make_small(3, seed)
    x = W.stochastic_inputs(w.spec, seed, w.logits)
    return w, x


def test_divergence_margin_is_none_on_the_oracle_path():
    w, x = stoch_case(1)
    lg, u = w.logits.numpy(), x["uniforms"].numpy()
    for b in range(w.B):
        path, _, _ = O.stochastic_walk(lg[b], w.draft_tokens[b], w.parents[b], 0.7, u[b], x["expo"][b].numpy())
        assert divergence_margin(lg[b], w.draft_tokens[b], w.parents[b], 0.7, u[b], None, path) is None


def test_divergence_margin_names_the_decision_where_the_paths_part():
    """A GPU path cut one node short parts from the rule at the test that
    accepted the dropped node: the margin returned is that test's margin."""
    w, x = stoch_case(2)
    lg, u = w.logits.numpy(), x["uniforms"].numpy()
    checked = 0
    for b in range(w.B):
        path, _, _ = O.stochastic_walk(lg[b], w.draft_tokens[b], w.parents[b], 0.7, u[b], x["expo"][b].numpy())
        if len(path) < 2:
            continue
        last = path[-1]
        parent = path[-2]
        # the rule's own margin at the test that accepted `last`
        r = O.target_probs(lg[b, parent], 0.7)
        for c in range(parent + 1, last):
            if w.parents[b, c] == parent:
                q = np.zeros(lg.shape[-1])
                q[int(w.draft_tokens[b, c])] = 1.0
                r = O.residual(r, q)
        tx = int(w.draft_tokens[b, last])
        lhs = float(u[b, last])
        want = abs(lhs - r[tx]) / max(lhs, r[tx])
        got = divergence_margin(lg[b], w.draft_tokens[b], w.parents[b], 0.7, u[b], None, path[:-1])
        assert got == pytest.approx(want, rel=1e-12)
        assert divergence_margin(lg[b], w.draft_tokens[b], w.parents[b], 0.7, u[b], None,
                                 path + [w.N + 5]) == np.inf
        checked += 1
    assert checked > 0


# ---------------------------------------------------------------- LM head

def test_accumulation_bound_covers_fp32_sums():
    """The LM-head tolerance holds for float32 sums of bf16 products taken
    in two different orders (BLAS blocks and a plain sequential loop)."""
    g = torch.Generator().manual_seed(0)
    H, V = 4096, 300
    h = (torch.randn(H, generator=g)).to(torch.bfloat16).double().numpy()
    w = (torch.randn(V, H, generator=g) * (2.0 / 64)).to(torch.bfloat16).double().numpy()
    exact = w @ h
    tol = accumulation_tol(h, w)
    s_blas = (w.astype(np.float32) @ h.astype(np.float32)).astype(np.float64)
    prods = (w * h).astype(np.float32)          # each bf16 product is exact in fp32
    s_seq = np.zeros(V, dtype=np.float32)
    for i in range(H):
        s_seq += prods[:, i]
    for s in (s_blas, s_seq.astype(np.float64)):
        err = np.abs(s - exact)
        assert (err <= tol).all()
        assert err.max() > 0                     # the sums did round
    # and it is far tighter than the per-score slack it replaces
    assert tol.max() < 1e-3 * (1 + np.abs(exact).max())
