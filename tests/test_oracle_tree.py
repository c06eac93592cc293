"""Pins of the oracle's draft-tree construction (CPU only).

The oracle grows the tree level by level: every kept node proposes its
topk most probable tokens, the topk best candidates (cumulative
log-probability) are kept for the next level, and the tree is the root plus
the N - 1 best generated nodes ("EAGLE代码实现原理" page, 树结构缓冲: branch
prediction and level pruning; "vLLM-TreeEagle" README, 核心组件 item 3).
The pins: a hand-worked case, the one-branch and one-level special cases,
an exhaustive two-level case checked against brute-force enumeration of all
paths, and invariants on random cases.
"""
import itertools

import numpy as np
import pytest

import oracle as O


def test_hand_worked():
    # V = 3, topk = 2, depth 2; rows given as probabilities (log of them is
    # the log softmax).  Level 0 from the root: token 0 (0.5), token 1 (0.3).
    # Slot 0 (token 0) proposes token 1 (0.5 * 0.5 = 0.25) and token 2
    # (0.5 * 0.4 = 0.20); slot 1 (token 1) proposes token 0 (0.3 * 0.7 =
    # 0.21) and token 1 (0.3 * 0.2 = 0.06).  The four best: 0.5, 0.3, 0.25,
    # 0.21 -> nodes [root, t0, t1, t0->t1, t1->t0].
    rows = np.log(np.array([[[0.5, 0.3, 0.2], [1 / 3, 1 / 3, 1 / 3]],
                            [[0.1, 0.5, 0.4], [0.7, 0.2, 0.1]]]))
    parents, tokens, scores = O.build_draft_tree(rows, 5, 2, root_token=9)
    assert parents.tolist() == [-1, 0, 0, 1, 2]
    assert tokens.tolist() == [9, 0, 1, 1, 0]
    np.testing.assert_allclose(np.exp(scores), [1.0, 0.5, 0.3, 0.25, 0.21], rtol=1e-12)


def test_one_branch_is_the_greedy_chain():
    rng = np.random.default_rng(1)
    depth, V = 5, 40
    rows = rng.normal(size=(depth, 1, V)) * 2
    parents, tokens, scores = O.build_draft_tree(rows, depth + 1, 1)
    assert parents.tolist() == [-1] + list(range(depth))
    assert tokens[1:].tolist() == [int(np.argmax(rows[l, 0])) for l in range(depth)]
    z = rows[:, 0, :]
    lp = z - z.max(axis=1, keepdims=True)
    lp = lp - np.log(np.exp(lp).sum(axis=1, keepdims=True))
    np.testing.assert_allclose(scores[1:], np.cumsum(lp.max(axis=1)), rtol=1e-12)


def test_one_level_is_a_star_of_the_top_tokens():
    rng = np.random.default_rng(2)
    V, k = 50, 8
    rows = rng.normal(size=(1, k, V))
    parents, tokens, _ = O.build_draft_tree(rows, 6, k)
    assert parents.tolist() == [-1, 0, 0, 0, 0, 0]
    assert tokens[1:].tolist() == np.argsort(-rows[0, 0])[:5].tolist()


@pytest.mark.parametrize("seed", range(4))
def test_exhaustive_two_levels_match_brute_force(seed):
    # topk = V: nothing is pruned, so the tree is the N - 1 most probable
    # paths of length 1 or 2; a level-1 node's row is its probability rank
    rng = np.random.default_rng(10 + seed)
    V, N = 5, 12
    rows = rng.normal(size=(2, V, V)) * 1.5
    p0 = np.exp(rows[0, 0]) / np.exp(rows[0, 0]).sum()
    rank = {int(t): r for r, t in enumerate(np.argsort(-p0, kind="stable"))}
    paths = {(t,): p0[t] for t in range(V)}
    for t1, t2 in itertools.product(range(V), range(V)):
        row = rows[1, rank[t1]]
        paths[(t1, t2)] = p0[t1] * np.exp(row[t2]) / np.exp(row).sum()
    best = sorted(paths, key=lambda k_: -paths[k_])[:N - 1]
    parents, tokens, scores = O.build_draft_tree(rows, N, V)
    got = set()
    for i in range(1, N):
        path, c = [], i
        while c != 0:
            path.append(int(tokens[c]))
            c = parents[c]
        got.add(tuple(reversed(path)))
        np.testing.assert_allclose(np.exp(scores[i]), paths[tuple(reversed(path))], rtol=1e-12)
    assert got == set(best)


@pytest.mark.parametrize("seed", range(6))
def test_invariants_on_random_trees(seed):
    rng = np.random.default_rng(100 + seed)
    depth, k, V = int(rng.integers(2, 7)), int(rng.integers(2, 9)), int(rng.integers(20, 300))
    rows = rng.normal(size=(depth, k, V)) * rng.uniform(0.5, 3)
    G = k + (depth - 1) * k * k
    N = int(rng.integers(2, min(G, 200) + 2))
    parents, tokens, scores, gen = O.build_draft_tree(rows, N, k, return_generated=True)
    assert O.tree_valid(parents)
    for i in range(1, N):
        assert scores[i] < scores[parents[i]]           # log-probabilities are negative
    for p in range(N):                                   # siblings carry distinct tokens
        kids = [int(tokens[c]) for c in range(1, N) if parents[c] == p]
        assert len(kids) == len(set(kids))
    depth_of = np.zeros(N, dtype=int)
    for i in range(1, N):
        depth_of[i] = depth_of[parents[i]] + 1
    assert np.all(np.diff(depth_of) >= 0)                # numbered level by level
    kept = sorted(scores[1:])
    dropped = sorted(g[0] for g in gen)[: len(gen) - (N - 1)]
    assert not dropped or max(dropped) <= min(kept)      # the N - 1 best generated nodes
    # every level's expanded nodes are that level's topk best candidates
    for lev in range(depth - 1):
        cand = [i for i, g in enumerate(gen) if g[1] == lev]
        expanded = {g[5] for g in gen if g[1] == lev + 1}
        top = sorted(cand, key=lambda i: (-gen[i][0], i))[:k]
        assert expanded == set(top)


def test_root_only_and_too_few_nodes():
    rows = np.zeros((1, 2, 4))
    parents, tokens, scores = O.build_draft_tree(rows, 1, 2, root_token=3)
    assert parents.tolist() == [-1] and tokens.tolist() == [3] and scores.tolist() == [0.0]
    with pytest.raises(AssertionError):
        O.build_draft_tree(rows, 4, 2)
