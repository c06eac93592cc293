"""Checks of the seeded input generators (structure only; no method arithmetic)."""
import numpy as np
import pytest

import workloads as W


def _depths(par):
    d = np.zeros(len(par), dtype=int)
    for i in range(1, len(par)):
        d[i] = d[par[i]] + 1
    return d


@pytest.mark.parametrize("i", [1, 2, 3, 4, 5])
def test_structure(i):
    w = W.make_config(i, dense=False, logits=False)
    s = w.spec
    assert w.parents.shape == (s.B, s.N)
    for b in range(s.B):
        par = w.parents[b]
        assert par[0] == -1
        assert all(0 <= par[j] < j for j in range(1, s.N))
        d = _depths(par)
        if s.tree[0] in ("uniform", "geometric"):
            assert d.max() == s.tree[2]
        elif s.tree[0] == "eagle2":
            assert d.max() <= s.tree[2]
        else:
            assert list(par) == list(range(-1, s.N - 1))
        # siblings carry distinct tokens, every token in range
        tok = w.draft_tokens[b]
        assert tok.min() >= 0 and tok.max() < s.V
        for p in range(s.N):
            kids = np.nonzero(par == p)[0]
            assert len(set(tok[kids].tolist())) == len(kids)
    # prefix lengths within the stated range
    if isinstance(s.prefix, tuple):
        assert w.prefix_lens.min() >= s.prefix[0] and w.prefix_lens.max() <= s.prefix[1]
    else:
        assert (w.prefix_lens == s.prefix).all()
    # block table: one permutation of physical ids, -1 padded
    used = w.block_table[w.block_table >= 0]
    assert sorted(used.tolist()) == list(range(w.num_blocks))
    for b in range(s.B):
        nblk = (int(w.prefix_lens[b]) + s.N + 15) // 16
        assert (w.block_table[b, :nblk] >= 0).all() and (w.block_table[b, nblk:] == -1).all()


@pytest.mark.parametrize("i", [1, 2, 3])
def test_deterministic_and_component_independent(i):
    a = W.make_small(i, seed=3)
    b = W.make_small(i, seed=3)
    c = W.make_small(i, seed=3, dense=False)
    assert (a.parents == b.parents).all() and (a.block_table == b.block_table).all()
    assert a.q.equal(b.q) and a.k_cache.equal(b.k_cache) and a.logits.equal(b.logits)
    # skipping the dense tensors changes nothing else
    assert (a.parents == c.parents).all() and a.logits.equal(c.logits)
    d = W.make_small(i, seed=4)
    assert not a.logits.equal(d.logits)


@pytest.mark.parametrize("i", [1, 2, 3, 5])
def test_planted_rows_have_unique_max(i):
    w = W.make_small(i)
    lg = w.logits.numpy()
    for b in range(w.B):
        for j in np.nonzero(w.planted[b])[0]:
            row = lg[b, w.parents[b, j]]
            tok = w.draft_tokens[b, j]
            assert row[tok] == row.max()
            assert (row == row.max()).sum() == 1
        # at most one planted child per parent
        par = w.parents[b][w.planted[b]]
        assert len(set(par.tolist())) == len(par)


def test_bf16_values_are_rounded_normals():
    w = W.make_small(2)
    import torch
    assert w.q.dtype == torch.bfloat16 and w.k_cache.dtype == torch.bfloat16
    x = w.k_cache.float().numpy().ravel()
    assert abs(x.mean()) < 0.01 and abs(x.std() - 1) < 0.01
    lg = w.logits.numpy()
    assert abs(lg.std() - 2.0) < 0.05


@pytest.mark.parametrize("i", [1, 2, 5])
def test_draft_tree_inputs(i):
    """The drafter's scores: seeded and repeatable, [B, depth, topk, V] fp32
    with the workload's spread, root tokens in range, and a stream of their
    own (the rest of the workload does not change when they are drawn)."""
    s = W.SMALL[i]
    depth, topk = W.draft_tree_shape(s)
    a = W.draft_tree_inputs(s, 0)
    b = W.draft_tree_inputs(s, 0)
    c = W.draft_tree_inputs(s, 1)
    lg = a["draft_logits"].numpy()
    assert lg.shape == (s.B, depth, topk, s.V) and lg.dtype == np.float32
    assert np.array_equal(lg, b["draft_logits"].numpy()) and not np.array_equal(lg, c["draft_logits"].numpy())
    assert abs(float(lg.std()) - s.logit_std) < 0.05 * s.logit_std
    r = a["root_tokens"].numpy()
    assert r.shape == (s.B,) and r.min() >= 0 and r.max() < s.V
    assert (a["depth"], a["topk"], a["N"]) == (depth, topk, s.N)
    w0 = W.make_small(i, dense=False)
    w1 = W.make_small(i, dense=False)
    assert np.array_equal(w0.parents, w1.parents) and np.array_equal(w0.logits.numpy(), w1.logits.numpy())
