"""Pins of the CPU oracle against facts that do not come from the oracle.

Each test states the fact it checks: a textbook special case computed by a
library routine (torch's scaled_dot_product_attention in float64), a closed
form, brute force on tiny inputs, or an invariance of the definition.
"""
import itertools
import json
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle as O
import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------- helpers

def rand_case(rng, B=2, N=7, Hq=4, Hkv=2, D=16, bs=4, plo=5, phi=23, tree="uniform"):
    """Small random case with a shuffled paged cache (float64 values)."""
    P = rng.integers(plo, phi + 1, size=B)
    parents = np.zeros((B, N), dtype=np.int64)
    for b in range(B):
        parents[b, 0] = -1
        for i in range(1, N):
            parents[b, i] = i - 1 if tree == "chain" else rng.integers(0, i)
    nblk = (P + N + bs - 1) // bs
    nb = int(nblk.sum()) + 3          # a few unused blocks
    perm = rng.permutation(nb)
    table = np.full((B, int(nblk.max())), -1, dtype=np.int64)
    off = 0
    for b in range(B):
        table[b, :nblk[b]] = perm[off:off + nblk[b]]
        off += nblk[b]
    q = rng.standard_normal((B, N, Hq, D))
    k = rng.standard_normal((nb, Hkv, bs, D))   # [block][head][slot][dim]
    v = rng.standard_normal((nb, Hkv, bs, D))
    return dict(q=q, k=k, v=v, table=table, P=P, parents=parents, bs=bs)


def gather(cache, table_row, positions, bs):
    """[len, Hkv, D] rows of the paged cache ``[block][head][slot][dim]`` at
    logical positions (written here from the paging rule itself,
    independent of the oracle's helpers)."""
    out = []
    for t in positions:
        out.append(cache[table_row[t // bs], :, t % bs])
    return np.stack(out)


def sdpa(qrows, K, V, scale, causal=False):
    """torch's scaled_dot_product_attention in float64: qrows [L, D],
    K/V [S, D]."""
    o = F.scaled_dot_product_attention(
        torch.from_numpy(np.ascontiguousarray(qrows))[None, None],
        torch.from_numpy(np.ascontiguousarray(K))[None, None],
        torch.from_numpy(np.ascontiguousarray(V))[None, None],
        is_causal=causal, scale=scale)
    return o[0, 0].numpy()


def root_paths(parents):
    """Path from the root to every node, by following parents."""
    paths = []
    for i in range(len(parents)):
        p, c = [], i
        while c != -1:
            p.append(c)
            c = parents[c]
        paths.append(p[::-1])
    return paths


def run_attention(c, scale=None, **kw):
    return O.tree_attention(c["q"], c["k"], c["v"], c["table"], c["P"], c["parents"],
                            scale=scale, **kw)


# ---------------------------------------------------------------- tree mask

def test_mask_bits_equal_ancestor_walk():
    """Bit j of node i's mask is set exactly for the nodes met on the walk
    from i up to the root (brute force), for trees with N up to 200 (several
    64-bit words)."""
    rng = np.random.default_rng(1)
    for N in (1, 2, 8, 63, 64, 65, 130, 200):
        par = np.array([-1] + [rng.integers(0, i) for i in range(1, N)])
        anc, depth = O.tree_structure(par)
        words = O.mask_words(anc)
        assert words.shape == (N, (N + 63) // 64)
        for i in range(N):
            walk, c = set(), i
            while c != -1:
                walk.add(c)
                c = par[c]
            bits = {w * 64 + j for w in range(words.shape[1]) for j in range(64)
                    if (int(words[i, w]) >> j) & 1}
            assert bits == walk
            assert depth[i] == len(walk) - 1


def test_invalid_trees_rejected():
    for par in ([0, 0], [-1, 1], [-1, 0, 3, 1], [-1, -1], [-1, 0, 2]):
        assert not O.tree_valid(par)
        with pytest.raises(ValueError):
            O.tree_structure(par)
    assert O.tree_valid([-1]) and O.tree_valid([-1, 0, 1, 0])


# ---------------------------------------------------------------- attention

def test_p1_every_path_equals_causal_decode():
    """Greedy speculative decoding must equal greedy decoding ("vLLM EAGLE
    投机解码实战", 无损性保障).  Per node this means: node i's output equals
    ordinary one-token decode over [prefix ; the tokens on the root-to-i path],
    computed here by torch's SDPA with no mask over exactly those keys."""
    rng = np.random.default_rng(2)
    for _ in range(6):
        c = rand_case(rng)
        out = run_attention(c)
        B, N, Hq, D = c["q"].shape
        g = Hq // c["k"].shape[1]
        for b in range(B):
            P = int(c["P"][b])
            for i, path in enumerate(root_paths(c["parents"][b])):
                pos = list(range(P)) + [P + j for j in path]
                K = gather(c["k"], c["table"][b], pos, c["bs"])
                V = gather(c["v"], c["table"][b], pos, c["bs"])
                for h in range(Hq):
                    ref = sdpa(c["q"][b, i, h][None], K[:, h // g], V[:, h // g], 1 / np.sqrt(D))
                    np.testing.assert_allclose(out[b, i, h], ref[0], rtol=0, atol=1e-12)


def test_p2_chain_equals_causal_attention_over_sequence():
    """A chain tree is ordinary multi-token causal attention: the last N rows
    of causal self-attention over [prefix ; chain] (torch SDPA, is_causal) with
    arbitrary queries at the prefix positions."""
    rng = np.random.default_rng(3)
    c = rand_case(rng, B=3, N=9, Hq=8, Hkv=1, D=32, tree="chain")
    out = run_attention(c)
    B, N, Hq, D = c["q"].shape
    for b in range(B):
        P = int(c["P"][b])
        pos = list(range(P + N))
        K = gather(c["k"], c["table"][b], pos, c["bs"])[:, 0]
        V = gather(c["v"], c["table"][b], pos, c["bs"])[:, 0]
        for h in range(Hq):
            qfull = np.concatenate([rng.standard_normal((P, D)), c["q"][b, :, h]])
            ref = sdpa(qfull, K, V, 1 / np.sqrt(D), causal=True)[P:]
            np.testing.assert_allclose(out[b, :, h], ref, rtol=0, atol=1e-12)


def test_p3_single_node_is_single_token_decode():
    rng = np.random.default_rng(4)
    c = rand_case(rng, B=3, N=1, Hq=6, Hkv=3, D=8)
    out = run_attention(c, scale=0.3)
    for b in range(3):
        P = int(c["P"][b])
        K = gather(c["k"], c["table"][b], range(P + 1), c["bs"])
        V = gather(c["v"], c["table"][b], range(P + 1), c["bs"])
        for h in range(6):
            ref = sdpa(c["q"][b, 0, h][None], K[:, h // 2], V[:, h // 2], 0.3)
            np.testing.assert_allclose(out[b, 0, h], ref[0], rtol=0, atol=1e-12)


def test_p4_zero_query_is_mean_of_visible_values():
    """q = 0 makes every visible score equal, so the output is the plain mean
    of the visible values: P_b prefix rows plus depth(i)+1 tree rows."""
    rng = np.random.default_rng(5)
    c = rand_case(rng, B=2, N=12)
    c["q"][:] = 0
    out = run_attention(c)
    for b in range(2):
        P = int(c["P"][b])
        for i, path in enumerate(root_paths(c["parents"][b])):
            V = gather(c["v"], c["table"][b], list(range(P)) + [P + j for j in path], c["bs"])
            assert V.shape[0] == P + len(path)
            for h in range(4):
                np.testing.assert_allclose(out[b, i, h], V[:, h // 2].mean(0), atol=1e-13)


@pytest.mark.parametrize("P", [3, 200, 4000])
def test_p5_mask_revealing_closed_form(P):
    """Tree keys aligned with the (shared) query give scores of 30 while prefix
    scores are O(1); tree values are one-hot, so node i's output is within
    1e-6 of (1/(depth(i)+1)) * sum of e_j over j in anc*(i).  Any wrong mask
    bit moves an entry by at least 1/(depth+2)."""
    rng = np.random.default_rng(6)
    N, D, bs = 20, 32, 16
    par = np.array([-1] + [rng.integers(0, i) for i in range(1, N)])
    nb = (P + N + bs - 1) // bs
    table = rng.permutation(nb)[None]
    u = rng.standard_normal(D)
    u /= np.linalg.norm(u)
    q = np.tile(u * np.sqrt(D), (1, N, 1, 1))              # scale*q.k = u.k
    k = rng.standard_normal((nb, 1, bs, D))
    v = rng.standard_normal((nb, 1, bs, D))
    for j in range(N):
        t = P + j
        k[table[0, t // bs], 0, t % bs] = 30.0 * u
        v[table[0, t // bs], 0, t % bs] = np.eye(D)[j]
    out = O.tree_attention(q, k, v, table, np.array([P]), par[None])
    anc, depth = O.tree_structure(par)
    for i in range(N):
        expect = anc[i, :].astype(float)
        expect = np.pad(expect, (0, D - N)) / (depth[i] + 1)
        np.testing.assert_allclose(out[0, i, 0], expect, atol=1e-6)


def test_p6_gqa_equals_mha_with_repeated_heads():
    rng = np.random.default_rng(7)
    c = rand_case(rng, Hq=6, Hkv=2)
    out = run_attention(c)
    mha = dict(c)
    mha["k"] = np.repeat(c["k"], 3, axis=1)
    mha["v"] = np.repeat(c["v"], 3, axis=1)
    np.testing.assert_allclose(run_attention(mha), out, rtol=0, atol=1e-13)


def test_p6_block_permutation_is_invisible():
    """Moving physical blocks and rewriting the table leaves results
    bit-identical."""
    rng = np.random.default_rng(8)
    c = rand_case(rng)
    out = run_attention(c)
    nb = c["k"].shape[0]
    perm = rng.permutation(nb)
    c2 = dict(c)
    c2["k"] = np.empty_like(c["k"])
    c2["v"] = np.empty_like(c["v"])
    c2["k"][perm] = c["k"]
    c2["v"][perm] = c["v"]
    c2["table"] = np.where(c["table"] >= 0, perm[np.maximum(c["table"], 0)], -1)
    assert np.array_equal(run_attention(c2), out)


def test_p6_relabelling_nodes_permutes_outputs():
    """Another topological numbering of the same tree (with each node's K/V
    moved to its new slot) permutes the outputs and nothing else."""
    rng = np.random.default_rng(9)
    c = rand_case(rng, B=1, N=10, bs=4)
    par = c["parents"][0]
    N, P, bs = 10, int(c["P"][0]), c["bs"]
    out = run_attention(c)
    # random topological order
    order, avail = [0], [i for i in range(1, N) if par[i] == 0]
    while avail:
        x = avail.pop(rng.integers(len(avail)))
        order.append(x)
        avail += [i for i in range(N) if par[i] == x]
    pos = np.empty(N, dtype=int)
    pos[order] = np.arange(N)
    par2 = np.array([-1] + [pos[par[o]] for o in order[1:]])
    c2 = dict(c)
    c2["parents"] = par2[None]
    c2["q"] = c["q"][:, order]
    c2["k"] = c["k"].copy()
    c2["v"] = c["v"].copy()
    for o in range(N):
        src, dst = P + o, P + pos[o]
        for name in ("k", "v"):
            c2[name][c["table"][0, dst // bs], :, dst % bs] = c[name][c["table"][0, src // bs], :, src % bs]
    out2 = run_attention(c2)
    np.testing.assert_allclose(out2[0, pos], out[0], rtol=0, atol=1e-13)


def test_p12_weights_sum_to_one_and_output_in_hull():
    rng = np.random.default_rng(10)
    c = rand_case(rng, B=2, N=9, D=8)
    out, wts = run_attention(c, return_weights=True)
    g = 2
    for (b, kh), (w, vis) in wts.items():
        np.testing.assert_allclose(w.sum(1), 1.0, atol=1e-12)
        assert (w[~vis] == 0).all() and (w[vis] > 0).all()
        P = int(c["P"][b])
        V = gather(c["v"], c["table"][b], range(P + 9), c["bs"])[:, kh]
        for r in range(w.shape[0]):
            Vv = V[vis[r]]
            o = out[b, r // g, kh * g + r % g]
            assert (o >= Vv.min(0) - 1e-12).all() and (o <= Vv.max(0) + 1e-12).all()


def test_seqs_subset_matches_full():
    rng = np.random.default_rng(11)
    c = rand_case(rng, B=4)
    full = run_attention(c)
    part = run_attention(c, seqs=[1, 3])
    assert np.array_equal(part[[1, 3]], full[[1, 3]])
    assert np.isnan(part[[0, 2]]).all()


# ---------------------------------------------------------------- acceptance

def brute_argmax(row):
    """Lowest index among the row's maxima, by a plain scan."""
    best = 0
    for x in range(1, len(row)):
        if row[x] > row[best]:
            best = x
    return best


def brute_accept(am, draft, parents):
    """Longest root path whose every edge is accepted, smallest node sequence
    on ties, by enumerating every node's root path."""
    best = None
    for path in root_paths(parents):
        if all(draft[path[k + 1]] == am[path[k]] for k in range(len(path) - 1)):
            key = (-len(path), path)
            if best is None or key < best:
                best = key
    return best[1]


def test_p7_acceptance_equals_brute_force():
    rng = np.random.default_rng(12)
    for trial in range(400):
        N = int(rng.integers(1, 12))
        V = int(rng.integers(2, 5))         # tiny vocab: many matches and shared sibling tokens
        par = np.array([-1] + [rng.integers(0, i) for i in range(1, N)])
        draft = rng.integers(0, V, size=N)
        logits = rng.integers(-2, 3, size=(1, N, V)).astype(np.float32)  # many exact ties
        res = O.accept_greedy(logits, draft[None], par[None])
        am = [brute_argmax(logits[0, i]) for i in range(N)]
        assert list(res["argmax"][0]) == am
        path = brute_accept(am, draft, par)
        L = len(path)
        assert res["accept_len"][0] == L - 1
        assert list(res["accepted_nodes"][0, :L]) == path
        assert (res["accepted_nodes"][0, L:] == -1).all()
        assert res["bonus"][0] == am[path[-1]]


def test_p8_all_match_all_miss_single_node():
    rng = np.random.default_rng(13)
    for _ in range(50):
        N, V = int(rng.integers(2, 40)), 50
        par = np.array([-1] + [rng.integers(0, i) for i in range(1, N)])
        draft = np.zeros(N, dtype=int)
        for p in range(N):
            kids = np.nonzero(par == p)[0]
            draft[kids] = rng.choice(V, size=len(kids), replace=False)
        _, depth = O.tree_structure(par)
        # all-match: every row's argmax is the token of the lowest-index child on
        # a deepest path through it
        deepest = depth.max()
        best_child = {}
        for leaf in sorted(np.nonzero(depth == deepest)[0]):
            path = root_paths(par)[leaf]
            for a, c in zip(path[:-1], path[1:]):
                best_child.setdefault(a, c)
        logits = rng.standard_normal((1, N, V)).astype(np.float32)
        for a, c in best_child.items():
            logits[0, a, draft[c]] = 10.0
        res = O.accept_greedy(logits, draft[None], par[None])
        assert res["accept_len"][0] == deepest
        # all-miss: every row's argmax is a token no child carries
        miss = np.full((1, N, V), -1.0, dtype=np.float32)
        for a in range(N):
            used = set(draft[par == a].tolist())
            free = [x for x in range(V) if x not in used]
            miss[0, a, free[0]] = 1.0
        res = O.accept_greedy(miss, draft[None], par[None])
        assert res["accept_len"][0] == 0
        assert res["bonus"][0] == brute_argmax(miss[0, 0])
        assert list(res["accepted_nodes"][0]) == [0] + [-1] * (N - 1)
    one = O.accept_greedy(np.array([[[0.5, 2.0, 1.0]]], dtype=np.float32), np.array([[1]]),
                          np.array([[-1]]))
    assert one["accept_len"][0] == 0 and one["bonus"][0] == 1


def test_p9_chain_acceptance_length_is_truncated_geometric():
    """Chain workload: a draft is accepted iff all earlier ones were and its own
    Bernoulli(0.7) draw succeeds, so accept_len is geometric truncated at K=8
    with mean sum_{j=1..8} 0.7^j = 2.1991; the 128-sequence sample mean lies
    within 3 standard errors."""
    w = W.make_config(5, dense=False)
    res = O.accept_greedy(w.logits.numpy(), w.draft_tokens, w.parents)
    p, K = 0.7, 8
    probs = np.array([p ** j * (1 - p) for j in range(K)] + [p ** K])
    mean = float((np.arange(K + 1) * probs).sum())
    assert abs(mean - sum(p ** j for j in range(1, K + 1))) < 1e-12
    sd = float(np.sqrt(((np.arange(K + 1) - mean) ** 2 * probs).sum()))
    assert abs(res["accept_len"].mean() - mean) < 3 * sd / np.sqrt(w.B)
    # and it is exactly the planted prefix of every chain
    for b in range(w.B):
        k = 0
        while k + 1 < w.N and w.planted[b, k + 1]:
            k += 1
        assert res["accept_len"][b] == k


def test_p10_argmax_ties_signed_zero_and_ends():
    rows = np.array([
        [1.0, 3.0, 3.0, 2.0],          # tie -> 1
        [-0.0, 0.0, -1.0, -2.0],       # -0 == +0 -> 0
        [0.0, -0.0, -1.0, -2.0],       # -> 0
        [-5.0, -4.0, -3.0, 7.0],       # max at V-1
        [9.0, 9.0, 9.0, 9.0],          # all equal -> 0
        [-np.inf, -1e30, -1e30, -3.0],  # -> 3
    ], dtype=np.float32)
    am = O.target_argmax(rows[None])[0]
    assert list(am) == [1, 0, 0, 3, 0, 3]
    assert list(am) == [brute_argmax(r) for r in rows]


def test_workload_acceptance_matches_planting():
    """On the generated trees every planted child whose parent lies on the
    accepted path extends it; the path ends where no child of the last node is
    planted (sibling tokens are distinct and planted maxima are unique)."""
    for i in (1, 2, 3):
        w = W.make_small(i, dense=False)
        res = O.accept_greedy(w.logits.numpy(), w.draft_tokens, w.parents)
        for b in range(w.B):
            L = res["accept_len"][b] + 1
            path = res["accepted_nodes"][b, :L]
            for a, c in zip(path[:-1], path[1:]):
                assert w.parents[b, c] == a and w.planted[b, c]
            assert not any(w.planted[b, c] for c in range(w.N) if w.parents[b, c] == path[-1])


# ---------------------------------------------------------------- compaction

def test_p11_compaction_equals_per_row_copies_bit_exact():
    rng = np.random.default_rng(14)
    for _ in range(30):
        c = rand_case(rng, B=3, N=9, bs=4)
        k16 = rng.integers(0, 65536, size=c["k"].shape).astype(np.uint16)   # raw bf16 bytes
        v16 = rng.integers(0, 65536, size=c["v"].shape).astype(np.uint16)
        paths, alen = np.full((3, 9), -1), np.zeros(3, dtype=int)
        for b in range(3):
            leaf = int(rng.integers(0, 9))
            p = root_paths(c["parents"][b])[leaf]
            paths[b, :len(p)] = p
            alen[b] = len(p) - 1
        kn, vn, nl = O.kv_compact(k16, v16, c["table"], c["P"], paths, alen)
        # brute force: element-by-element copies from a snapshot
        kb, vb = k16.copy(), v16.copy()
        bs = c["bs"]
        for b in range(3):
            P = int(c["P"][b])
            for j in range(alen[b] + 1):
                s, d = P + paths[b, j], P + j
                for hh in range(k16.shape[1]):
                    for e in range(k16.shape[3]):
                        kb[c["table"][b, d // bs], hh, d % bs, e] = k16[c["table"][b, s // bs], hh, s % bs, e]
                        vb[c["table"][b, d // bs], hh, d % bs, e] = v16[c["table"][b, s // bs], hh, s % bs, e]
        assert np.array_equal(kn, kb) and np.array_equal(vn, vb)
        assert list(nl) == list(c["P"] + alen + 1)


def test_p11_overlapping_moves_gather_before_write():
    """Path [0, 2, 3]: slot 2 is both a source (for 1) and a destination (from
    3); the gather-then-write order makes slot 1 hold node 2's old row."""
    k = np.arange(8, dtype=np.float64).reshape(2, 1, 4, 1)     # 2 blocks of 4 rows, 1 head
    table = np.array([[0, 1]])
    kn, _, nl = O.kv_compact(k, k, table, np.array([2]), np.array([[0, 2, 3, -1]]), np.array([2]))
    flat = kn.reshape(-1)
    assert list(flat) == [0, 1, 2, 4, 5, 5, 6, 7]
    assert nl[0] == 5


def test_p11_decode_after_compaction_equals_decode_over_accepted_sequence():
    """After compaction, a new query over the first P + L positions sees the
    prefix followed by the accepted nodes' K/V -- exactly causal decode over
    prefix + accepted tokens."""
    rng = np.random.default_rng(15)
    c = rand_case(rng, B=2, N=8, Hq=2, Hkv=1, D=8, bs=4)
    for b in range(2):
        leaf = int(rng.integers(1, 8))
        path = root_paths(c["parents"][b])[leaf]
        nodes = np.full((2, 8), -1)
        nodes[b, :len(path)] = path
        alen = np.zeros(2, dtype=int)
        alen[b] = len(path) - 1
        kn, vn, nl = O.kv_compact(c["k"], c["v"], c["table"], c["P"], nodes, alen)
        P = int(c["P"][b])
        pos_new = list(range(nl[b]))
        pos_old = list(range(P)) + [P + j for j in path]
        qn = rng.standard_normal(8)
        a = sdpa(qn[None], gather(kn, c["table"][b], pos_new, 4)[:, 0],
                 gather(vn, c["table"][b], pos_new, 4)[:, 0], 0.35)
        r = sdpa(qn[None], gather(c["k"], c["table"][b], pos_old, 4)[:, 0],
                 gather(c["v"], c["table"][b], pos_old, 4)[:, 0], 0.35)
        assert np.array_equal(a, r)


# ---------------------------------------------------------------- status bits

def test_input_status_bits():
    par = np.array([[-1, 0, 1], [-1, 0, 0]])
    table = np.array([[0, 1], [2, 3]])
    P = np.array([20, 10])
    ok = O.input_status(par, table, P, 4, 20, 16, np.array([[0, 1, 2], [5, 6, 7]]), 8)
    assert ok == 0
    assert O.input_status(np.array([[-1, 0, 2], [-1, 0, 0]])) == O.ST_BAD_TREE
    assert O.input_status(par, np.array([[0, 4], [2, 3]]), P, 4, 20) == O.ST_BAD_CACHE
    assert O.input_status(par, table, P, 4, 19) == O.ST_BAD_CACHE
    assert O.input_status(par, table, P, 4, 20, 16, np.array([[0, 1, 8], [9, 6, 7]]), 8) == O.ST_BAD_TOKEN


# ---------------------------------------------------------------- golden fixtures

def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def test_golden_attention_hand_worked():
    g = _load("attention_hand_worked.json")
    for case in g["cases"]:
        bs = case["block_size"]
        # the fixtures list each block's rows as [slot][head][dim]; the cache
        # layout is [block][head][slot][dim]
        k = np.array(case["k_cache"], dtype=np.float64).transpose(0, 2, 1, 3)
        v = np.array(case["v_cache"], dtype=np.float64).transpose(0, 2, 1, 3)
        out = O.tree_attention(np.array(case["q"], dtype=np.float64), k, v,
                               np.array(case["block_table"]), np.array(case["prefix_lens"]),
                               np.array(case["parents"]), scale=case["scale"])
        expect = np.array([[eval(x) if isinstance(x, str) else x for x in row]
                           for row in case["expected_out_node_major"]], dtype=np.float64)
        np.testing.assert_allclose(out[0, :, 0, :], expect, rtol=0, atol=1e-12)


def test_golden_acceptance_hand_worked():
    g = _load("acceptance_hand_worked.json")
    for case in g["cases"]:
        res = O.accept_greedy(np.array(case["logits"], dtype=np.float32)[None],
                              np.array(case["draft_tokens"])[None], np.array(case["parents"])[None])
        assert list(res["argmax"][0]) == case["expected_argmax"]
        assert res["accept_len"][0] == case["expected_accept_len"]
        assert list(res["accepted_nodes"][0]) == case["expected_accepted_nodes"]
        assert res["bonus"][0] == case["expected_bonus"]


# ---------------------------------------------------------------- tree K/V write (rotary positions)

def _complex_rope(x, m, theta):
    """Rotary embedding written as complex multiplication: pair j forms
    z_j = x[j] + i x[j + D/2], rotated to z_j * exp(i m / theta**(2 j / D))."""
    x = np.asarray(x, dtype=np.float64)
    h = x.shape[-1] // 2
    z = x[..., :h] + 1j * x[..., h:]
    w = np.exp(1j * m / np.power(float(theta), np.arange(0, x.shape[-1], 2) / x.shape[-1]))
    r = z * w
    return np.concatenate([r.real, r.imag], axis=-1)


def test_rope_equals_complex_rotation():
    rng = np.random.default_rng(31)
    for D, theta in ((2, 1.0), (8, 100.0), (64, 10000.0), (128, 500000.0)):
        x = rng.standard_normal((5, D))
        for m in (0, 1, 7, 2048, 32775):
            np.testing.assert_allclose(O.rope(x, np.full(5, m), theta), _complex_rope(x, m, theta),
                                       rtol=0, atol=1e-9)


def test_rope_known_angles():
    """D = 4, theta = 10000: pair 0 turns by m radians, pair 1 by m / 100
    (theta ** (-2/4)); pairs are (0, 2) and (1, 3)."""
    e = np.eye(4)
    r = O.rope(e, np.full(4, 100), 10000.0)
    np.testing.assert_allclose(r[0], [np.cos(100.0), 0, np.sin(100.0), 0], atol=1e-12)
    np.testing.assert_allclose(r[1], [0, np.cos(1.0), 0, np.sin(1.0)], atol=1e-12)
    np.testing.assert_allclose(r[2], [-np.sin(100.0), 0, np.cos(100.0), 0], atol=1e-12)


def test_rope_identity_norm_relative_and_composition():
    rng = np.random.default_rng(32)
    D, theta = 32, 10000.0
    q, k = rng.standard_normal(D), rng.standard_normal(D)
    assert np.array_equal(O.rope(q, 0, theta), q)
    h = D // 2
    r = O.rope(q, 12345, theta)
    np.testing.assert_allclose(r[:h] ** 2 + r[h:] ** 2, q[:h] ** 2 + q[h:] ** 2, rtol=1e-12)
    for m, n in ((5, 3), (100, 2000), (32768, 7)):
        lhs = O.rope(q, m, theta) @ O.rope(k, n, theta)
        rhs = O.rope(q, m - n, theta) @ k
        assert abs(lhs - rhs) < 1e-9 * (1 + abs(rhs))
    np.testing.assert_allclose(O.rope(O.rope(q, 700, theta), 333, theta), O.rope(q, 1033, theta),
                               rtol=0, atol=1e-9)


def test_tree_positions_brute_force():
    rng = np.random.default_rng(33)
    B, N = 4, 12
    par = np.zeros((B, N), dtype=np.int64)
    for b in range(B):
        par[b, 0] = -1
        for i in range(1, N):
            par[b, i] = rng.integers(0, i)
    P = rng.integers(0, 50, size=B)
    pos = O.tree_positions(par, P)
    for b in range(B):
        for i in range(N):
            d, c = 0, i
            while c != 0:
                c = par[b, c]
                d += 1
            assert pos[b, i] == P[b] + d
    # a chain gets consecutive positions; siblings share one
    chain = np.array([[-1, 0, 1, 2, 3]])
    assert list(O.tree_positions(chain, [10])[0]) == [10, 11, 12, 13, 14]
    star = np.array([[-1, 0, 0, 0]])
    assert list(O.tree_positions(star, [7])[0]) == [7, 8, 8, 8]


def test_tree_kv_write_path_equals_causal_rope_attention():
    """After the write, every root-to-leaf path attends exactly as causal
    decoding with RoPE at consecutive positions over [prefix ; path]: scores
    of rotated pairs depend only on the position difference."""
    rng = np.random.default_rng(34)
    B, N, Hq, Hkv, D, theta = 1, 7, 2, 1, 16, 10000.0
    par = np.array([[-1, 0, 0, 1, 1, 2, 4]])
    P = 5
    q = rng.standard_normal((B, N, Hq, D))
    k_new = rng.standard_normal((B, N, Hkv, D))
    kpre = O.rope(rng.standard_normal((P, Hkv, D)), np.arange(P)[:, None], theta)
    q_rot, k_rot, pos = O.tree_kv_write(q, k_new, par, np.array([P]), theta)
    for i, path in enumerate(root_paths(par[0])):
        # causal decode of [prefix ; path]: token t sits at position t
        keys = np.concatenate([kpre, O.rope(k_new[0, path], np.arange(P, P + len(path))[:, None], theta)])
        qd = O.rope(q[0, i], P + len(path) - 1, theta)
        tree_keys = np.concatenate([kpre, k_rot[0, path]])
        np.testing.assert_allclose(q_rot[0, i] @ tree_keys[:, 0].T, qd @ keys[:, 0].T, rtol=0, atol=1e-9)
