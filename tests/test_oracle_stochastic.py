"""Pins of the oracle's stochastic acceptance (CPU only).

The rule under test: children of the current node are tested in index order,
child c (token x, proposal q) is accepted iff u_c * q(x) < r(x), a rejection
replaces r by the normalised positive part of r - q, and the bonus token is
the largest r[v] / E[v] over the vocabulary ("P-EAGLE" page, 技术原理和实现方式
steps 3-4; "vLLM EAGLE 投机解码实战", 无损性保障: the sampler must converge to
the target distribution).

The pins do not restate that rule.  They check what the mathematics fixes:
hand-worked examples, the zero-temperature limit (greedy acceptance), the
distribution of the emitted tokens (it must be the target's, whatever the
proposals), the textbook acceptance rate 1 - TV(p, q) of a single proposal,
and the distribution of the bonus token after a rejection.
"""
import numpy as np
import pytest

import oracle as O
import workloads as W


def softmax(z):
    e = np.exp(z - z.max())
    return e / e.sum()


def first_token(path, bonus, tokens):
    return int(tokens[path[1]]) if len(path) > 1 else int(bonus)


# ---------------------------------------------------------------------------
# hand-worked examples
# ---------------------------------------------------------------------------

def test_worked_example_point_mass_proposals():
    # V = 4, T = 1, rows given as log-probabilities so that softmax returns
    # them.  Root 0 has children 1 (token 1), 2 (token 0), 3 (token 3); node 2
    # has child 4 (token 2).
    p0 = np.array([0.5, 0.2, 0.2, 0.1])
    p2 = np.array([0.1, 0.3, 0.4, 0.2])
    logits = np.log(np.stack([p0, p0, p2, p0, p0]))
    parents = np.array([-1, 0, 0, 0, 2])
    tokens = np.array([0, 1, 0, 3, 2])
    # node 1: 0.5 < p0[1] = 0.2 fails -> rejected; token 1 leaves the
    #   distribution: r = [0.5, 0, 0.2, 0.1] / 0.8 = [0.625, 0, 0.25, 0.125]
    # node 2: 0.6 < r[0] = 0.625 holds -> accepted (node 3, whose 0.05 would
    #   also pass, is never tested)
    # node 4: 0.45 < p2[2] = 0.4 fails -> rejected; r = [0.1, 0.3, 0, 0.2] / 0.6
    # bonus: r / E = [1/6 / 0.1, 0.5 / 1, 0, 1/3 / 0.5] = [1.67, 0.5, 0, 0.67]
    #   -> token 0 (token 2 would win with 0.4 / 0.01 if it had not been removed)
    u = np.array([0.0, 0.5, 0.6, 0.05, 0.45])
    expo = np.array([0.1, 1.0, 0.01, 0.5])
    path, bonus, margin = O.stochastic_walk(logits, tokens, parents, 1.0, u, expo)
    assert path == [0, 2]
    assert bonus == 0
    # the closest call was node 2: |0.6 - 0.625| / 0.625 = 0.04
    assert margin == pytest.approx(0.04, rel=1e-9)


def test_worked_example_proposal_distribution():
    # chain 0 -> 1, token 2 drawn from q = [0.1, 0.1, 0.6, 0.2]; target at the
    # root p0 = [0.5, 0.2, 0.2, 0.1].
    p0 = np.array([0.5, 0.2, 0.2, 0.1])
    q = np.array([0.1, 0.1, 0.6, 0.2])
    logits = np.log(np.stack([p0, p0]))
    parents = np.array([-1, 0])
    tokens = np.array([0, 2])
    probs = np.stack([np.full(4, 0.25), q])
    # acceptance needs u * 0.6 < 0.2, i.e. u < 1/3
    path, _, _ = O.stochastic_walk(logits, tokens, parents, 1.0, np.array([0.0, 0.33]),
                                   np.ones(4), probs)
    assert path == [0, 1]
    # u = 0.4 rejects; the rest of the choice is max(p0 - q, 0) / 0.5 =
    # [0.8, 0.2, 0, 0]; with E = [2, 0.1, 0.001, 0.001] the ratios are
    # [0.4, 2, 0, 0] -> token 1 (tokens 2 and 3 have no mass left)
    path, bonus, _ = O.stochastic_walk(logits, tokens, parents, 1.0, np.array([0.0, 0.4]),
                                       np.array([2.0, 0.1, 0.001, 0.001]), probs)
    assert path == [0]
    assert bonus == 1


def test_threshold_sits_at_the_target_probability():
    rng = np.random.default_rng(5)
    V, T = 9, 0.7
    logits = rng.normal(size=(2, V)) * 2
    parents = np.array([-1, 0])
    x = 4
    tokens = np.array([0, x])
    p = softmax(logits[0] / T)[x]
    q_big = 0.5 * rng.dirichlet(np.ones(V)) + 0.5 * np.eye(V)[x]
    for q_row, thr in ((None, p), (q_big, None)):
        probs = None
        if q_row is not None:
            probs = np.stack([np.full(V, 1.0 / V), q_row])
            thr = p / q_row[x]
        assert thr < 1
        below = O.stochastic_walk(logits, tokens, parents, T, np.array([0.0, thr * (1 - 1e-9)]),
                                  np.ones(V), probs)[0]
        above = O.stochastic_walk(logits, tokens, parents, T, np.array([0.0, thr * (1 + 1e-9)]),
                                  np.ones(V), probs)[0]
        assert below == [0, 1] and above == [0]


def test_race_draw_hand_values():
    i, gap = O.race_draw(np.array([0.5, 0.3, 0.2]), np.array([1.0, 0.5, 0.1]))
    assert i == 2 and gap == pytest.approx((2.0 - 0.6) / 2.0)
    # equal ratios: the first index wins
    assert O.race_draw(np.array([0.2, 0.4, 0.4]), np.array([1.0, 2.0, 2.0]))[0] == 0


# ---------------------------------------------------------------------------
# zero-temperature limit: greedy acceptance
# ---------------------------------------------------------------------------

def _separated_logits(rng, shape, gap=0.05):
    """Rows whose largest entry leads the second by at least ``gap``."""
    x = rng.normal(size=shape) * 2
    srt = np.sort(x, axis=-1)
    lead = srt[..., -1] - srt[..., -2]
    am = np.argmax(x, axis=-1)
    bump = np.maximum(gap - lead, 0)
    np.put_along_axis(x, am[..., None], (srt[..., -1] + bump)[..., None], axis=-1)
    return x


@pytest.mark.parametrize("cfg", [2, 3, 4, 5])
def test_zero_temperature_is_greedy(cfg):
    w = W.make_small(cfg, logits=False)
    rng = np.random.default_rng(cfg)
    B, N, V = w.spec.B, w.spec.N, w.spec.V
    lg = _separated_logits(rng, (B, N, V))
    tok = w.draft_tokens.copy()
    # per node, the child with the tallest subtree carries the greedy choice
    # and its siblings carry other, distinct tokens (then the first accepted
    # child is the only one carrying the parent's choice)
    for b in range(B):
        par = w.parents[b]
        height = np.zeros(N, dtype=int)
        for c in range(N - 1, 0, -1):
            height[par[c]] = max(height[par[c]], height[c] + 1)
        for p in range(N):
            kids = [c for c in range(1, N) if par[c] == p]
            if not kids:
                continue
            am = int(np.argmax(lg[b, p]))
            best = max(kids, key=lambda c: height[c])
            seen = {am}
            tok[b, best] = am
            for c in kids:
                if c == best:
                    continue
                while int(tok[b, c]) in seen:
                    tok[b, c] = (int(tok[b, c]) + 1) % V
                seen.add(int(tok[b, c]))
    u = rng.random((B, N))
    expo = rng.exponential(size=(B, V))
    g = O.accept_greedy(lg, tok, w.parents)
    s = O.accept_stochastic(lg, tok, w.parents, 1e-4, u, expo)
    np.testing.assert_array_equal(s["accept_len"], g["accept_len"])
    np.testing.assert_array_equal(s["accepted_nodes"], g["accepted_nodes"])
    np.testing.assert_array_equal(s["bonus"], g["bonus"])
    if cfg == 5:
        # chains with sampled proposals reach the same limit
        probs = rng.dirichlet(np.ones(V) * 0.3, size=(B, N))
        s2 = O.accept_stochastic(lg, tok, w.parents, 1e-4, u, expo, probs)
        np.testing.assert_array_equal(s2["accepted_nodes"], g["accepted_nodes"])
        np.testing.assert_array_equal(s2["bonus"], g["bonus"])
    assert g["accept_len"].min() >= 2


# ---------------------------------------------------------------------------
# distribution of the emitted tokens
# ---------------------------------------------------------------------------

TRIALS = 48000


def _assert_matches(counts, p, trials, what):
    emp = counts / trials
    sd = np.sqrt(p * (1 - p) / trials) + 1e-12
    z = np.abs(emp - p) / sd
    assert z.max() < 5.0, f"{what}: empirical {np.round(emp, 4)} vs {np.round(p, 4)} (max z {z.max():.1f})"


def test_first_token_follows_target_point_mass_siblings():
    # four siblings, two of them carrying the same token
    rng = np.random.default_rng(11)
    V, T = 6, 0.5
    logits = rng.normal(size=(5, V))
    parents = np.array([-1, 0, 0, 0, 0])
    tokens = np.array([0, 2, 4, 2, 0])
    p0 = softmax(logits[0] / T)
    counts = np.zeros(V)
    for _ in range(TRIALS):
        path, bonus, _ = O.stochastic_walk(logits, tokens, parents, T, rng.random(5),
                                           rng.exponential(size=V))
        counts[first_token(path, bonus, tokens)] += 1
    _assert_matches(counts, p0, TRIALS, "point-mass siblings")


def test_first_token_follows_target_sampled_siblings():
    # three siblings, each token drawn from its own proposal distribution
    rng = np.random.default_rng(12)
    V, T = 6, 0.5
    logits = rng.normal(size=(4, V))
    parents = np.array([-1, 0, 0, 0])
    probs = rng.dirichlet(np.ones(V), size=4)
    p0 = softmax(logits[0] / T)
    counts = np.zeros(V)
    for _ in range(TRIALS):
        tokens = np.array([0] + [rng.choice(V, p=probs[c]) for c in (1, 2, 3)])
        path, bonus, _ = O.stochastic_walk(logits, tokens, parents, T, rng.random(4),
                                           rng.exponential(size=V), probs)
        counts[first_token(path, bonus, tokens)] += 1
    _assert_matches(counts, p0, TRIALS, "sampled siblings")


def test_second_token_follows_target_after_acceptance():
    # chain 0 -> 1 -> 2 with sampled proposals: given that node 1 was accepted,
    # the next emitted token follows node 1's target row
    rng = np.random.default_rng(13)
    V, T = 5, 0.6
    logits = rng.normal(size=(3, V)) * 1.5
    parents = np.array([-1, 0, 1])
    probs = rng.dirichlet(np.ones(V) * 2, size=3)
    p1 = softmax(logits[1] / T)
    counts = np.zeros(V)
    n = 0
    for _ in range(TRIALS):
        tokens = np.array([0, rng.choice(V, p=probs[1]), rng.choice(V, p=probs[2])])
        path, bonus, _ = O.stochastic_walk(logits, tokens, parents, T, rng.random(3),
                                           rng.exponential(size=V), probs)
        if len(path) >= 2:
            n += 1
            counts[int(tokens[2]) if len(path) == 3 else bonus] += 1
    assert n > TRIALS // 4
    _assert_matches(counts, p1, n, "second token")


def test_acceptance_rate_and_residual_of_one_proposal():
    # textbook single-proposal facts: x ~ q is accepted with probability
    # sum_x min(p(x), q(x)) = 1 - TV(p, q); after a rejection the bonus
    # follows max(p - q, 0) / TV(p, q)
    rng = np.random.default_rng(14)
    V, T = 5, 0.8
    logits = rng.normal(size=(2, V)) * 1.5
    parents = np.array([-1, 0])
    q = rng.dirichlet(np.ones(V))
    probs = np.stack([np.full(V, 1.0 / V), q])
    p = softmax(logits[0] / T)
    tv = 0.5 * np.abs(p - q).sum()
    acc = 0
    counts = np.zeros(V)
    for _ in range(TRIALS):
        tokens = np.array([0, rng.choice(V, p=q)])
        path, bonus, _ = O.stochastic_walk(logits, tokens, parents, T, rng.random(2),
                                           rng.exponential(size=V), probs)
        if len(path) == 2:
            acc += 1
        else:
            counts[bonus] += 1
    rate = 1 - tv
    assert abs(acc / TRIALS - rate) < 5 * np.sqrt(rate * (1 - rate) / TRIALS)
    _assert_matches(counts, np.maximum(p - q, 0) / tv, TRIALS - acc, "residual")


def test_proposal_equal_to_target_is_always_accepted():
    rng = np.random.default_rng(15)
    V, N, T = 50, 7, 0.9
    logits = rng.normal(size=(N, V))
    parents = np.arange(-1, N - 1)
    probs = np.stack([O.target_probs(logits[max(c - 1, 0)], T) for c in range(N)])
    for _ in range(50):
        tokens = np.array([0] + [rng.choice(V, p=probs[c]) for c in range(1, N)])
        u = rng.random(N) * (1 - 1e-12)
        path, _, _ = O.stochastic_walk(logits, tokens, parents, T, u, rng.exponential(size=V), probs)
        assert path == list(range(N))


def test_rejected_tokens_never_come_back_as_bonus():
    rng = np.random.default_rng(16)
    V, T = 8, 1.0
    logits = rng.normal(size=(4, V)) * 0.3
    parents = np.array([-1, 0, 0, 0])
    tokens = np.array([0, 1, 5, 6])
    for _ in range(400):
        u = np.array([0.0, 0.999, 0.999, 0.999])   # every p(x) here is below 0.99
        path, bonus, _ = O.stochastic_walk(logits, tokens, parents, T, u, rng.exponential(size=V))
        assert path == [0] and bonus not in (1, 5, 6)


# ---------------------------------------------------------------------------
# batch wrapper, invalid input, status bits
# ---------------------------------------------------------------------------

def test_batch_wrapper_and_invalid_sequences():
    rng = np.random.default_rng(17)
    B, N, V, T = 3, 5, 12, 0.7
    logits = rng.normal(size=(B, N, V))
    parents = np.tile(np.array([-1, 0, 0, 1, 1]), (B, 1))
    tokens = rng.integers(0, V, (B, N))
    parents[1, 3] = 3          # not a tree
    tokens[2, 4] = V           # token out of range
    u = rng.random((B, N))
    expo = rng.exponential(size=(B, V))
    out = O.accept_stochastic(logits, tokens, parents, T, u, expo)
    one = O.stochastic_walk(logits[0], tokens[0], parents[0], T, u[0], expo[0])
    assert out["accepted_nodes"][0][:len(one[0])].tolist() == one[0] and out["bonus"][0] == one[1]
    for b in (1, 2):
        assert out["accept_len"][b] == 0 and out["accepted_nodes"][b].tolist() == [0] + [-1] * (N - 1)
        assert out["bonus"][b] == int(np.argmax(softmax(logits[b, 0] / T) / expo[b]))
    st = O.input_status(parents, draft_tokens=tokens, V=V)
    assert st == O.ST_BAD_TREE | O.ST_BAD_TOKEN


def test_status_bits_for_random_inputs_and_chains():
    par = np.array([[-1, 0, 1, 2], [-1, 0, 0, 1]])
    u = np.full((2, 4), 0.5)
    e = np.ones((2, 7))
    assert O.input_status(par, uniforms=u, expo=e) == 0
    u[1, 2] = 1.0
    assert O.input_status(par, uniforms=u, expo=e) == O.ST_BAD_RANDOM
    u[1, 2] = 0.5
    u[0, 0] = 7.0              # the root's entry is never used
    assert O.input_status(par, uniforms=u, expo=e) == 0
    for bad in (0.0, -1.0, np.inf, np.nan):
        e2 = e.copy()
        e2[0, 3] = bad
        assert O.input_status(par, uniforms=u, expo=e2) == O.ST_BAD_RANDOM
    assert O.input_status(par, proposal_rows=True) == O.ST_UNSUPPORTED
    assert O.input_status(par[:1], proposal_rows=True) == 0
