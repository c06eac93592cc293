"""Pins of the oracle's fused LM head -> greedy choice (CPU only).

The oracle projects every row's final hidden state onto every vocabulary
row and takes the lowest index among the maxima ("P-EAGLE" page, 技术原理和
实现方式 step 3; "vLLM EAGLE 投机解码实战", 无损性保障).  The pins check it
against plain loops, special weights whose answer is known, invariances, and
the tie rule.
"""
import numpy as np

import oracle as O
import workloads as W


def test_brute_force_dot_products():
    rng = np.random.default_rng(1)
    M, H, V = 3, 8, 11
    h = rng.normal(size=(M, H))
    w = rng.normal(size=(V, H))
    am, mx = O.lm_head_argmax(h, w)
    for m in range(M):
        scores = []
        for v in range(V):
            acc = 0.0
            for k in range(H):
                acc += h[m, k] * w[v, k]
            scores.append(acc)
        best = max(range(V), key=lambda v: (scores[v], -v))
        assert am[m] == best
        assert abs(mx[m] - scores[best]) < 1e-12


def test_identity_weight_returns_the_hidden_argmax():
    rng = np.random.default_rng(2)
    h = rng.normal(size=(5, 16))
    am, mx = O.lm_head_argmax(h, np.eye(16))
    np.testing.assert_array_equal(am, np.argmax(h, axis=1))
    np.testing.assert_allclose(mx, h.max(axis=1), rtol=0, atol=0)


def test_aligned_row_wins():
    # a vocabulary row parallel to the hidden state and longer than every
    # other row wins (Cauchy-Schwarz)
    rng = np.random.default_rng(3)
    M, H, V = 4, 32, 50
    h = rng.normal(size=(M, H))
    w = rng.normal(size=(V, H))
    w /= np.linalg.norm(w, axis=1, keepdims=True)
    targets = [7, 0, 49, 23]
    for m, t in enumerate(targets):
        w[t] = 1.5 * h[m] / np.linalg.norm(h[m])
    # every other row scores at most 1.5 |h| with equality only when parallel
    # to h (unit rows score at most |h|), so the planted row wins strictly
    am, mx = O.lm_head_argmax(h, w)
    for m, t in enumerate(targets):
        assert am[m] == t
        assert abs(mx[m] - 1.5 * np.linalg.norm(h[m])) < 1e-9


def test_permutation_and_scale_invariance():
    rng = np.random.default_rng(4)
    h = rng.normal(size=(6, 24))
    w = rng.normal(size=(40, 24))
    am, mx = O.lm_head_argmax(h, w)
    perm = rng.permutation(40)
    am2, mx2 = O.lm_head_argmax(h, w[perm])
    np.testing.assert_array_equal(perm[am2], am)
    np.testing.assert_allclose(mx2, mx, rtol=1e-12)
    am3, mx3 = O.lm_head_argmax(2.0 * h, w)
    np.testing.assert_array_equal(am3, am)
    np.testing.assert_allclose(mx3, 2 * mx, rtol=1e-12)


def test_ties_take_the_lowest_index():
    rng = np.random.default_rng(5)
    h = rng.normal(size=(2, 8))
    w = rng.normal(size=(12, 8)) * 0.01
    best = 3.0 * h[0] / np.linalg.norm(h[0])
    w[9] = best
    w[4] = best
    am, _ = O.lm_head_argmax(h[:1], w)
    assert am[0] == 4


def test_agrees_with_greedy_acceptance_on_its_scores():
    # the fused choice feeds greedy acceptance exactly as the scores would
    w_ = W.make_small(2, logits=False)
    hid, wt = W.lm_head_inputs(w_.spec)
    h = hid.float().numpy().reshape(-1, hid.shape[-1])
    wf = wt.float().numpy()
    am, _ = O.lm_head_argmax(h, wf)
    lg = O.lm_head_logits(h, wf).reshape(w_.spec.B, w_.spec.N, -1)
    np.testing.assert_array_equal(O.accept_greedy(lg, w_.draft_tokens, w_.parents)["argmax"].reshape(-1), am)
    assert W.hidden_size(w_.spec) == 4096 and hid.shape == (w_.spec.B, w_.spec.N, 4096)
    assert abs(float(lg.std()) - w_.spec.logit_std) < 0.1
