"""GPU parity of tv_lm_head_argmax against the oracle.

Scores are bf16 products summed in fp32 on the GPU and in float64 by the
oracle.  Each row's best score must match the oracle's within
1e-3 * (1 + |score|); the chosen index must equal the oracle's unless the
oracle scores the GPU's choice within 2e-3 * (1 + |score|) of its own best
(a near tie that fp32 rounding may flip), which at most one row per case
may do.  Small cases compare every row; full-size workloads compare sampled
rows, the oracle run over vocabulary slices to bound its float64 memory."""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from gpu_util import log

pytestmark = pytest.mark.gpu

T = None


def setup_module():
    global T
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import tree_attention_verification_05_amd as lib
    T = lib


def oracle_rows(h_rows, w, slab=16384):
    """float64 scores of some rows against every vocabulary row, a slab of
    the weight at a time."""
    V = w.shape[0]
    out = np.empty((h_rows.shape[0], V))
    for v0 in range(0, V, slab):
        out[:, v0:v0 + slab] = O.lm_head_logits(h_rows, w[v0:v0 + slab])
    return out


def check(hidden, weight, rows=None, label=""):
    """hidden [M, H] and weight [V, H] bf16 host tensors."""
    M, H = hidden.shape
    V = weight.shape[0]
    log(f"[lm_head] {label} M={M} H={H} V={V}")
    am, mx = T.tv_lm_head_argmax(hidden.cuda(), weight.cuda())
    torch.cuda.synchronize()
    am, mx = am.cpu().numpy(), mx.cpu().numpy()
    rows = np.arange(M) if rows is None else np.asarray(rows)
    h = hidden.float().numpy()[rows]
    w = weight.float().numpy()
    sc = oracle_rows(h, w)
    ref_am = np.argmax(sc, axis=1)
    ref_mx = sc[np.arange(len(rows)), ref_am]
    np.testing.assert_array_less(np.abs(mx[rows] - ref_mx), 1e-3 * (1 + np.abs(ref_mx)))
    differ = 0
    for i, r in enumerate(rows):
        if am[r] == ref_am[i]:
            continue
        g = int(am[r])
        assert 0 <= g < V, f"{label} row {r}: index {g} out of range"
        gap = ref_mx[i] - sc[i, g]
        assert gap <= 2e-3 * (1 + abs(ref_mx[i])), (
            f"{label} row {r}: gpu {g} (oracle score {sc[i, g]:.6f}), oracle {ref_am[i]} ({ref_mx[i]:.6f})")
        differ += 1
    assert differ <= 1, f"{label}: {differ} rows differ at near ties"
    return am, mx


def rand_bf16(shape, std, seed):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(shape, generator=g) * std).to(torch.bfloat16)


@pytest.mark.parametrize("M,H,V", [(60, 4096, 5003), (64, 256, 1000), (65, 512, 777), (130, 1024, 4099),
                                   (1, 64, 1), (3, 64, 300), (257, 192, 2600)])
def test_shapes(M, H, V):
    # row tiles of 64 and 128 with tails, vocabulary tails, one row, one column
    check(rand_bf16((M, H), 1.0, M + H), rand_bf16((V, H), 2.0 / np.sqrt(H), V), label=f"shape-{M}-{H}-{V}")


def test_planted_rows_and_ties():
    # every row's best entry planted (some in the vocabulary tail tile), and
    # two identical weight rows: the lower index must win
    M, H, V = 100, 512, 3000
    hid = rand_bf16((M, H), 1.0, 1)
    w = rand_bf16((V, H), 2.0 / np.sqrt(H), 2)
    rng = np.random.default_rng(3)
    targets = rng.choice(np.arange(10, 2800), size=M, replace=False)
    targets[0], targets[1] = V - 1, 2816   # last column; first column of the last tile
    hf = hid.float()
    for m, t in enumerate(targets):
        w[t] = (4.0 * hf[m] / hf[m].norm()).to(torch.bfloat16)
    w[5] = w[targets[7]]
    targets[7] = min(5, targets[7])
    am, _ = check(hid, w, label="planted")
    np.testing.assert_array_equal(am, targets)


def test_identity_weight():
    H = 256
    hid = rand_bf16((40, H), 1.0, 9)
    am, mx = check(hid, torch.eye(H, dtype=torch.bfloat16), label="identity")
    np.testing.assert_array_equal(am, np.argmax(hid.float().numpy(), axis=1))


def test_small_workload_feeds_greedy_acceptance():
    w_ = W.make_small(2, logits=False)
    hid, wt = W.lm_head_inputs(w_.spec)
    s = w_.spec
    am, _ = T.tv_lm_head_argmax(hid.cuda(), wt.cuda())
    torch.cuda.synchronize()
    assert tuple(am.shape) == (s.B, s.N)
    lg = O.lm_head_logits(hid.float().numpy().reshape(-1, hid.shape[-1]), wt.float().numpy())
    ref = np.argmax(lg, axis=1).reshape(s.B, s.N)
    assert (am.cpu().numpy() == ref).mean() > 0.99


@pytest.mark.parametrize("cfg", [2, 3, 4, 5])
def test_full_size(cfg):
    """The full workload's rows (B * N) against its LM head, in the launch
    configuration the benchmark times; 12 sampled rows checked."""
    spec = W.CONFIGS[cfg]
    hid, wt = W.lm_head_inputs(spec)
    hid = hid.reshape(-1, hid.shape[-1])
    M = hid.shape[0]
    rows = np.unique(np.concatenate([[0, M - 1], np.random.default_rng(cfg).choice(M, 10, replace=False)]))
    check(hid, wt, rows=rows, label=f"full{cfg}")
