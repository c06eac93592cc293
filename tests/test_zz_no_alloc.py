"""tv_accept_greedy_noalloc (the allocation-free variant, whose chunk keys
live in the library's static per-GPU scratch buffer) against
tv_accept_greedy with a caller workspace: bit-identical outputs on two calls
in a row, the second with a smaller input, so that keys left in the shared
buffer by the larger call cannot reach the smaller one's result.  Both are
also checked against the oracle."""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as W

pytestmark = pytest.mark.gpu


def _lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import tree_attention_verification_05_amd as T
    return T


def run_both(T, w):
    """Both calls on the same device inputs; returns their outputs on the host."""
    dev = "cuda"
    lg = w.logits.to(dev)
    dt = torch.from_numpy(w.draft_tokens).to(dev)
    par = torch.from_numpy(w.parents).to(dev)
    B, N = w.draft_tokens.shape
    print(f"[no-alloc] {w.spec.name} B={B} N={N} V={lg.shape[-1]} "
          f"keys {T.lib.tv_accept_greedy_workspace_size(B, N, lg.shape[-1]) // 8}", flush=True)
    st0 = torch.zeros(1, dtype=torch.int32, device=dev)
    st1 = torch.zeros(1, dtype=torch.int32, device=dev)
    ref = T.tv_accept_greedy(lg, dt, par, dev_status=st0)
    # outputs pre-filled with values no call writes, so an unwritten entry shows
    out = (torch.full((B,), -7, dtype=torch.int32, device=dev),
           torch.full((B, N), -7, dtype=torch.int32, device=dev),
           torch.full((B,), -7, dtype=torch.int32, device=dev),
           torch.full((B, N), -7, dtype=torch.int32, device=dev))
    T.tv_accept_greedy_noalloc(lg, dt, par, *out, dev_status=st1)
    torch.cuda.synchronize()
    assert int(st0.item()) == 0 and int(st1.item()) == 0
    return [t.cpu().numpy() for t in ref], [t.cpu().numpy() for t in out]


def test_noalloc_matches_workspace_call_on_two_calls_shrinking():
    T = _lib()
    large = W.build(W.CONFIGS[5], 0, dense=False)   # 1152 rows of 128256 logits: 2304 chunk keys
    small = W.make_small(3, seed=9, dense=False)     # 130 rows of 1000
    for w in (large, small):
        ref, got = run_both(T, w)
        for name, a, b in zip(("accept_len", "accepted_nodes", "bonus", "argmax"), ref, got):
            assert np.array_equal(a, b), f"{w.spec.name}: {name} differs"
        want = O.accept_greedy(w.logits.numpy(), w.draft_tokens, w.parents)
        assert np.array_equal(got[0], want["accept_len"])
        assert np.array_equal(got[1], want["accepted_nodes"])
        assert np.array_equal(got[2], want["bonus"])
        assert np.array_equal(got[3], want["argmax"])


def test_noalloc_refuses_sizes_beyond_its_scratch():
    T = _lib()
    dev = "cuda"
    B, N, V = 2049, 256, 8
    lg = torch.zeros((B, N, V), dtype=torch.float32, device=dev)
    i32 = lambda *s: torch.zeros(s, dtype=torch.int32, device=dev)
    with pytest.raises(T.TVError) as e:
        T.tv_accept_greedy_noalloc(lg, i32(B, N), i32(B, N), i32(B), i32(B, N), i32(B))
    assert e.value.status == T.TV_ERR_TOO_LARGE
