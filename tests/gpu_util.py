"""Helpers for the GPU tests: move a workload to the device, run the four
library calls, and compare with the oracle."""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle as O


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def upload(w, dev="cuda"):
    d = {
        "q": w.q.to(dev),
        "k": w.k_cache.to(dev),
        "v": w.v_cache.to(dev),
        "table": torch.from_numpy(w.block_table).to(dev),
        "prefix": torch.from_numpy(w.prefix_lens).to(dev),
        "parents": torch.from_numpy(w.parents).to(dev),
        "draft": torch.from_numpy(w.draft_tokens).to(dev),
        "logits": w.logits.to(dev),
        "status": torch.zeros(1, dtype=torch.int32, device=dev),
    }
    return d


def run_step(T, d, max_prefix_len, compact=True):
    """One verification pass: mask -> attention -> accept -> compaction."""
    mask, depth = T.tv_build_tree_mask(d["parents"], dev_status=d["status"])
    out = T.tv_tree_attention(d["q"], d["k"], d["v"], d["table"], d["prefix"], max_prefix_len,
                              mask, dev_status=d["status"])
    al, an, bt, am = T.tv_accept_greedy(d["logits"], d["draft"], d["parents"],
                                        dev_status=d["status"])
    nl = None
    if compact:
        nl = T.tv_kv_compact(d["k"], d["v"], d["table"], d["prefix"], an, al,
                             dev_status=d["status"])
    torch.cuda.synchronize()
    return dict(mask=mask, depth=depth, out=out, accept_len=al, accepted_nodes=an, bonus=bt,
                argmax=am, new_lens=nl)


def host_f(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy()


def raw_bits(t: torch.Tensor) -> np.ndarray:
    """Bytes of a tensor as unsigned integers of the same width."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.float32:
        return t.view(torch.int32).numpy().view(np.uint32)
    raise TypeError(t.dtype)


def attention_tolerance(dtype):
    """Per-element bound |gpu - oracle| <= atol + rtol * |oracle|: bf16 outputs
    max-abs 2e-2 / rel 1e-2; fp32 outputs 1e-4 / 1e-4."""
    return (2e-2, 1e-2) if dtype == torch.bfloat16 else (1e-4, 1e-4)


def relative_l2_bound(dtype):
    """Per-sequence bound on ||gpu - oracle||_2 / ||oracle||_2.

    bf16: an output passes through at most three round-to-nearest-even bf16
    roundings that the oracle does not make -- the softmax weights before the
    P V product, the normalised partial state of a split key range, and the
    final output.  Each has relative error at most 2^-8 and, over many
    elements, a root-mean-square of at most 2^-8 / sqrt(3); three independent
    ones give sqrt(3) * 2^-8 / sqrt(3) = 2^-8 = 3.9e-3, so 4e-3.  The
    per-element bound alone is loose at long prefixes, where |out| shrinks as
    1 / sqrt(prefix length) (about 0.01 at 32768 keys, half the absolute
    tolerance): the relative L2 error is what shows a mis-weighted piece or a
    dropped key there.
    fp32: only summation order differs; 1e-5."""
    return 4e-3 if dtype == torch.bfloat16 else 1e-5


# worst relative L2 error per checked case, reported at the end of the run
# (tests/conftest.py prints it and, if TV_PARITY_SUMMARY names a file, writes
# it there as JSON)
RESULTS = {}


def record(label: str, **fields) -> None:
    RESULTS.setdefault(label, {}).update(fields)


def check_attention(gpu_out: torch.Tensor, ref: np.ndarray, seqs, dtype, label: str = ""):
    """Element-wise tolerance and per-sequence relative L2 error against the
    oracle on sequences ``seqs``; returns the worst relative L2 error."""
    atol, rtol = attention_tolerance(dtype)
    rel_max = relative_l2_bound(dtype)
    g = host_f(gpu_out)
    worst = 0.0
    worst_abs = 0.0
    for b in seqs:
        diff = np.abs(g[b] - ref[b])
        bound = atol + rtol * np.abs(ref[b])
        bad = ~(diff <= bound)  # NaN anywhere counts as a failure
        if bad.any():
            idx = np.argwhere(bad)[0]
            raise AssertionError(
                f"{label} seq {b}: {int(bad.sum())} elements outside tolerance; first at node,head,dim="
                f"{tuple(idx)}: gpu {g[b][tuple(idx)]} oracle {ref[b][tuple(idx)]}")
        rel = float(np.linalg.norm(g[b] - ref[b]) / max(np.linalg.norm(ref[b]), 1e-30))
        assert rel <= rel_max, f"{label} seq {b}: relative L2 error {rel:.3e} > {rel_max:.1e}"
        worst = max(worst, rel)
        worst_abs = max(worst_abs, float(diff.max()))
    if label:
        record(label, seqs=len(list(seqs)), rel_l2=worst, max_abs=worst_abs)
    return worst


def check_accept(res, ref):
    assert np.array_equal(res["argmax"].cpu().numpy(), ref["argmax"])
    assert np.array_equal(res["accept_len"].cpu().numpy(), ref["accept_len"])
    assert np.array_equal(res["accepted_nodes"].cpu().numpy(), ref["accepted_nodes"])
    assert np.array_equal(res["bonus"].cpu().numpy(), ref["bonus"])


def oracle_attention(w, seqs=None):
    return O.tree_attention(w.q.float().numpy(), w.k_cache.float().numpy(),
                            w.v_cache.float().numpy(), w.block_table, w.prefix_lens, w.parents,
                            seqs=seqs)
