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


def check_attention(gpu_out: torch.Tensor, ref: np.ndarray, seqs, dtype):
    atol, rtol = attention_tolerance(dtype)
    g = host_f(gpu_out)
    worst = 0.0
    for b in seqs:
        diff = np.abs(g[b] - ref[b])
        bound = atol + rtol * np.abs(ref[b])
        bad = ~(diff <= bound)  # NaN anywhere counts as a failure
        if bad.any():
            idx = np.argwhere(bad)[0]
            raise AssertionError(
                f"seq {b}: {int(bad.sum())} elements outside tolerance; first at node,head,dim="
                f"{tuple(idx)}: gpu {g[b][tuple(idx)]} oracle {ref[b][tuple(idx)]}")
        rel = np.linalg.norm(g[b] - ref[b]) / max(np.linalg.norm(ref[b]), 1e-30)
        worst = max(worst, float(rel))
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
