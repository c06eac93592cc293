"""Throughput of one verification step on one GPU.

A step is one pass of the whole path over one batch: tree-masked attention
over the paged prefix, with the tree masks built from the parent array in
the attention kernels (tv_tree_attention_parents), then greedy acceptance
over the target logits with the KV compaction of the accepted paths (one
call, tv_accept_greedy_compact: the workgroup that walks a sequence moves
its rows), each on the current stream.  Inputs are synthetic (seeded) and
resident in HBM before timing.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 2] [--workloads 3,4,5]

Prints ONE JSON line.  `value` is verified tree tokens per second
(B * N / mean step time) of the main workload (--config, default the
Llama-3-8B-shaped layer).  Before every timed step a 1 GiB read-only pass
over a scratch buffer evicts the 256 MB Infinity Cache and the L2 (outside
the step's events), so every step reads its inputs from HBM; the flush only
reads, so it leaves no dirty lines whose write-back would land inside the
step.  The K timed steps carry one event pair each; a second pass of K steps
with an event between every call gives the per-call times.  Compaction
rewrites the tree slots in place; later steps accept the same paths and move
the same number of rows, so the work per step is unchanged.

The other workloads named by --workloads (default: the batched-serving,
long-context and 70B-chain workloads, where the attention targets sit) are
measured in the same run with the same protocol and reported under
`workloads`, each with its attention roofline fraction against its target.

The tree K/V write (rotary positions and paged append of the step's new
rows, the path's upstream neighbour), stochastic acceptance (temperature
> 0, the alternative to the greedy call) and the target's LM head fused with
the greedy choice (bf16 hidden states and weight of the workload's model,
hidden 4096 / 3584 / 8192) and the draft-tree construction that produces
the step's parents and tokens (the drafter's scores of every level, fp32)
are timed on the main workload on their own, K calls after an eviction each,
and reported under `extra_calls`; they are not part of `value`.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "verified tree-tokens/s + achieved HBM GB/s / MFMA util, Llama-3-8B-shape layer"
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
PROFILES = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "tree_attention_verification_05_amd", "csrc")
# the sources each call's kernels are built from (the shared device helpers
# included): counter runs taken on other sources are not reported
KERNEL_SOURCES = {
    "tv_tree_attention": ["attn_mfma.hip", "attn_rowwave.hip", "tv_internal.h"],
    "tv_tree_attention_parents": ["attn_mfma.hip", "attn_rowwave.hip", "tv_internal.h"],
    "tv_accept_greedy": ["accept.hip", "kv_compact_rows.h", "tv_internal.h"],
    "tv_accept_greedy_compact": ["accept.hip", "kv_compact_rows.h", "tv_internal.h"],
    "tv_kv_compact": ["kv_compact.hip", "kv_compact_rows.h", "tv_internal.h"],
    "tv_build_tree_mask": ["tree_mask.hip", "tv_internal.h"],
    "tv_tree_kv_write": ["tree_kv_write.hip", "tv_internal.h"],
    "tv_accept_stochastic": ["accept_stochastic.hip", "tv_internal.h"],
    "tv_lm_head_argmax": ["lm_head.hip", "tv_internal.h"],
    "tv_build_draft_tree": ["draft_tree.hip", "tv_internal.h"],
}


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=2, choices=[1, 2, 3, 4, 5],
                    help="workload 1..5 (default 2: Llama-3-8B-shaped layer, EAGLE-2 60-node tree)")
    ap.add_argument("--workloads", default="3,4,5",
                    help="other workloads timed in the same run (comma list, or 'none')")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--oracle-seconds", type=float, default=12.0,
                    help="host time budget of the CPU-oracle baseline (0 disables it)")
    ap.add_argument("--no-flush", action="store_true", help="do not flush caches between steps")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a 256 MiB elementwise copy kernel (calibrates HBM counters under a profiler)")
    return ap.parse_args()


def source_digest(kernel: str) -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


RIDGE_FLOP_PER_BYTE = BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)


def step_work(w, accept_len, accepted_nodes):
    """Algorithmic bytes (and flops) each call moves for this batch: what the
    method must read or write at least, with every K/V row of a KV head read
    once for all its nodes and query heads.  The compaction count comes from
    the accepted paths of the step."""
    import numpy as np
    s = w.spec
    B, N = s.B, s.N
    elt = 2 if s.dtype == "bf16" else 4
    Wd = (N + 63) // 64
    P = w.prefix_lens.astype(np.int64)
    depth = np.zeros((B, N), np.int64)
    rows = np.arange(B)
    for i in range(1, N):
        depth[:, i] = depth[rows, w.parents[:, i]] + 1
    nblk = (P + N + s.block_size - 1) // s.block_size
    kv_bytes = int((2 * (P + N) * s.Hkv * s.D * elt).sum())
    qo_bytes = 2 * B * N * s.Hq * s.D * elt
    attn_bytes = kv_bytes + qo_bytes + B * N * Wd * 8 + int(nblk.sum()) * 4 + B * 4
    # built from the parents: the parent array (4 bytes a node) instead of the masks
    attn_parents_bytes = attn_bytes - B * N * Wd * 8 + B * N * 4
    attn_flops = int(4 * s.D * s.Hq * (N * P + (depth + 1).sum(axis=1)).sum())
    moved = 0
    for b in range(B):
        L = int(accept_len[b]) + 1
        path = accepted_nodes[b, :L]
        moved += int((path != np.arange(L)).sum())
    row_bytes = s.Hkv * s.D * elt
    accept_bytes = B * N * s.V * 4 + B * N * 4 * 3 + B * (N + 2) * 4
    compact_bytes = moved * 2 * 2 * row_bytes + B * (N + 3) * 4
    return {
        "tv_build_tree_mask": {"bytes": B * N * (4 + 8 * Wd + 4)},
        "tv_tree_attention": {"bytes": attn_bytes, "flops": attn_flops,
                              "bound": "mfma" if attn_flops / attn_bytes > RIDGE_FLOP_PER_BYTE
                              else "hbm"},
        "tv_tree_attention_parents": {"bytes": attn_parents_bytes, "flops": attn_flops,
                                      "bound": "mfma" if attn_flops / attn_parents_bytes > RIDGE_FLOP_PER_BYTE
                                      else "hbm"},
        "tv_accept_greedy": {"bytes": accept_bytes},
        "tv_kv_compact": {"bytes": compact_bytes},
        # the fused call moves what the two do, less the path and length
        # arrays the compaction would read back
        "tv_accept_greedy_compact": {"bytes": accept_bytes + compact_bytes - B * (N + 1) * 4},
    }


# the attention targets: HBM fraction on the memory-bound workloads,
# bf16 matrix-core fraction on the one above the ridge
TARGETS = {3: ("hbm", 0.60), 4: ("mfma", 0.40), 5: ("hbm", 0.60)}
# the step: attention with the tree masks built from the parents inside it,
# then acceptance with the compaction of its accepted paths in the same call
# (the walking workgroup moves the rows)
ATTN_CALL = "tv_tree_attention_parents"
STEP_CALLS = [ATTN_CALL, "tv_accept_greedy_compact"]
TIME_BASE = ("mean HIP-event time of each call, events recorded on the launch stream around the "
             "call's launches (for attention: the main kernel, plus the launch gap and merge kernel "
             "where a second kernel merges the split key ranges), one eviction before every step")


class StepBench:
    """The calls of one workload's step on device-resident inputs, with its
    buffers allocated once."""

    def __init__(self, T, W, cfg: int, seed: int, dev):
        import torch
        self.T, self.torch, self.dev = T, torch, dev
        w = W.make_config(cfg, seed=seed)
        self.w, self.spec = w, w.spec
        B, N, V = w.spec.B, w.spec.N, w.spec.V
        self.q, self.k, self.v = w.q.to(dev), w.k_cache.to(dev), w.v_cache.to(dev)
        self.table = torch.from_numpy(w.block_table).to(dev)
        self.prefix = torch.from_numpy(w.prefix_lens).to(dev)
        self.parents = torch.from_numpy(w.parents).to(dev)
        self.draft = torch.from_numpy(w.draft_tokens).to(dev)
        self.logits = w.logits.to(dev)
        self.status = torch.zeros(1, dtype=torch.int32, device=dev)
        Wd = (N + 63) // 64
        self.mask = torch.empty((B, N, Wd), dtype=torch.int64, device=dev)
        self.depth = torch.empty((B, N), dtype=torch.int32, device=dev)
        self.out = torch.empty_like(self.q)
        self.dt = T.TV_BF16 if self.q.dtype == torch.bfloat16 else T.TV_F32
        ws_bytes = T.tv_tree_attention_workspace_size(B, N, w.spec.Hq, w.spec.Hkv, w.spec.D,
                                                      w.max_prefix_len)
        # (zero-filled once: the arrival counters start at zero, and every call
        # leaves them so)
        self.attn_ws = torch.zeros(max(ws_bytes, 16), dtype=torch.uint8, device=dev)
        self.acc_len = torch.empty(B, dtype=torch.int32, device=dev)
        self.acc_nodes = torch.empty((B, N), dtype=torch.int32, device=dev)
        self.bonus = torch.empty(B, dtype=torch.int32, device=dev)
        self.am = torch.empty((B, N), dtype=torch.int32, device=dev)
        self.new_lens = torch.empty(B, dtype=torch.int32, device=dev)
        self.acc_ws = torch.zeros(max(int(T.lib.tv_accept_greedy_workspace_size(B, N, V)), 16),
                                  dtype=torch.uint8, device=dev)
        self.stream = torch.cuda.current_stream(dev)
        # the node depths the tree K/V write (timed outside the step) takes;
        # the step itself builds its masks inside attention
        T.tv_build_tree_mask(self.parents, mask=self.mask, depth=self.depth, dev_status=self.status)

    def run_step(self, ev=None):
        T, st = self.T, self.stream
        if ev is not None:
            ev[0].record(st)
        T.tv_tree_attention_parents(self.q, self.k, self.v, self.table, self.prefix, self.w.max_prefix_len,
                                    self.parents, out=self.out, workspace=self.attn_ws, dev_status=self.status)
        if ev is not None:
            ev[1].record(st)
        T.tv_accept_greedy_compact(self.logits, self.draft, self.parents, self.k, self.v, self.table, self.prefix,
                                   accept_len=self.acc_len, accepted_nodes=self.acc_nodes, bonus_token=self.bonus,
                                   target_argmax=self.am, new_lens=self.new_lens, workspace=self.acc_ws,
                                   dev_status=self.status)
        if ev is not None:
            ev[2].record(st)

    def measure(self, steps: int, warmup: int, evict):
        """W warm-up steps, then exactly K timed steps (one event pair each,
        an eviction before each outside the events), then K more steps with
        an event between every call.  Returns the per-workload record."""
        import numpy as np
        torch = self.torch
        for _ in range(warmup):
            self.run_step()
        torch.cuda.synchronize()
        if int(self.status.item()) != 0:
            raise RuntimeError(f"device status {int(self.status.item())} on generated inputs")
        step_ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
        torch.cuda.synchronize()
        t_wall = time.perf_counter()
        for s in range(steps):
            evict()
            step_ev[s][0].record(self.stream)
            self.run_step()
            step_ev[s][1].record(self.stream)
        torch.cuda.synchronize()
        self.t_wall = time.perf_counter() - t_wall
        self.step_ms = np.array([step_ev[s][0].elapsed_time(step_ev[s][1]) for s in range(steps)])
        ncalls = len(STEP_CALLS)
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(ncalls + 1)] for _ in range(steps)]
        for s in range(steps):
            evict()
            self.run_step(evs[s])
        torch.cuda.synchronize()
        self.per = np.array([[evs[s][j].elapsed_time(evs[s][j + 1]) for j in range(ncalls)]
                             for s in range(steps)])  # ms
        return self.record()

    def record(self):
        import numpy as np
        spec, w = self.spec, self.w
        B, N = spec.B, spec.N
        ms = float(self.step_ms.mean())
        al = self.acc_len.cpu().numpy()
        work = step_work(w, al, self.acc_nodes.cpu().numpy())
        kern = {}
        for j, n in enumerate(STEP_CALLS):
            t_us = float(self.per[:, j].mean()) * 1e3
            byt = work[n]["bytes"]
            kern[n] = {"us": round(t_us, 3), "us_median": round(float(np.median(self.per[:, j])) * 1e3, 3),
                       "bytes": int(byt), "GB_s": round(byt / (t_us * 1e-6) / 1e9, 1)}
            if work[n].get("flops"):
                kern[n]["flops"] = int(work[n]["flops"])
                kern[n]["TFLOP_s"] = round(work[n]["flops"] / (t_us * 1e-6) / 1e12, 2)
                kern[n]["bound"] = work[n]["bound"]
        a = kern[ATTN_CALL]
        a["hbm_frac"] = round(a["GB_s"] / HBM_PEAK_GBS, 4)
        a["mfma_frac"] = round(a["TFLOP_s"] / BF16_PEAK_TFLOPS, 4)
        a["frac"] = a["mfma_frac"] if a["bound"] == "mfma" else a["hbm_frac"]
        a["traffic"] = measured_traffic(ATTN_CALL, spec.name)
        # acceptance statistics of the step (the pages' evaluation reports the
        # mean acceptance length and the accepted count per draft position)
        depth_max = int(al.max()) if B else 0
        per_depth = [int((al >= d).sum()) for d in range(1, max(depth_max, 1) + 1)]
        return {
            "workload": spec.name, "batch": B, "tree_nodes": N, "q_heads": spec.Hq,
            "kv_heads": spec.Hkv, "head_dim": spec.D, "vocab": spec.V,
            "prefix_len": [int(w.prefix_lens.min()), int(w.prefix_lens.max())],
            "ms_per_step": round(ms, 5),
            "ms_per_step_median": round(float(np.median(self.step_ms)), 5),
            "ms_per_step_min": round(float(self.step_ms.min()), 5),
            "tree_tokens_per_s": round(B * N / (ms * 1e-3), 1),
            "accepted_tokens_per_s": round(float((al + 1).sum()) / (ms * 1e-3), 1),
            "mean_accept_len": round(float(al.mean()), 4),
            "accepted_per_depth": per_depth,
            "kernels": kern,
            "dtype": "bf16" if self.dt == self.T.TV_BF16 else "f32",
        }

    def free(self):
        for n in list(vars(self)):
            if isinstance(getattr(self, n), self.torch.Tensor):
                delattr(self, n)
        self.torch.cuda.empty_cache()


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}): the library has no "
              "multi-GPU path; the per-GPU shard runs as --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import tree_attention_verification_05_amd as T
    import workloads as W

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    flush = None if args.no_flush else torch.empty(256 * 1024 * 1024, dtype=torch.float32,
                                                   device=dev)

    def evict():
        if flush is not None:
            flush.sum()  # reads 1 GiB, writes a scalar

    sb = StepBench(T, W, args.config, args.seed, dev)
    w, spec = sb.w, sb.spec
    B, N, V = spec.B, spec.N, spec.V
    main_rec = sb.measure(args.steps, args.warmup, evict)
    ms_per_step = main_rec["ms_per_step"]
    stream = sb.stream
    q, k, v, depth, table, prefix, status = sb.q, sb.k, sb.v, sb.depth, sb.table, sb.prefix, sb.status
    logits, parents, dt = sb.logits, sb.parents, sb.dt

    def time_call(fn):
        """W warm-up calls, then K calls after an eviction each, one event
        pair around each call; the times in ms."""
        for _ in range(args.warmup):
            fn()
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
        for s in range(args.steps):
            evict()
            ev[s][0].record(stream)
            fn()
            ev[s][1].record(stream)
        torch.cuda.synchronize()
        return np.array([e[0].elapsed_time(e[1]) for e in ev])

    # ---- the boundary's separate calls that the step's two calls fuse (the
    # mask kernel, attention on given masks, greedy acceptance, compaction),
    # each on its own ----
    sep_ms = {
        "tv_build_tree_mask": time_call(lambda: T.tv_build_tree_mask(parents, mask=sb.mask, depth=depth,
                                                                     dev_status=status)),
        "tv_tree_attention": time_call(lambda: T.tv_tree_attention(q, k, v, table, prefix, w.max_prefix_len, sb.mask,
                                                                   out=sb.out, workspace=sb.attn_ws,
                                                                   dev_status=status)),
        "tv_accept_greedy": time_call(lambda: T.tv_accept_greedy(logits, sb.draft, parents, accept_len=sb.acc_len,
                                                                 accepted_nodes=sb.acc_nodes, bonus_token=sb.bonus,
                                                                 target_argmax=sb.am, workspace=sb.acc_ws,
                                                                 dev_status=status)),
        "tv_kv_compact": time_call(lambda: T.tv_kv_compact(k, v, table, prefix, sb.acc_nodes, sb.acc_len,
                                                           new_lens=sb.new_lens, dev_status=status)),
    }

    # ---- the tree K/V write (the step's upstream neighbour, before the mask
    # and attention): timed on its own, K calls after an eviction each ----
    k_new, v_new = W.tree_kv_inputs(spec, args.seed)
    k_new, v_new = k_new.to(dev), v_new.to(dev)
    q_rot = torch.empty_like(q)
    theta = W.rope_theta(spec)
    for _ in range(args.warmup):
        T.tv_tree_kv_write(q, k_new, v_new, depth, k, v, table, prefix, theta, q_out=q_rot,
                           dev_status=status)
    kvw_ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    for s in range(args.steps):
        evict()
        kvw_ev[s][0].record(stream)
        T.tv_tree_kv_write(q, k_new, v_new, depth, k, v, table, prefix, theta, q_out=q_rot,
                           dev_status=status)
        kvw_ev[s][1].record(stream)
    torch.cuda.synchronize()
    kvw_ms = np.array([e[0].elapsed_time(e[1]) for e in kvw_ev])
    del k_new, v_new, q_rot

    # ---- stochastic acceptance (temperature > 0), the alternative to the
    # greedy call: timed on its own, K calls after an eviction each; chains
    # carry proposal rows, trees point-mass proposals ----
    chain = spec.tree[0] == "chain"
    sx = W.stochastic_inputs(spec, args.seed, w.logits, proposals=chain)
    s_tok = (sx["draft_tokens"] if chain else torch.from_numpy(w.draft_tokens)).to(dev)
    s_u, s_e = sx["uniforms"].to(dev), sx["expo"].to(dev)
    s_q = sx["draft_probs"].to(dev) if chain else None
    s_al = torch.empty(B, dtype=torch.int32, device=dev)
    s_an = torch.empty((B, N), dtype=torch.int32, device=dev)
    s_bt = torch.empty(B, dtype=torch.int32, device=dev)
    s_ws = torch.zeros(max(int(T.lib.tv_accept_stochastic_workspace_size(B, N, V)), 16),
                       dtype=torch.uint8, device=dev)

    def run_stochastic():
        T.tv_accept_stochastic(logits, s_tok, parents, sx["temperature"], s_u, s_e, s_q,
                               accept_len=s_al, accepted_nodes=s_an, bonus_token=s_bt,
                               workspace=s_ws, dev_status=status)
    for _ in range(args.warmup):
        run_stochastic()
    st_ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    for s in range(args.steps):
        evict()
        st_ev[s][0].record(stream)
        run_stochastic()
        st_ev[s][1].record(stream)
    torch.cuda.synchronize()
    st_ms = np.array([e[0].elapsed_time(e[1]) for e in st_ev])
    if int(status.item()) != 0:
        raise RuntimeError(f"device status {int(status.item())} after the stochastic call")
    s_al_h = s_al.cpu().numpy()
    del s_tok, s_u, s_e, s_q, s_ws

    # ---- the target's LM head fused with the greedy choice (upstream of the
    # acceptance walk; the [B, N, V] scores are never written) ----
    lm_hid, lm_w = W.lm_head_inputs(spec, args.seed)
    lm_hid = lm_hid.reshape(-1, lm_hid.shape[-1]).to(dev)
    lm_w = lm_w.to(dev)
    lm_am = torch.empty(lm_hid.shape[0], dtype=torch.int32, device=dev)
    lm_mx = torch.empty(lm_hid.shape[0], dtype=torch.float32, device=dev)
    for _ in range(args.warmup):
        T.tv_lm_head_argmax(lm_hid, lm_w, argmax=lm_am, max_score=lm_mx)
    lm_ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    for s in range(args.steps):
        evict()
        lm_ev[s][0].record(stream)
        T.tv_lm_head_argmax(lm_hid, lm_w, argmax=lm_am, max_score=lm_mx)
        lm_ev[s][1].record(stream)
    torch.cuda.synchronize()
    lm_ms = np.array([e[0].elapsed_time(e[1]) for e in lm_ev])
    lm_M, lm_H = lm_hid.shape
    del lm_hid, lm_w

    # ---- draft-tree construction (the producer of the step's parents and
    # tokens): the drafter's score rows of every level read once ----
    dx = W.draft_tree_inputs(spec, args.seed)
    d_lg = dx["draft_logits"].to(dev)
    d_root = dx["root_tokens"].to(dev)
    d_par = torch.empty((B, N), dtype=torch.int32, device=dev)
    d_tok = torch.empty((B, N), dtype=torch.int32, device=dev)
    d_sc = torch.empty((B, N), dtype=torch.float32, device=dev)
    d_ws = torch.empty(max(int(T.lib.tv_build_draft_tree_workspace_size(B, dx["depth"], dx["topk"], V)), 16),
                       dtype=torch.uint8, device=dev)

    def run_draft_tree():
        T.tv_build_draft_tree(d_lg, N, root_tokens=d_root, parents=d_par, tokens=d_tok, scores=d_sc,
                              workspace=d_ws)
    for _ in range(args.warmup):
        run_draft_tree()
    dt_ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    for s in range(args.steps):
        evict()
        dt_ev[s][0].record(stream)
        run_draft_tree()
        dt_ev[s][1].record(stream)
    torch.cuda.synchronize()
    dt_ms = np.array([e[0].elapsed_time(e[1]) for e in dt_ev])
    del d_lg, d_ws

    # back-to-back steps with warm caches, for reference
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(args.steps):
        sb.run_step()
    e1.record(stream)
    torch.cuda.synchronize()
    warm_ms = e0.elapsed_time(e1) / args.steps

    if args.copy_calibration:
        # a plain elementwise kernel of known traffic: 256 MiB read, 256 MiB written
        src = torch.ones(64 * 1024 * 1024, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.mul(src, 2.0, out=dst)
        torch.cuda.synchronize()
        del src, dst

    kern = main_rec["kernels"]

    # the tree K/V write, outside the step: its own time and algorithmic bytes
    elt = 2 if dt == T.TV_BF16 else 4
    kvw_bytes = (2 * B * N * spec.Hq * spec.D * elt          # q read, q_out written
                 + 4 * B * N * spec.Hkv * spec.D * elt       # k_new, v_new read; K/V rows written
                 + B * N * 4 + B * 4 + B * N * 4)            # depth, prefix, one table entry per node
    kvw_us = float(kvw_ms.mean()) * 1e3
    extra = {"tv_tree_kv_write": {"us": round(kvw_us, 3), "us_median": round(float(np.median(kvw_ms)) * 1e3, 3),
                                  "bytes": int(kvw_bytes), "GB_s": round(kvw_bytes / (kvw_us * 1e-6) / 1e9, 1),
                                  "rope_theta": theta, "in_step": False}}

    # stochastic acceptance: the logits scan, the gathers of the tree, and
    # one row each of logits and Exp(1) variates per sequence for the draw
    # (plus the rejected child's proposal row on chains that stopped early)
    st_us = float(st_ms.mean()) * 1e3
    rejected = int((s_al_h < N - 1).sum()) if chain else 0
    st_bytes = (B * N * V * 4 + B * N * 4 * (4 + (1 if chain else 0))
                + B * V * 8 + rejected * V * 4)
    extra["tv_accept_stochastic"] = {
        "us": round(st_us, 3), "us_median": round(float(np.median(st_ms)) * 1e3, 3),
        "bytes": int(st_bytes), "GB_s": round(st_bytes / (st_us * 1e-6) / 1e9, 1),
        "temperature": sx["temperature"], "proposals": "rows" if chain else "point mass",
        "mean_accept_len": float(s_al_h.mean()), "in_step": False}

    # fused LM head: weight and hidden states read once, per-tile keys
    # written and read back; 2 M H V flops, MFMA-bound above the ridge
    lm_us = float(lm_ms.mean()) * 1e3
    lm_tiles = (V + 255) // 256
    lm_bytes = V * lm_H * 2 + lm_M * lm_H * 2 + 2 * lm_M * lm_tiles * 8 + lm_M * 8
    lm_flops = 2.0 * lm_M * lm_H * V
    extra["tv_lm_head_argmax"] = {
        "us": round(lm_us, 3), "us_median": round(float(np.median(lm_ms)) * 1e3, 3),
        "bytes": int(lm_bytes), "GB_s": round(lm_bytes / (lm_us * 1e-6) / 1e9, 1),
        "flops": int(lm_flops), "TFLOP_s": round(lm_flops / (lm_us * 1e-6) / 1e12, 2),
        "rows": int(lm_M), "hidden": int(lm_H),
        "bound": "mfma" if lm_flops / lm_bytes > RIDGE_FLOP_PER_BYTE else "hbm", "in_step": False}
    lm_rec = extra["tv_lm_head_argmax"]
    lm_rec["frac"] = round(lm_rec["TFLOP_s"] / BF16_PEAK_TFLOPS if lm_rec["bound"] == "mfma"
                           else lm_rec["GB_s"] / HBM_PEAK_GBS, 4)

    # draft-tree construction: each used score row read once (the root's
    # row and topk rows per later level), the per-chunk statistics and keys
    # written and read back, the tree written
    dt_us = float(dt_ms.mean()) * 1e3
    dt_rows = B * (1 + (dx["depth"] - 1) * dx["topk"])
    dt_chunks = dt_rows * ((V + 8191) // 8192)
    dt_bytes = dt_rows * V * 4 + 2 * dt_chunks * (8 + 8 * dx["topk"]) + B * 4 + 3 * B * N * 4
    extra["tv_build_draft_tree"] = {
        "us": round(dt_us, 3), "us_median": round(float(np.median(dt_ms)) * 1e3, 3),
        "bytes": int(dt_bytes), "GB_s": round(dt_bytes / (dt_us * 1e-6) / 1e9, 1),
        "frac": round(dt_bytes / (dt_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4), "bound": "hbm",
        "depth": dx["depth"], "topk": dx["topk"], "rows": int(dt_rows), "in_step": False}

    # roofline of the dominant call of the main workload's step
    work = step_work(w, sb.acc_len.cpu().numpy(), sb.acc_nodes.cpu().numpy())
    fused_into = {"tv_build_tree_mask": "tv_tree_attention_parents", "tv_tree_attention": "tv_tree_attention_parents",
                  "tv_accept_greedy": "tv_accept_greedy_compact", "tv_kv_compact": "tv_accept_greedy_compact"}
    for n, t_ms in sep_ms.items():
        t_us = float(t_ms.mean()) * 1e3
        rec = {"us": round(t_us, 3), "us_median": round(float(np.median(t_ms)) * 1e3, 3),
               "bytes": int(work[n]["bytes"]), "GB_s": round(work[n]["bytes"] / (t_us * 1e-6) / 1e9, 1),
               "in_step": False, "step_call": fused_into[n]}
        if work[n].get("flops"):
            rec["flops"] = int(work[n]["flops"])
            rec["TFLOP_s"] = round(work[n]["flops"] / (t_us * 1e-6) / 1e12, 2)
        extra[n] = rec
    dom = max(STEP_CALLS, key=lambda n: kern[n]["us"])
    d_us = kern[dom]["us"]
    bound = work[dom].get("bound", "hbm")
    if bound == "mfma":
        achieved = work[dom]["flops"] / (d_us * 1e-6) / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / BF16_PEAK_TFLOPS, 4)}
    else:
        achieved = work[dom]["bytes"] / (d_us * 1e-6) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4)}
    roof["traffic"] = measured_traffic(dom, spec.name)
    roof["kernel"] = dom
    roof["time_base"] = TIME_BASE

    main_tokens = main_rec.pop("tree_tokens_per_s")
    result = {
        "metric": METRIC,
        "value": main_tokens,
        "unit": "tree-tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "ms_per_step_median": main_rec.pop("ms_per_step_median"),
        "ms_per_step_min": main_rec.pop("ms_per_step_min"),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": main_rec.pop("dtype"),
        "data": "synthetic",
        "config": {"workload": spec.name, "batch": B, "tree_nodes": N, "q_heads": spec.Hq,
                   "kv_heads": spec.Hkv, "head_dim": spec.D, "vocab": V,
                   "prefix_len": main_rec["prefix_len"],
                   "block_size": spec.block_size, "cache_flushed_between_steps": flush is not None},
        "roofline": roof,
        "kernels": kern,
        "accepted_tokens_per_s": main_rec["accepted_tokens_per_s"],
        "mean_accept_len": main_rec["mean_accept_len"],
        "accepted_per_depth": main_rec["accepted_per_depth"],
        "extra_calls": extra,
        "warm_cache_ms_per_step": round(warm_ms, 5),
        "wall_s_timed_region": round(sb.t_wall, 4),
    }
    w_main = w
    sb.free()
    del logits, parents, q, k, v, depth, table, prefix, status

    # ---- the other workloads, same protocol, same run ----
    others = {}
    for cfg in parse_workloads(args.workloads, args.config):
        t0 = time.perf_counter()
        ob = StepBench(T, W, cfg, args.seed, dev)
        rec = ob.measure(args.steps, args.warmup, evict)
        ob.free()
        del ob
        if cfg in TARGETS:
            bnd, tgt = TARGETS[cfg]
            a = rec["kernels"][ATTN_CALL]
            got = a["hbm_frac"] if bnd == "hbm" else a["mfma_frac"]
            rec["attention_target"] = {"bound": bnd, "frac": tgt, "achieved_frac": got, "met": got >= tgt}
        rec["wall_s"] = round(time.perf_counter() - t0, 2)
        others[str(cfg)] = rec
    if others:
        result["workloads"] = others
        result["workloads_time_base"] = TIME_BASE

    if args.oracle_seconds > 0:
        result["cpu_baseline"] = cpu_baseline(w_main, args.oracle_seconds)
    print(json.dumps(result), flush=True)


def parse_workloads(text: str, main_cfg: int):
    if not text or text.lower() == "none":
        return []
    out = []
    for tok in text.split(","):
        c = int(tok)
        if c not in (1, 2, 3, 4, 5):
            raise SystemExit(f"--workloads: no workload {c}")
        if c != main_cfg and c not in out:
            out.append(c)
    return out


def measured_traffic(kernel: str, workload: str):
    """HBM bytes per launch from committed counter runs, if they were taken on
    the current kernel source; otherwise None."""
    path = os.path.join(PROFILES, f"{kernel}__{workload}__traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_sha") != source_digest(kernel):
        return None
    return rec.get("bytes_per_launch")


def cpu_baseline(w, seconds: float):
    """The CPU oracle (test infrastructure, float64 NumPy) timed on this host
    over whole steps of the same workload, as many as fit the time budget."""
    import numpy as np

    import oracle as O

    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = os.cpu_count() or 1
    q = w.q.float().numpy()
    kf = w.k_cache.float().numpy()
    vf = w.v_cache.float().numpy()
    k16 = w.k_cache.view(dtype=__import__("torch").int16).numpy()
    v16 = w.v_cache.view(dtype=__import__("torch").int16).numpy()
    lg = w.logits.numpy()
    B = w.B
    seqs_all = list(range(B))
    done_tokens = 0
    done_steps = 0
    seq_cursor = 0
    t0 = time.perf_counter()
    # whole steps when they fit; otherwise one sequence at a time (the oracle
    # treats sequences independently), until the budget is spent
    while time.perf_counter() - t0 < seconds:
        seqs = [seqs_all[seq_cursor % B]]
        seq_cursor += 1
        O.build_tree_mask(w.parents[seqs])
        O.tree_attention(q, kf, vf, w.block_table, w.prefix_lens, w.parents, seqs=seqs)
        acc = O.accept_greedy(lg[seqs], w.draft_tokens[seqs], w.parents[seqs])
        O.kv_compact(k16, v16, w.block_table[seqs], w.prefix_lens[seqs], acc["accepted_nodes"],
                     acc["accept_len"])
        done_tokens += w.N * len(seqs)
        done_steps += 1
    el = time.perf_counter() - t0
    return {"value": round(done_tokens / el, 2), "unit": "tree-tokens/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"{done_steps} single-sequence passes (mask, attention, acceptance, "
                      f"compaction) of the same workload in {el:.1f} s, float64 NumPy",
            "precision": "float64 (inputs are the same bf16 values, upcast exactly)",
            "cpu_model": cpu_model(),
            "host_cpus": os.cpu_count(),
            "affinity_cpus": len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else None}


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


if __name__ == "__main__":
    main()
