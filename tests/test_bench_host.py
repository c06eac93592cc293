"""Host logic of bench.py (no GPU): the one-GPU refusal, the workload list,
and the algorithmic bytes and flops it divides by the measured times."""
import os
import subprocess
import sys

import numpy as np
import pytest

import bench
import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and not r.stdout.strip()


def test_workload_list():
    assert bench.parse_workloads("3,4,5", 2) == [3, 4, 5]
    assert bench.parse_workloads("3,2,3", 2) == [3]
    assert bench.parse_workloads("none", 2) == []
    with pytest.raises(SystemExit):
        bench.parse_workloads("7", 2)


def test_step_work_by_hand():
    """A chain of N = 3 nodes over prefixes 5 and 0, two KV heads of D = 64
    (bf16), four query heads: every figure counted by hand."""
    import dataclasses
    spec = dataclasses.replace(W.SMALL[5], name="hand", B=2, Hq=4, Hkv=2, D=64, V=10,
                               tree=("chain", 3), prefix_lengths=(5, 0), dtype="bf16")
    w = W.build(spec, 0)
    assert list(w.prefix_lens) == [5, 0] and w.N == 3
    accept_len = np.array([2, 0])
    accepted = np.array([[0, 1, 2], [0, -1, -1]])
    work = bench.step_work(w, accept_len, accepted)
    # K and V rows of every visible position, once per KV head: (5 + 3) + (0 + 3) positions
    kv = 2 * (8 + 3) * 2 * 64 * 2
    qo = 2 * 2 * 3 * 4 * 64 * 2
    blocks = 1 + 1                       # ceil(8 / 16) + ceil(3 / 16)
    attn = kv + qo + 2 * 3 * 8 + blocks * 4 + 2 * 4
    assert work["tv_tree_attention"]["bytes"] == attn
    # flops: 4 D per (node, query head, visible key); chain node i sees P + i + 1 keys
    flops = 4 * 64 * 4 * ((5 + 1) + (5 + 2) + (5 + 3) + (0 + 1) + (0 + 2) + (0 + 3))
    assert work["tv_tree_attention"]["flops"] == flops
    assert work["tv_accept_greedy"]["bytes"] == 2 * 3 * 10 * 4 + 2 * 3 * 4 * 3 + 2 * 5 * 4
    # a chain's accepted path is the identity: nothing moves
    assert work["tv_kv_compact"]["bytes"] == 2 * 6 * 4
    # fused: both, less the path (N entries) and length the compaction reads back
    assert work["tv_accept_greedy_compact"]["bytes"] == (work["tv_accept_greedy"]["bytes"]
                                                         + work["tv_kv_compact"]["bytes"] - 2 * 4 * 4)
