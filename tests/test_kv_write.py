"""GPU parity of tv_tree_kv_write against the oracle: rotated queries and
keys within one bf16 unit in the last place (or 1e-5 for fp32) of the
float64 rotation, values copied bit for bit, and every other cache row
unchanged bit for bit."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from gpu_util import log, raw_bits

pytestmark = pytest.mark.gpu

T = None


def setup_module():
    global T
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import tree_attention_verification_05_amd as lib
    T = lib


def _tol(dtype):
    # bf16: one unit in the last place (2^-7 relative) plus the fp32 rotation
    return (1e-6, 2.0 ** -7) if dtype == torch.bfloat16 else (1e-5, 1e-5)


def _close(gpu, ref, dtype, what):
    atol, rtol = _tol(dtype)
    g = gpu.detach().float().cpu().numpy()
    bad = ~(np.abs(g - ref) <= atol + rtol * np.abs(ref))
    if bad.any():
        idx = tuple(np.argwhere(bad)[0])
        raise AssertionError(f"{what}: {int(bad.sum())} elements off; first {idx}: gpu {g[idx]} oracle {ref[idx]}")


def _swap_layout(t: torch.Tensor) -> torch.Tensor:
    """[num_blocks, Hkv, 16, D] <-> [num_blocks, 16, Hkv, D]."""
    return t.permute(0, 2, 1, 3).contiguous()


def check_write(w, in_place=False, label="", token_major=False):
    s = w.spec
    theta = W.rope_theta(s)
    k_new, v_new = W.tree_kv_inputs(s)
    log(f"[kv_write] {label} {s.name} B={w.B} N={w.N} theta={theta}")
    dev = "cuda"
    q = w.q.to(dev)
    kc, vc = w.k_cache.to(dev), w.v_cache.to(dev)
    table = torch.from_numpy(w.block_table).to(dev)
    prefix = torch.from_numpy(w.prefix_lens).to(dev)
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    _, depth = T.tv_build_tree_mask(torch.from_numpy(w.parents).to(dev))
    q_out = q if in_place else None
    if token_major:
        # the call writes token-major caches; the checks below read them back
        # in head-major order
        kt, vt = _swap_layout(kc), _swap_layout(vc)
        qo = T.tv_tree_kv_write(q, k_new.to(dev), v_new.to(dev), depth, kt, vt, table, prefix, theta,
                                q_out=q_out, dev_status=status, token_major=True)
        kc, vc = _swap_layout(kt), _swap_layout(vt)
    else:
        qo = T.tv_tree_kv_write(q, k_new.to(dev), v_new.to(dev), depth, kc, vc, table, prefix, theta,
                                q_out=q_out, dev_status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    q_rot, k_rot, pos = O.tree_kv_write(w.q.float().numpy(), k_new.float().numpy(), w.parents,
                                        w.prefix_lens, theta)
    _close(qo, q_rot, w.q.dtype, "q_out")
    # cache rows: the tree slots hold the rotated keys and the values; all
    # other rows keep their bytes
    k_rows = O.token_rows(kc.float().cpu().numpy())
    v_bits = O.token_rows(raw_bits(vc))
    k_bits, k0 = O.token_rows(raw_bits(kc)), O.token_rows(raw_bits(w.k_cache))
    v0 = O.token_rows(raw_bits(w.v_cache))
    bs = s.block_size
    touched = np.zeros(k_rows.shape[0], dtype=bool)
    vnew_bits = raw_bits(v_new)
    for b in range(w.B):
        rows = O.cache_rows(w.block_table[b], int(w.prefix_lens[b]) + np.arange(w.N), bs)
        touched[rows] = True
        _close(torch.from_numpy(k_rows[rows]), k_rot[b], w.q.dtype, f"k rows of sequence {b}")
        assert np.array_equal(v_bits[rows], vnew_bits[b]), f"v rows of sequence {b}"
    assert np.array_equal(k_bits[~touched], k0[~touched])
    assert np.array_equal(v_bits[~touched], v0[~touched])
    return qo


@pytest.mark.parametrize("i", [1, 2, 3, 4, 5])
def test_small_configs(i):
    check_write(W.make_small(i), label=f"small{i}")


@pytest.mark.parametrize("i", [2, 3, 4, 5])
def test_full_configs(i):
    check_write(W.make_config(i), label=f"full{i}")


@pytest.mark.parametrize("i", [1, 3])
def test_token_major_caches(i):
    """Token-major caches ([num_blocks, 16, Hkv, D]): the same rows written,
    every other byte kept (fp32 and bf16)."""
    check_write(W.make_small(i), label=f"small{i} token-major", token_major=True)


def test_in_place_queries():
    check_write(W.make_small(3, seed=3), in_place=True, label="in place")


def test_head_dim_64_and_tiny_prefix():
    w = W.build(dataclasses.replace(W.SMALL[3], name="kvw-d64", tag=117, D=64, Hq=8, Hkv=2,
                                    prefix=(0, 3), B=6))
    check_write(w, label="D=64 P<=3")


def test_chain_positions_are_consecutive():
    """A chain tree rotates node i to P + i, exactly like decoding the chain."""
    w = W.build(dataclasses.replace(W.SMALL[5], name="kvw-chain", tag=118))
    qo = check_write(w, label="chain")
    theta = W.rope_theta(w.spec)
    ref = O.rope(w.q.float().numpy(), (w.prefix_lens[:, None] + np.arange(w.N))[:, :, None], theta)
    _close(qo, ref, w.q.dtype, "chain q")


def test_device_status_and_untouched_rows():
    """A bad depth raises TV_DEV_BAD_TREE; a slot whose block id is outside
    the cache raises TV_DEV_BAD_CACHE and that node's rows are not written."""
    w = W.make_small(3, seed=9)
    s = w.spec
    dev = "cuda"
    k_new, v_new = W.tree_kv_inputs(s)
    kc, vc = w.k_cache.to(dev), w.v_cache.to(dev)
    table_np = w.block_table.copy()
    b_bad = 1
    t = int(w.prefix_lens[b_bad])  # node 0 of sequence 1
    good_block = int(table_np[b_bad, t // s.block_size])
    table_np[b_bad, t // s.block_size] = w.num_blocks + 5
    table = torch.from_numpy(table_np).to(dev)
    prefix = torch.from_numpy(w.prefix_lens).to(dev)
    _, depth = T.tv_build_tree_mask(torch.from_numpy(w.parents).to(dev))
    depth[0, 2] = -3
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    T.tv_tree_kv_write(w.q.to(dev), k_new.to(dev), v_new.to(dev), depth, kc, vc, table, prefix,
                       W.rope_theta(s), dev_status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == T.TV_DEV_BAD_TREE | T.TV_DEV_BAD_CACHE
    # the block that held sequence 1's node 0 slot is untouched at that slot
    k_after = raw_bits(kc)
    k_before = raw_bits(w.k_cache)
    assert np.array_equal(k_after[good_block, :, t % s.block_size], k_before[good_block, :, t % s.block_size])
