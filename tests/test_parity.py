"""GPU parity: every library call against the CPU oracle on the same seeded
inputs.  Masks, argmax, accepted paths and compacted caches must be
bit-exact; attention outputs must satisfy |gpu - oracle| <= 2e-2 + 1e-2*|oracle|
(bf16) or 1e-4 + 1e-4*|oracle| (fp32) element by element, and every
sequence's relative L2 error must stay within 4e-3 (bf16) or 1e-5 (fp32)."""
import dataclasses
import functools

import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from gpu_util import (check_accept, check_attention, host_f, log, oracle_attention, raw_bits,
                      run_step, upload)

pytestmark = pytest.mark.gpu

T = None


def setup_module():
    global T
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import tree_attention_verification_05_amd as lib
    T = lib


@functools.lru_cache(maxsize=2)
def full(i):
    return W.make_config(i)


def verify(w, seqs=None, compact=True, label=""):
    """Run the whole step on the GPU and compare everything with the oracle."""
    log(f"[parity] {label} {w.spec.name} B={w.B} N={w.N} P={w.prefix_lens.min()}..{w.prefix_lens.max()}")
    d = upload(w)
    k0 = raw_bits(w.k_cache)
    v0 = raw_bits(w.v_cache)
    res = run_step(T, d, w.max_prefix_len, compact=compact)
    assert int(d["status"].item()) == 0
    # mask and depth
    mref, dref = O.build_tree_mask(w.parents)
    assert np.array_equal(res["mask"].cpu().numpy().view(np.uint64), mref)
    assert np.array_equal(res["depth"].cpu().numpy(), dref)
    # attention
    seqs = list(range(w.B)) if seqs is None else list(seqs)
    ref = oracle_attention(w, seqs)
    rel = check_attention(res["out"], ref, seqs, w.q.dtype, label=f"{label} {w.spec.name}")
    log(f"[parity]   attention ok on {len(seqs)} sequences, worst relative L2 error {rel:.2e}")
    # acceptance
    aref = O.accept_greedy(w.logits.numpy(), w.draft_tokens, w.parents)
    check_accept(res, aref)
    # compaction: whole caches, bit for bit
    if compact:
        kref, vref, nl = O.kv_compact(k0, v0, w.block_table, w.prefix_lens, aref["accepted_nodes"],
                                      aref["accept_len"])
        assert np.array_equal(res["new_lens"].cpu().numpy(), nl)
        assert np.array_equal(raw_bits(d["k"]), kref)
        assert np.array_equal(raw_bits(d["v"]), vref)
    return res, aref


@pytest.mark.parametrize("i", [1, 2, 3, 4, 5])
def test_small_configs(i):
    verify(W.make_small(i), label=f"small{i}")


@pytest.mark.parametrize("i", [1, 2, 3, 4, 5])
def test_full_config_all_sequences(i):
    """The five workloads at full size, in the launch configuration the
    benchmark times, every sequence compared."""
    verify(full(i), label=f"full{i}")


def test_attention_workspace_reused_across_shapes():
    """One zero-filled workspace serves attention calls of different shapes
    and both schedules in turn: balanced shares that cut sequences (the
    workgroup finishing a cut sequence's last piece merges it, found through
    the arrival counters at the workspace's start) and fixed pieces of one
    sequence (merged by a second kernel).  Every result matches the oracle,
    and the counters (the first 2048 bytes) are zero again after every call,
    as the next call needs them."""
    cases = [("small3", W.make_small(3)), ("small2", W.make_small(2)), ("full3", full(3)),
             ("small5", W.make_small(5)), ("small4", W.make_small(4)), ("small3 again", W.make_small(3))]
    need = max(T.tv_tree_attention_workspace_size(w.B, w.N, w.spec.Hq, w.spec.Hkv, w.spec.D, w.max_prefix_len)
               for _, w in cases)
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    for name, w in cases:
        log(f"[parity] shared attention workspace: {name} B={w.B} N={w.N}")
        d = upload(w)
        out = T.tv_tree_attention_parents(d["q"], d["k"], d["v"], d["table"], d["prefix"], w.max_prefix_len,
                                          d["parents"], workspace=ws, dev_status=d["status"])
        torch.cuda.synchronize()
        assert int(d["status"].item()) == 0
        assert int(torch.count_nonzero(ws[:2048]).item()) == 0, f"{name}: arrival counters not reset"
        seqs = sorted({0, w.B - 1, int(np.argmin(w.prefix_lens)), int(np.argmax(w.prefix_lens))})
        check_attention(out, oracle_attention(w, seqs), seqs, w.q.dtype, label=f"shared workspace {name}")


def mask_revealing(w, planted=(0.1, 0.5, 0.9), seed=0):
    """A copy of workload ``w`` whose tree keys dominate every score (the
    pins' mask-revealing construction) and whose value rows name their source.

    All query rows are sqrt(D) u for one random unit vector u, so with scale
    1/sqrt(D) a key 30 u scores 30 while the N(0, 1) prefix keys score about
    N(0, 1).  Every tree slot P_b + j holds key 30 u and value e_j (one-hot
    at dim j).  In addition the prefix positions floor(f P_b), f in
    ``planted``, hold key 30 u and value e_{N + m}: with a key range split over
    many workgroups they fall in different pieces, so each piece's weight in
    the merge shows in the output.  Node i of sequence b then attends (to
    within 1e-8 of the total weight: P e^0.5 / e^30 at P = 32768) exactly to its ancestors-or-self and the
    planted keys, all with equal weight, and its output is the mean of their
    one-hot rows: a wrong mask bit or a mis-weighted piece moves an entry by at
    least 1 / (depth + 2 + planted), far beyond the tolerance.

    Returns (workload, planted positions per sequence)."""
    spec = w.spec
    D, N = spec.D, w.N
    assert N + len(planted) <= D
    rng = np.random.default_rng([seed, 909])
    u = rng.standard_normal(D)
    u /= np.linalg.norm(u)
    bf = torch.bfloat16
    q = torch.from_numpy(np.broadcast_to(u * np.sqrt(D), tuple(w.q.shape)).copy()).to(bf)
    k = w.k_cache.clone()
    v = w.v_cache.clone()
    key = torch.from_numpy(30.0 * u).to(bf)
    eye = torch.eye(D, dtype=bf)
    bs = spec.block_size
    where = []
    for b in range(w.B):
        P = int(w.prefix_lens[b])
        pos = sorted({int(f * P) for f in planted}) if P > 0 else []
        where.append(pos)
        slots = [(P + j, j) for j in range(N)] + [(t, N + m) for m, t in enumerate(pos)]
        for t, hot in slots:
            blk = int(w.block_table[b, t // bs])
            k[blk, :, t % bs, :] = key
            v[blk, :, t % bs, :] = eye[hot]
    return dataclasses.replace(w, q=q, k_cache=k, v_cache=v), where


def check_mask_revealing(w, where, out):
    """The GPU output against the closed form of ``mask_revealing``."""
    got = host_f(out)
    for b in range(w.B):
        anc, depth = O.tree_structure(w.parents[b])
        for i in range(w.N):
            expect = np.zeros(w.spec.D)
            expect[:w.N] = anc[i]
            expect[w.N:w.N + len(where[b])] = 1.0
            expect /= expect.sum()
            err = np.abs(got[b, i] - expect[None, :]).max()
            assert err <= 1e-2, f"seq {b} node {i}: {err:.3e} from the closed form"


@pytest.mark.parametrize("i", [3, 4])
def test_mask_revealing_full_size(i):
    """The mask-revealing construction on the batched workload's ragged
    prefixes (512..8192) and on the long-context workload (four prefixes of
    32768, each split over many workgroups and merged)."""
    w, where = mask_revealing(full(i), seed=i)
    res, _ = verify(w, label=f"mask-revealing{i}")
    check_mask_revealing(w, where, res["out"])


def test_mask_revealing_ragged_small():
    """The same construction on prefixes of 0..47 tokens (no planted keys
    where the prefix is empty)."""
    w, where = mask_revealing(_variant(5, name="ragged-mr", tag=117, B=12,
                                       prefix_lengths=(0, 1, 2, 5, 17, 31, 47, 0, 33, 16, 15, 3)), seed=5)
    res, _ = verify(w, label="mask-revealing small")
    check_mask_revealing(w, where, res["out"])


def _variant(i, **kw):
    return W.build(dataclasses.replace(W.SMALL[i], **kw))


def test_single_node_tree():
    """N = 1: each sequence verifies only its root (single-token decode)."""
    w = _variant(3, name="n1", tag=101, tree=("uniform", 1, 0))
    res, aref = verify(w, label="N=1")
    assert (aref["accept_len"] == 0).all()


def test_empty_and_tiny_prefix():
    """Prefix lengths 0..3: attention over the tree keys alone or nearly."""
    w = _variant(3, name="p0", tag=102, prefix=(0, 3), B=6)
    verify(w, label="P<=3")


def test_prefix_not_multiple_of_block():
    w = _variant(5, name="ragged", tag=103, prefix=(17, 47), B=12)
    assert (w.prefix_lens % 16 != 0).any()
    verify(w, label="ragged")


def test_head_dim_64_bf16():
    w = _variant(3, name="d64", tag=104, D=64, Hq=8, Hkv=2, dtype="bf16")
    verify(w, label="D=64")


def test_head_dim_64_bf16_single_sequence():
    """One sequence (fixed pieces with the deep ring) at head dim 64."""
    w = _variant(2, name="d64-b1", tag=116, D=64, Hq=8, Hkv=2)
    assert w.B == 1
    verify(w, label="D=64 B=1")


def test_fp32_d128():
    w = _variant(2, name="f32d128", tag=105, dtype="f32", prefix=300)
    verify(w, label="fp32 D=128")


def test_all_match_and_all_miss():
    w = _variant(3, name="allmatch", tag=106, match=1.0)
    _, aref = verify(w, label="all-match")
    assert aref["accept_len"].min() > 0
    w = _variant(3, name="allmiss", tag=107, match=0.0)
    _, aref = verify(w, label="all-miss")
    assert (aref["accept_len"] == 0).all()


def test_many_sequences_four_wave_schedule():
    """More sequences than one workgroup scans at once (the share schedule's
    prefix sum runs over several chunks), most shares spanning many short
    sequences, some prefixes empty."""
    w = _variant(3, name="many-seq", tag=108, B=600, prefix=(0, 200), V=1000)
    assert (w.prefix_lens == 0).any()
    verify(w, label="B=600 4-wave")


def test_many_sequences_eight_wave_schedule():
    """The eight-wave, two-row-chunk layout with more sequences than one
    eight-wave workgroup scans at once."""
    w = _variant(4, name="many-seq-8w", tag=109, B=520, prefix=(0, 120), V=1000)
    verify(w, label="B=520 8-wave")


def test_mixed_empty_short_and_long_prefixes():
    """One long prefix among empty and short ones: the long sequence is split
    over many shares while single shares cover several short sequences, and
    the batch's total is far below its upper bound so that many workgroups
    find no tiles at all."""
    lengths = (0, 0, 5000, 1, 0, 17, 31, 32, 33, 63, 64, 65, 0, 2047, 3, 0, 511, 0, 1, 700)
    w = _variant(3, name="mixed", tag=110, B=len(lengths), prefix_lengths=lengths, V=1000)
    verify(w, label="mixed lengths")
    w = _variant(4, name="mixed-8w", tag=111, B=6, prefix_lengths=(0, 4100, 0, 5, 0, 1500),
                 V=1000)
    verify(w, label="mixed lengths 8-wave")


@pytest.mark.parametrize("batch", [1, 3])
def test_largest_tree(batch):
    """N at its maximum of 256 nodes (four 64-bit mask words per row, eight
    (one sequence) or four (batched) row chunks per KV head)."""
    w = _variant(3, name=f"n256-b{batch}", tag=112 + batch, B=batch, tree=("uniform", 256, 9),
                 prefix=(100, 400), V=1000)
    assert w.N == 256
    verify(w, label=f"N=256 B={batch}")


def test_argmax_ties_and_signed_zero():
    """Exact ties (lowest index wins), maxima at index 0 and V-1, and rows
    whose maximum is a mix of -0.0 and +0.0."""
    w = W.make_small(3, seed=5)
    lg = w.logits.numpy()
    rng = np.random.default_rng(0)
    B, N, V = lg.shape
    for b in range(B):
        for i in range(N):
            kind = (b * N + i) % 5
            row = lg[b, i]
            kids = [c for c in range(N) if w.parents[b, c] == i]
            if kind == 0 and kids:      # tie between a child's token and a lower index
                t = int(w.draft_tokens[b, kids[0]])
                lo = int(rng.integers(0, max(t, 1)))
                row[t] = row.max() + 1
                row[lo] = row[t]
            elif kind == 1:             # signed zeros as the maximum
                row[:] = -np.abs(row) - 1
                row[int(rng.integers(0, V))] = -0.0
                row[int(rng.integers(0, V))] = 0.0
            elif kind == 2:
                row[V - 1] = row.max() + 1
            elif kind == 3:
                row[0] = row.max() + 1
    w.logits = torch.from_numpy(lg)
    verify(w, label="ties")


def test_shared_sibling_tokens_longest_path():
    """Siblings that carry the same token: the longest accepted path wins."""
    w = W.make_small(3, seed=6)
    par = w.parents.copy()
    draft = w.draft_tokens.copy()
    lg = w.logits.numpy()
    for b in range(w.B):
        for p in range(w.N):
            kids = [c for c in range(w.N) if par[b, c] == p]
            if len(kids) >= 2:
                draft[b, kids[1]] = draft[b, kids[0]]
                lg[b, p, draft[b, kids[0]]] = lg[b, p].max() + 1
    w.draft_tokens = draft
    w.logits = torch.from_numpy(lg)
    verify(w, label="shared-siblings")


def token_major(t: torch.Tensor) -> torch.Tensor:
    """[num_blocks, Hkv, 16, D] <-> [num_blocks, 16, Hkv, D] (the swap is its
    own inverse)."""
    return t.permute(0, 2, 1, 3).contiguous()


@pytest.mark.parametrize("which", ["small1", "small3", "full2", "full3", "full4"])
def test_token_major_cache_layout(which):
    """The step on token-major caches ([num_blocks, 16, Hkv, D], selected by
    the TV_KV_TOKEN_MAJOR flag): attention is bit-identical to the same call
    on head-major caches (only the copy source addresses differ) and within
    the oracle's bounds; acceptance and compaction are bit-exact against the
    oracle, the compacted caches compared once put back in head-major order.
    Covers the fp32 path (small1), one sequence in fixed pieces (full2),
    balanced shares (small3, full3) and four row chunks per KV head (full4)."""
    w = W.make_small(int(which[-1])) if which.startswith("small") else full(int(which[-1]))
    log(f"[parity] token-major {which} {w.spec.name} B={w.B} N={w.N}")
    d = upload(w)
    st = d["status"]
    mask, _ = T.tv_build_tree_mask(d["parents"], dev_status=st)
    out_hm = T.tv_tree_attention(d["q"], d["k"], d["v"], d["table"], d["prefix"], w.max_prefix_len, mask,
                                 dev_status=st)
    k_tm, v_tm = token_major(d["k"]), token_major(d["v"])
    del d["k"], d["v"]
    out_tm = T.tv_tree_attention(d["q"], k_tm, v_tm, d["table"], d["prefix"], w.max_prefix_len, mask,
                                 dev_status=st, token_major=True)
    al, an, bt, am = T.tv_accept_greedy(d["logits"], d["draft"], d["parents"], dev_status=st)
    nl = T.tv_kv_compact(k_tm, v_tm, d["table"], d["prefix"], an, al, dev_status=st, token_major=True)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    assert torch.equal(out_tm.view(torch.int16) if out_tm.dtype == torch.bfloat16 else out_tm.view(torch.int32),
                       out_hm.view(torch.int16) if out_hm.dtype == torch.bfloat16 else out_hm.view(torch.int32))
    seqs = list(range(w.B))
    check_attention(out_tm, oracle_attention(w, seqs), seqs, w.q.dtype, label=f"token-major {which}")
    aref = O.accept_greedy(w.logits.numpy(), w.draft_tokens, w.parents)
    check_accept(dict(argmax=am, accept_len=al, accepted_nodes=an, bonus=bt), aref)
    kref, vref, nlref = O.kv_compact(raw_bits(w.k_cache), raw_bits(w.v_cache), w.block_table, w.prefix_lens,
                                     aref["accepted_nodes"], aref["accept_len"])
    assert np.array_equal(nl.cpu().numpy(), nlref)
    assert np.array_equal(raw_bits(token_major(k_tm)), kref)
    assert np.array_equal(raw_bits(token_major(v_tm)), vref)


def test_repeated_runs_bitwise_identical():
    w = W.make_small(2)
    d = upload(w)
    r1 = run_step(T, d, w.max_prefix_len, compact=False)
    r2 = run_step(T, d, w.max_prefix_len, compact=False)
    assert torch.equal(r1["out"], r2["out"])
    assert torch.equal(r1["argmax"], r2["argmax"])


def test_fused_merge_bitwise_identical_across_runs():
    """On the batched workload the workgroup that completes a cut sequence
    merges it, and which workgroup that is depends on timing; the pieces are
    still folded in share order, so repeated calls give identical bits."""
    w = full(3)
    log(f"[parity] fused merge repeatability: {w.spec.name} B={w.B}")
    d = upload(w)
    outs = [T.tv_tree_attention_parents(d["q"], d["k"], d["v"], d["table"], d["prefix"], w.max_prefix_len,
                                        d["parents"], dev_status=d["status"]) for _ in range(4)]
    torch.cuda.synchronize()
    assert int(d["status"].item()) == 0
    for o in outs[1:]:
        assert torch.equal(o.view(torch.int16), outs[0].view(torch.int16))


def test_device_status_bits():
    w = W.make_small(3, seed=7)
    # bad tree in sequence 1, out-of-range token in sequence 2, bad block in sequence 3
    par = w.parents.copy()
    par[1, 3] = 5
    draft = w.draft_tokens.copy()
    draft[2, 4] = w.spec.V
    table = w.block_table.copy()
    table[3, int(w.prefix_lens[3]) // 16] = w.num_blocks   # the block holding sequence 3's root
    w.parents, w.draft_tokens, w.block_table = par, draft, table
    d = upload(w)
    st = d["status"]
    mask, _ = T.tv_build_tree_mask(d["parents"], dev_status=st)
    torch.cuda.synchronize()
    assert int(st.item()) == T.TV_DEV_BAD_TREE
    assert (mask[1] == 0).all()
    st.zero_()
    T.tv_tree_attention(d["q"], d["k"], d["v"], d["table"], d["prefix"], w.max_prefix_len, mask,
                        dev_status=st)
    torch.cuda.synchronize()
    assert int(st.item()) & T.TV_DEV_BAD_CACHE
    st.zero_()
    al, an, bt, am = T.tv_accept_greedy(d["logits"], d["draft"], d["parents"], dev_status=st)
    torch.cuda.synchronize()
    assert int(st.item()) == T.TV_DEV_BAD_TREE | T.TV_DEV_BAD_TOKEN
    assert al[1].item() == 0 and al[2].item() == 0
    # the untouched sequences are still exact
    aref = O.accept_greedy(w.logits.numpy(), w.draft_tokens, w.parents.clip(-1, None))
    for b in (0, 4):
        assert al[b].item() == aref["accept_len"][b]
    st.zero_()
    T.tv_kv_compact(d["k"], d["v"], d["table"], d["prefix"], an, al, dev_status=st)
    torch.cuda.synchronize()
    assert int(st.item()) & T.TV_DEV_BAD_CACHE


def test_device_status_on_fused_merge_schedule():
    """Forty sequences: enough segments that cut sequences are merged inside
    the attention kernel.  A block id outside the cache in one sequence and a
    prefix length above max_prefix_len in another are reported
    (TV_DEV_BAD_CACHE); every other sequence, cut ones included, still
    matches the oracle, and the arrival counters end at zero."""
    w0 = _variant(3, name="fused-status", tag=111, B=40, prefix=(100, 600), V=1000)
    bad_block, bad_len = 5, 9
    table = w0.block_table.copy()
    table[bad_block, 0] = w0.num_blocks
    prefix = w0.prefix_lens.copy()
    prefix[bad_len] = w0.max_prefix_len + 10
    w = dataclasses.replace(w0, block_table=table, prefix_lens=prefix)
    log(f"[parity] device status on the fused merge schedule: B={w.B}")
    d = upload(w)
    # the bound the caller states stays that of the intact batch
    mpl = w0.max_prefix_len
    need = T.tv_tree_attention_workspace_size(w.B, w.N, w.spec.Hq, w.spec.Hkv, w.spec.D, mpl)
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    out = T.tv_tree_attention_parents(d["q"], d["k"], d["v"], d["table"], d["prefix"], mpl,
                                      d["parents"], workspace=ws, dev_status=d["status"])
    torch.cuda.synchronize()
    assert int(d["status"].item()) == T.TV_DEV_BAD_CACHE
    assert int(torch.count_nonzero(ws[:2048]).item()) == 0
    seqs = [b for b in range(w.B) if b not in (bad_block, bad_len)]
    check_attention(out, oracle_attention(w0, seqs), seqs, w.q.dtype, label="fused-merge status")


@pytest.mark.parametrize("which", ["small1", "small2", "small3", "small4", "small5", "full2", "full3", "full4",
                                   "full5", "small3-token-major", "bad-tree", "n64"])
def test_attention_from_parents(which):
    """tv_tree_attention_parents (masks built in the attention kernels from
    the parent array) against tv_build_tree_mask + tv_tree_attention on the
    same inputs: bit-identical outputs and device status, and within the
    oracle's bounds.  'bad-tree' breaks sequence 1's tree (its nodes then see
    no tree key, as the mask kernel leaves them); 'n64' is the largest tree
    one wave handles."""
    tm = which.endswith("token-major")
    if which == "bad-tree":
        w = W.make_small(3, seed=11)
        par = w.parents.copy()
        par[1, 4] = 7
        w.parents = par
    elif which == "n64":
        w = _variant(3, name="n64", tag=121, tree=("uniform", 64, 9), B=3)
        assert w.N == 64
    elif which.startswith("small"):
        w = W.make_small(int(which[5]))
    else:
        w = full(int(which[-1]))
    log(f"[parity] attention from parents {which} {w.spec.name} B={w.B} N={w.N}")
    d = upload(w)
    if tm:
        d["k"], d["v"] = token_major(d["k"]), token_major(d["v"])
    st1 = torch.zeros(1, dtype=torch.int32, device="cuda")
    st2 = torch.zeros(1, dtype=torch.int32, device="cuda")
    mask, _ = T.tv_build_tree_mask(d["parents"], dev_status=st1)
    out1 = T.tv_tree_attention(d["q"], d["k"], d["v"], d["table"], d["prefix"], w.max_prefix_len, mask,
                               dev_status=st1, token_major=tm)
    out2 = T.tv_tree_attention_parents(d["q"], d["k"], d["v"], d["table"], d["prefix"], w.max_prefix_len,
                                       d["parents"], dev_status=st2, token_major=tm)
    torch.cuda.synchronize()
    assert int(st1.item()) == int(st2.item())
    assert np.array_equal(raw_bits(out1), raw_bits(out2))
    if which == "bad-tree":
        assert int(st2.item()) == T.TV_DEV_BAD_TREE
        return
    assert int(st2.item()) == 0
    seqs = list(range(w.B))
    check_attention(out2, oracle_attention(w, seqs), seqs, w.q.dtype, label=f"from parents {which}")


@pytest.mark.parametrize("which", ["small1", "small2", "small3", "small4", "small5", "full2", "full3", "full5",
                                   "small3-token-major", "statuses"])
def test_accept_compact_fused(which):
    """tv_accept_greedy_compact against the two separate calls on copies of
    the same inputs: identical outputs, caches, new lengths and device status
    bits, byte for byte; and against the oracle.  'statuses' plants a bad
    tree (sequence 1), an out-of-range token (2) and a block id outside the
    cache in the tree region (3): the separate calls and the fused one must
    report and write the same."""
    tm = which.endswith("token-major")
    if which == "statuses":
        w = W.make_small(3, seed=7)
        par, draft, table = w.parents.copy(), w.draft_tokens.copy(), w.block_table.copy()
        par[1, 3] = 5
        draft[2, 4] = w.spec.V
        table[3, int(w.prefix_lens[3]) // 16] = w.num_blocks
        w.parents, w.draft_tokens, w.block_table = par, draft, table
    elif which.startswith("small"):
        w = W.make_small(int(which[5]))
    else:
        w = full(int(which[-1]))
    log(f"[parity] accept+compact {which} {w.spec.name} B={w.B} N={w.N}")
    d = upload(w)
    k2, v2 = d["k"].clone(), d["v"].clone()
    if tm:
        d["k"], d["v"] = token_major(d["k"]), token_major(d["v"])
        k2, v2 = token_major(k2), token_major(v2)
    st1 = torch.zeros(1, dtype=torch.int32, device="cuda")
    st2 = torch.zeros(1, dtype=torch.int32, device="cuda")
    al, an, bt, am = T.tv_accept_greedy(d["logits"], d["draft"], d["parents"], dev_status=st1)
    nl = T.tv_kv_compact(d["k"], d["v"], d["table"], d["prefix"], an, al, dev_status=st1, token_major=tm)
    al2, an2, bt2, am2, nl2 = T.tv_accept_greedy_compact(d["logits"], d["draft"], d["parents"], k2, v2, d["table"],
                                                         d["prefix"], dev_status=st2, token_major=tm)
    torch.cuda.synchronize()
    assert int(st1.item()) == int(st2.item())
    for x, y in ((al, al2), (an, an2), (bt, bt2), (am, am2)):
        assert torch.equal(x, y)
    ok = [b for b in range(w.B) if which != "statuses" or b not in (3,)]
    assert torch.equal(nl[ok], nl2[ok])  # a sequence left untouched gets no new length from either call
    assert np.array_equal(raw_bits(d["k"]), raw_bits(k2)) and np.array_equal(raw_bits(d["v"]), raw_bits(v2))
    if which == "statuses":
        assert int(st2.item()) == T.TV_DEV_BAD_TREE | T.TV_DEV_BAD_TOKEN | T.TV_DEV_BAD_CACHE
        return
    assert int(st2.item()) == 0
    aref = O.accept_greedy(w.logits.numpy(), w.draft_tokens, w.parents)
    check_accept(dict(argmax=am2, accept_len=al2, accepted_nodes=an2, bonus=bt2), aref)
    kref, vref, nlref = O.kv_compact(raw_bits(w.k_cache), raw_bits(w.v_cache), w.block_table, w.prefix_lens,
                                     aref["accepted_nodes"], aref["accept_len"])
    assert np.array_equal(nl2.cpu().numpy(), nlref)
    kk, vv = (token_major(k2), token_major(v2)) if tm else (k2, v2)
    assert np.array_equal(raw_bits(kk), kref) and np.array_equal(raw_bits(vv), vref)


def test_python_binding_rejects_host_tensors():
    w = W.make_small(1)
    with pytest.raises(ValueError):
        T.tv_build_tree_mask(torch.from_numpy(w.parents))


def test_accept_workspace_reused_across_batch_sizes():
    """One cached workspace serves calls of growing and shrinking batch size:
    every key a call reads was written by the same call, so nothing stale
    from a larger earlier call leaks into a smaller later one."""
    for i, seed in ((5, 1), (3, 2), (5, 3), (1, 4)):
        w = W.make_small(i, seed=seed, dense=False)
        d = {"logits": w.logits.cuda(), "draft": torch.from_numpy(w.draft_tokens).cuda(),
             "parents": torch.from_numpy(w.parents).cuda()}
        log(f"[parity] accept workspace reuse: small{i} B={w.B}")
        al, an, bt, am = T.tv_accept_greedy(d["logits"], d["draft"], d["parents"])
        torch.cuda.synchronize()
        ref = O.accept_greedy(w.logits.numpy(), w.draft_tokens, w.parents)
        check_accept(dict(accept_len=al, accepted_nodes=an, bonus=bt, argmax=am), ref)


def test_accept_workspace_per_stream():
    """Acceptance calls on two streams at once: each stream gets its own
    cached workspace, and both results stay exact."""
    from tree_attention_verification_05_amd import _lib
    cases = [W.make_small(3, seed=11, dense=False), W.make_small(5, seed=12, dense=False)]
    inputs = [(w.logits.cuda(), torch.from_numpy(w.draft_tokens).cuda(), torch.from_numpy(w.parents).cuda())
              for w in cases]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = []
    for s, x in zip(streams, inputs):
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            outs.append(T.tv_accept_greedy(*x))
    torch.cuda.synchronize()
    keys = {k for k in _lib._cached_ws if k[1] in (streams[0].cuda_stream, streams[1].cuda_stream) and k[2] == 0}
    assert len(keys) == 2
    for w, (al, an, bt, am) in zip(cases, outs):
        ref = O.accept_greedy(w.logits.numpy(), w.draft_tokens, w.parents)
        check_accept(dict(accept_len=al, accepted_nodes=an, bonus=bt, argmax=am), ref)
