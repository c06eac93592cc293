"""The C-ABI library loads, exports every function include/tv.h declares, and
rejects bad arguments on the host before launching anything (no GPU needed:
every call below returns before its first HIP call)."""
import ctypes
import subprocess

import pytest

import tree_attention_verification_05_amd as T
from tree_attention_verification_05_amd import _lib

lib = T.lib
P16 = 0x10000  # a 16-byte aligned non-null pointer value, never dereferenced


def test_every_declared_symbol_is_exported():
    names = T.header_functions()
    assert set(names) >= {"tv_build_tree_mask", "tv_tree_attention", "tv_accept_greedy",
                          "tv_kv_compact"}
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {l.split()[-1] for l in out.splitlines() if " T " in l}
    for n in names:
        assert n in exported, n
        assert hasattr(lib, n)
    # nothing else leaks out of the library (hidden visibility)
    assert {e for e in exported if e.startswith("tv_")} == set(names)


def test_status_strings():
    for s in range(9):
        assert lib.tv_status_string(s).decode().startswith(
            ["TV_OK", "TV_ERR_NULL", "TV_ERR_SHAPE", "TV_ERR_DTYPE", "TV_ERR_UNSUPPORTED",
             "TV_ERR_ALIGN", "TV_ERR_WORKSPACE", "TV_ERR_LAUNCH", "TV_ERR_TOO_LARGE"][s])
    assert lib.tv_version() >= 100


def test_mask_host_checks():
    assert lib.tv_build_tree_mask(None, 1, 4, P16, None, None, None) == 1
    assert lib.tv_build_tree_mask(P16, 1, 4, None, None, None, None) == 1
    assert lib.tv_build_tree_mask(P16, 0, 4, P16, None, None, None) == 2
    assert lib.tv_build_tree_mask(P16, 1, 257, P16, None, None, None) == 2


def attn(**kw):
    a = dict(q=P16, k=P16, v=P16, nb=10, table=P16, mb=4, bs=16, pl=P16, mpl=40, mask=P16,
             out=P16, B=1, N=8, Hq=8, Hkv=2, D=128, scale=0.0, dt=1, ws=None, wsb=0, st=None,
             stream=None)
    a.update(kw)
    return lib.tv_tree_attention(a["q"], a["k"], a["v"], a["nb"], a["table"], a["mb"], a["bs"],
                                 a["pl"], a["mpl"], a["mask"], a["out"], a["B"], a["N"], a["Hq"],
                                 a["Hkv"], a["D"], a["scale"], a["dt"], a["ws"], a["wsb"], a["st"],
                                 a["stream"])


def test_attention_host_checks():
    assert attn(q=None) == 1 and attn(mask=None) == 1 and attn(out=None) == 1
    assert attn(dt=7) == 3
    # the layout flag combines with a dtype; other bits do not
    assert attn(dt=0x200 | 1) == 3 and attn(dt=0x100 | 7) == 3
    assert attn(Hq=6, Hkv=4) == 2 and attn(B=0) == 2 and attn(N=300) == 2
    assert attn(mpl=57) == 2          # 57 + 8 > 4 blocks * 16
    assert attn(D=96) == 4 and attn(bs=32) == 4
    assert attn(q=P16 + 8) == 5 and attn(k=P16 + 2) == 5 and attn(out=P16 + 4) == 5


def test_attention_from_parents_host_checks():
    """The parents variant: the attention checks, a NULL parent array, and
    trees of more than 64 nodes (one wave builds the masks) refused."""
    f = lib.tv_tree_attention_parents

    def call(**kw):
        a = dict(q=P16, k=P16, v=P16, nb=10, table=P16, mb=8, bs=16, pl=P16, mpl=40, par=P16,
                 out=P16, B=1, N=8, Hq=8, Hkv=2, D=128, scale=0.0, dt=1, ws=None, wsb=0, st=None,
                 stream=None)
        a.update(kw)
        return f(a["q"], a["k"], a["v"], a["nb"], a["table"], a["mb"], a["bs"], a["pl"], a["mpl"], a["par"],
                 a["out"], a["B"], a["N"], a["Hq"], a["Hkv"], a["D"], a["scale"], a["dt"], a["ws"], a["wsb"],
                 a["st"], a["stream"])
    assert call(par=None) == 1 and call(q=None) == 1
    assert call(dt=7) == 3 and call(D=96) == 4
    assert call(N=65) == 4 and call(N=300) == 2
    assert call(q=P16 + 8) == 5


def test_attention_workspace_check():
    need = lib.tv_tree_attention_workspace_size(4, 64, 28, 4, 128, 32768)
    if need:
        assert attn(B=4, N=64, Hq=28, Hkv=4, mpl=32768, mb=2100, ws=None, wsb=0) == 6
        assert attn(B=4, N=64, Hq=28, Hkv=4, mpl=32768, mb=2100, ws=P16, wsb=need - 1) == 6


def test_accept_host_checks():
    f = lib.tv_accept_greedy
    ok = dict(lg=P16, dt=P16, par=P16, B=2, N=8, V=1000, al=P16, an=P16, bt=P16, am=None,
              ws=P16, wsb=1 << 20, st=None, s=None)

    def call(**kw):
        a = dict(ok)
        a.update(kw)
        return f(a["lg"], a["dt"], a["par"], a["B"], a["N"], a["V"], a["al"], a["an"], a["bt"],
                 a["am"], a["ws"], a["wsb"], a["st"], a["s"])
    assert call(lg=None) == 1 and call(bt=None) == 1
    assert call(V=0) == 2 and call(N=257) == 2
    assert call(lg=P16 + 4) == 5
    need = lib.tv_accept_greedy_workspace_size(2, 8, 1000)
    assert need > 0
    assert call(ws=None) == 6 and call(wsb=need - 1) == 6


def test_accept_noalloc_host_checks():
    """The allocation-free variant's host checks, and its size limit: sizes
    whose chunk keys exceed the static scratch are refused before anything
    touches a device."""
    f = lib.tv_accept_greedy_noalloc
    args = lambda **kw: [kw.get("lg", P16), kw.get("dt", P16), kw.get("par", P16), kw.get("B", 2),
                         kw.get("N", 8), kw.get("V", 1000), kw.get("al", P16), kw.get("an", P16),
                         kw.get("bt", P16), None, None, None]
    assert f(*args(lg=None)) == 1 and f(*args(al=None)) == 1 and f(*args(bt=None)) == 1
    assert f(*args(B=0)) == 2 and f(*args(N=257)) == 2 and f(*args(V=0)) == 2
    assert f(*args(lg=P16 + 4)) == 5
    limit = T.TV_ACCEPT_NOALLOC_SCRATCH_BYTES
    # 2048 sequences of 256 nodes: one key per row, 4 MiB exactly, still fits
    assert lib.tv_accept_greedy_workspace_size(2048, 256, 1000) == limit
    # one more sequence does not
    assert lib.tv_accept_greedy_workspace_size(2049, 256, 1000) > limit
    assert f(*args(B=2049, N=256)) == T.TV_ERR_TOO_LARGE


def test_compact_host_checks():
    f = lib.tv_kv_compact

    def call(**kw):
        a = dict(k=P16, v=P16, nb=10, table=P16, mb=4, bs=16, pl=P16, an=P16, al=P16, B=1, N=8,
                 Hkv=2, D=128, dt=1, nl=None, st=None, s=None)
        a.update(kw)
        return f(a["k"], a["v"], a["nb"], a["table"], a["mb"], a["bs"], a["pl"], a["an"], a["al"],
                 a["B"], a["N"], a["Hkv"], a["D"], a["dt"], a["nl"], a["st"], a["s"])
    assert call(k=None) == 1 and call(an=None) == 1
    assert call(dt=2) == 3 and call(dt=0x100 | 2) == 3 and call(dt=0x400 | 1) == 3
    assert call(N=0) == 2 and call(Hkv=0) == 2
    assert call(D=80) == 4 and call(bs=8) == 4
    assert call(v=P16 + 2) == 5


def test_tree_kv_write_host_checks():
    f = lib.tv_tree_kv_write

    def call(**kw):
        a = dict(q=P16, kn=P16, vn=P16, dep=P16, qo=P16, k=P16, v=P16, nb=10, table=P16, mb=4, bs=16,
                 pl=P16, B=1, N=8, Hq=4, Hkv=2, D=128, theta=10000.0, dt=1, st=None, s=None)
        a.update(kw)
        return f(a["q"], a["kn"], a["vn"], a["dep"], a["qo"], a["k"], a["v"], a["nb"], a["table"],
                 a["mb"], a["bs"], a["pl"], a["B"], a["N"], a["Hq"], a["Hkv"], a["D"], a["theta"],
                 a["dt"], a["st"], a["s"])
    assert call(q=None) == 1 and call(dep=None) == 1 and call(qo=None) == 1 and call(v=None) == 1
    assert call(dt=5) == 3
    assert call(B=0) == 2 and call(N=300) == 2 and call(Hq=6, Hkv=4) == 2
    assert call(theta=0.0) == 2 and call(theta=-1.0) == 2
    assert call(D=96) == 4 and call(bs=32) == 4
    assert call(qo=P16 + 4) == 5 and call(kn=P16 + 2) == 5


def test_accept_workspace_grows_with_rows():
    a = lib.tv_accept_greedy_workspace_size(1, 60, 128256)
    b = lib.tv_accept_greedy_workspace_size(128, 9, 128256)
    assert a > 0 and b > 0
    assert lib.tv_accept_greedy_workspace_size(0, 9, 100) == 0


def test_accept_stochastic_host_checks():
    f = lib.tv_accept_stochastic
    need = lib.tv_accept_stochastic_workspace_size(2, 8, 1000)
    assert need > 0 and lib.tv_accept_stochastic_workspace_size(2, 0, 1000) == 0

    def call(**kw):
        a = dict(lg=P16, qp=None, dt=P16, par=P16, u=P16, e=P16, B=2, N=8, V=1000, T=0.7,
                 al=P16, an=P16, bt=P16, ws=P16, wsb=need, st=None, s=None)
        a.update(kw)
        return f(a["lg"], a["qp"], a["dt"], a["par"], a["u"], a["e"], a["B"], a["N"], a["V"], a["T"],
                 a["al"], a["an"], a["bt"], a["ws"], a["wsb"], a["st"], a["s"])
    assert call(lg=None) == 1 and call(u=None) == 1 and call(e=None) == 1 and call(bt=None) == 1
    assert call(B=0) == 2 and call(N=257) == 2 and call(V=0) == 2
    assert call(T=0.0) == 2 and call(T=-1.0) == 2 and call(T=float("inf")) == 2
    assert call(T=float("nan")) == 2
    assert call(lg=P16 + 4) == 5 and call(qp=P16 + 8) == 5
    assert call(ws=None) == 6 and call(wsb=need - 1) == 6
    assert call(ws=P16 + 8) == 5


def test_accept_compact_host_checks():
    """The fused acceptance-and-compaction call: the union of both calls'
    host checks (nothing is launched on an error)."""
    f = lib.tv_accept_greedy_compact
    need = lib.tv_accept_greedy_workspace_size(2, 8, 1000)

    def call(**kw):
        a = dict(lg=P16, dt=P16, par=P16, B=2, N=8, V=1000, al=P16, an=P16, bt=P16, am=None, ws=P16, wsb=need,
                 k=P16, v=P16, nb=10, table=P16, mb=4, bs=16, pl=P16, Hkv=2, D=128, dty=1, nl=None, st=None, s=None)
        a.update(kw)
        return f(a["lg"], a["dt"], a["par"], a["B"], a["N"], a["V"], a["al"], a["an"], a["bt"], a["am"], a["ws"],
                 a["wsb"], a["k"], a["v"], a["nb"], a["table"], a["mb"], a["bs"], a["pl"], a["Hkv"], a["D"],
                 a["dty"], a["nl"], a["st"], a["s"])
    assert call(lg=None) == 1 and call(bt=None) == 1 and call(k=None) == 1 and call(pl=None) == 1
    assert call(V=0) == 2 and call(N=257) == 2 and call(Hkv=0) == 2 and call(nb=0) == 2
    assert call(dty=2) == 3 and call(dty=0x200 | 1) == 3
    assert call(D=96) == 4 and call(bs=32) == 4
    assert call(lg=P16 + 4) == 5 and call(k=P16 + 8) == 5
    assert call(ws=None) == 6 and call(wsb=need - 1) == 6


def test_lm_head_host_checks():
    f = lib.tv_lm_head_argmax
    need = lib.tv_lm_head_argmax_workspace_size(60, 4096, 128256)
    assert need == 60 * 501 * 8 and lib.tv_lm_head_argmax_workspace_size(0, 64, 10) == 0

    def call(**kw):
        a = dict(h=P16, w=P16, M=60, H=4096, V=128256, dt=1, am=P16, mx=None, ws=P16, wsb=need, s=None)
        a.update(kw)
        return f(a["h"], a["w"], a["M"], a["H"], a["V"], a["dt"], a["am"], a["mx"], a["ws"], a["wsb"], a["s"])
    assert call(h=None) == 1 and call(w=None) == 1 and call(am=None) == 1
    assert call(dt=0) == 3
    # the cache-layout flag belongs to the calls that take a cache
    assert call(dt=0x100 | 1) == 3
    assert call(M=0) == 2 and call(V=0) == 2 and call(H=0) == 2 and call(H=1 << 21) == 2
    assert call(H=4000) == 4
    assert call(h=P16 + 2) == 5 and call(w=P16 + 8) == 5
    assert call(ws=None) == 6 and call(wsb=need - 1) == 6
