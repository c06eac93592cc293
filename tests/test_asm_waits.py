"""The LDS reads that the attention and LM-head kernels issue as inline
assembly are invisible to the compiler's wait tracking: the compiler takes an
asm output as written when the asm statement ends.  Each kernel therefore
waits for them with an explicit ``s_waitcnt lgkmcnt(0)`` that names the read
destinations as operands.  That is only safe if nothing reads (or copies) a
destination register between the read and the wait.

This test compiles both translation units to gfx950 assembly (device code
only, no GPU needed) and scans every such read: from the read to the next
``s_waitcnt`` that waits for all LDS operations, no instruction may name one
of its destination registers.  The scan is linear over the listing, which
covers the unrolled straight-line tile bodies these reads live in."""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "tree_attention_verification_05_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

_REG = re.compile(r"\bv\[(\d+):(\d+)\]|\bv(\d+)\b")


def _vregs(text: str) -> set:
    out = set()
    for m in _REG.finditer(text):
        if m.group(1):
            out.update(range(int(m.group(1)), int(m.group(2)) + 1))
        else:
            out.add(int(m.group(3)))
    return out


def early_uses(asm: str, opcode: str):
    """(read count, [(line, instruction, registers)]) of instructions that name
    a pending read destination before the wait that covers it."""
    pending = {}
    bad = []
    n = 0
    for i, line in enumerate(asm.splitlines()):
        t = line.split(";")[0].strip()
        if not t or t.startswith(".") or t.endswith(":"):
            continue
        mnem = t.split()[0]
        ops = t[len(mnem):]
        if mnem == "s_waitcnt" and "lgkmcnt(0)" in ops:
            pending.clear()
            continue
        if mnem == opcode:
            n += 1
            for r in _vregs(ops.split(",")[0]):
                pending[r] = i
            continue
        used = _vregs(ops) & pending.keys()
        if used:
            bad.append((i + 1, t, sorted(used)))
    return n, bad


def compile_asm(src: str, tmp_path) -> str:
    out = tmp_path / (os.path.basename(src) + ".s")
    cmd = [HIPCC, "-O3", "-std=c++17", "--offload-arch=gfx950", "--cuda-device-only", "-S",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}", src, "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    return out.read_text()


@pytest.mark.skipif(shutil.which(HIPCC) is None and not os.path.exists(HIPCC), reason="no hipcc")
@pytest.mark.parametrize("src,opcode,min_reads", [
    ("attn_mfma.hip", "ds_read_b64_tr_b16", 64),
    ("lm_head.hip", "ds_read_b128", 16),
])
def test_no_use_of_lds_read_results_before_their_wait(src, opcode, min_reads, tmp_path):
    asm = compile_asm(os.path.join(CSRC, src), tmp_path)
    n, bad = early_uses(asm, opcode)
    assert n >= min_reads, f"{src}: only {n} {opcode} found (did the kernel change form?)"
    assert not bad, f"{src}: {len(bad)} early uses, first {bad[:5]}"


def test_scanner_flags_an_early_copy():
    """The scanner itself: a copy of a pending destination is reported, a use
    after the wait is not."""
    asm = "\n".join([
        "\tds_read_b64_tr_b16 v[10:11], v2 offset:0",
        "\tv_mov_b32 v20, v11",
        "\ts_waitcnt lgkmcnt(0)",
        "\tv_mfma_f32_32x32x16_bf16 v[0:15], v[10:13], v[30:33], v[0:15]",
    ])
    n, bad = early_uses(asm, "ds_read_b64_tr_b16")
    assert n == 1 and len(bad) == 1 and bad[0][2] == [11]
    n, bad = early_uses(asm.replace("\tv_mov_b32 v20, v11\n", ""), "ds_read_b64_tr_b16")
    assert n == 1 and not bad
