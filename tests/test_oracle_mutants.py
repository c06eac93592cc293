"""The oracle's pins catch plausible mistakes.

Each case plants one mistake in a copy of the oracle's source (a dropped or
transposed mask term, a wrong GQA index, an off-by-one prefix, a missing
scale, the wrong argmax tie rule, a greedy instead of longest path, the bonus
taken at the wrong node, compaction without gather-before-write, a wrong new
length, a flipped rotation, a wrong rotary frequency or pairing, node index
instead of tree depth as position, and in stochastic acceptance: siblings
tested in the wrong order, the acceptance test reversed, the temperature
dropped, a residual that keeps the rejected mass or is not normalised, the
final draw multiplying instead of dividing, the proposal probability
dropped, the target row of the wrong node; and in the fused LM head: a
dropped hidden column, the score taken from the wrong row; and in draft-tree
construction: the kept nodes taken in candidate order, probabilities added
instead of log-probabilities, nodes numbered by score alone, one drafter row
for every kept node) and runs the pin suites against that copy in a
separate process, on the CPU.  The suites must
fail for every one of them.
"""
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

MUTANTS = {
    "ancestor_mask_transposed": ("visible[:, P:] = anc", "visible[:, P:] = anc.T"),
    "node_does_not_see_itself": ("        anc[i, i] = True\n", ""),
    "gqa_interleaved_heads": (
        "Qg = q[b, :, kh * g:(kh + 1) * g, :].reshape(N * g, D)",
        "Qg = q[b, :, kh::Hkv, :].reshape(N * g, D)"),
    "prefix_off_by_one": ("visible[:, :P] = True", "visible[:, :P-1] = True"),
    "scale_missing": ("s = scale * (Qg @ K[:, kh, :].T)", "s = (Qg @ K[:, kh, :].T)"),
    "argmax_highest_index_on_ties": (
        "return np.argmax(np.asarray(logits), axis=-1).astype(np.int64)",
        "a = np.asarray(logits); "
        "return (a.shape[-1] - 1 - np.argmax(a[..., ::-1], axis=-1)).astype(np.int64)"),
    "first_child_instead_of_longest": ("                if len(cand) > len(best):",
                                       "                if len(best) == 1:"),
    "bonus_at_root": ("return path, int(am[path[-1]])", "return path, int(am[0])"),
    "compaction_in_descending_order": (
        "        ks = kf[src].copy()\n        vs = vf[src].copy()\n"
        "        kf[dst] = ks\n        vf[dst] = vs",
        "        for s_, d_ in zip(src[::-1], dst[::-1]):\n"
        "            kf[d_] = kf[s_]; vf[d_] = vf[s_]"),
    "new_length_without_root": ("new_lens[b] = P + L", "new_lens[b] = P + L - 1"),
    "rope_rotation_sign_flipped": ("[x1 * c - x2 * s, x2 * c + x1 * s]", "[x1 * c + x2 * s, x2 * c - x1 * s]"),
    "rope_frequency_exponent_halved": ("inv = float(theta) ** (-2.0 * np.arange(h, dtype=np.float64) / D)",
                                       "inv = float(theta) ** (-1.0 * np.arange(h, dtype=np.float64) / D)"),
    "rope_interleaved_pairs": ("    x1, x2 = x[..., :h], x[..., h:]\n    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)",
                               "    x1, x2 = x[..., 0::2], x[..., 1::2]\n    y = np.empty_like(x)\n"
                               "    y[..., 0::2] = x1 * c - x2 * s\n    y[..., 1::2] = x2 * c + x1 * s\n    return y"),
    "tree_position_is_node_index": ("pos[b] = int(prefix_lens[b]) + depth", "pos[b] = int(prefix_lens[b]) + np.arange(N)"),
    "stochastic_children_descending": ("        for c in range(cur + 1, N):\n            if parents[c] != cur:\n                continue",
                                       "        for c in range(N - 1, cur, -1):\n            if parents[c] != cur:\n                continue"),
    "stochastic_accept_when_uniform_above": ("            if lhs < r[x]:", "            if lhs > r[x]:"),
    "stochastic_temperature_ignored": ("z = np.asarray(logits_row, dtype=np.float64) / float(temperature)",
                                       "z = np.asarray(logits_row, dtype=np.float64)"),
    "stochastic_residual_keeps_rejected_mass": ("d = np.maximum(np.asarray(r, dtype=np.float64) - q, 0.0)",
                                                "d = np.maximum(np.asarray(r, dtype=np.float64), 0.0)"),
    "stochastic_residual_unnormalised": ("return d / m if m > 0 else np.asarray(r, dtype=np.float64)",
                                         "return d if m > 0 else np.asarray(r, dtype=np.float64)"),
    "stochastic_race_multiplies": ("t = np.asarray(r, dtype=np.float64) / np.asarray(expo, dtype=np.float64)",
                                   "t = np.asarray(r, dtype=np.float64) * np.asarray(expo, dtype=np.float64)"),
    "stochastic_acceptance_ignores_proposal": ("lhs = float(uniforms[c]) * q[x]", "lhs = float(uniforms[c])"),
    "lm_head_drops_last_hidden_column": ("    return h @ w.T", "    return h[:, :-1] @ w[:, :-1].T"),
    "lm_head_max_from_first_row": ("return am, lg[np.arange(lg.shape[0]), am]", "return am, lg[0, am]"),
    "draft_tree_frontier_in_candidate_order": ("        order = sorted(range(len(cands)), key=lambda i: (-cands[i][0], i))",
                                               "        order = list(range(len(cands)))"),
    "draft_tree_adds_probabilities": ("cands.append((fs + lp[t], lev, j, r, int(t), fid))",
                                      "cands.append((fs + np.exp(lp[t]), lev, j, r, int(t), fid))"),
    "draft_tree_numbered_by_score_only": ("keep = sorted(keep, key=lambda g: (gen[g][1], -gen[g][0], gen[g][2], gen[g][3]))",
                                          "keep = sorted(keep, key=lambda g: (-gen[g][0], gen[g][2], gen[g][3]))"),
    "draft_tree_first_row_for_every_slot": ("            lp = log_softmax(lg[lev, j])", "            lp = log_softmax(lg[lev, 0])"),
    "stochastic_target_row_of_child": ("        r = target_probs(logits[cur], temperature)\n        moved = False",
                                       "        r = target_probs(logits[min(cur + 1, N - 1)], temperature)\n        moved = False"),
}

PIN_FILES = [os.path.join("tests", "test_oracle.py"), os.path.join("tests", "test_oracle_stochastic.py"),
             os.path.join("tests", "test_oracle_lmhead.py"), os.path.join("tests", "test_oracle_tree.py")]
COPY = ["pytest.ini", "workloads", os.path.join("tests", "conftest.py"),
        os.path.join("tests", "golden")] + PIN_FILES


def _run_mutant(base, name, old, new):
    src = open(os.path.join(ROOT, "oracle", "__init__.py")).read()
    assert src.count(old) == 1, f"{name}: the planted site is not unique in the oracle"
    d = os.path.join(base, name)
    os.makedirs(os.path.join(d, "tests"))
    os.makedirs(os.path.join(d, "oracle"))
    for rel in COPY:
        s = os.path.join(ROOT, rel)
        if os.path.isdir(s):
            shutil.copytree(s, os.path.join(d, rel), ignore=shutil.ignore_patterns("__pycache__"))
        else:
            shutil.copy(s, os.path.join(d, rel))
    with open(os.path.join(d, "oracle", "__init__.py"), "w") as f:
        f.write(src.replace(old, new))
    env = dict(os.environ, OMP_NUM_THREADS="2", OPENBLAS_NUM_THREADS="2", MKL_NUM_THREADS="2")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        *PIN_FILES], cwd=d, capture_output=True, text=True, env=env,
                       timeout=600)
    tail = (r.stdout.strip().splitlines() or [""])[-1]
    return name, r.returncode, tail


def test_every_planted_mistake_fails_a_pin(tmp_path):
    with ThreadPoolExecutor(max_workers=4) as ex:
        results = list(ex.map(lambda kv: _run_mutant(str(tmp_path), kv[0], *kv[1]),
                              MUTANTS.items()))
    survived = [(n, tail) for n, rc, tail in results if rc == 0]
    broken = [(n, rc, tail) for n, rc, tail in results if rc not in (0, 1)]
    assert not broken, f"mutant runs that did not complete: {broken}"
    assert not survived, f"planted mistakes that no pin caught: {survived}"


def test_unmutated_copy_passes(tmp_path):
    """Control: the same copy procedure with no mistake planted passes."""
    name, rc, tail = _run_mutant(str(tmp_path), "control", "import numpy as np",
                                 "import numpy as np")
    assert rc == 0, tail


if __name__ == "__main__":
    sys.exit(pytest.main([__file__, "-q"]))
