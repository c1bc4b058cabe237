"""Plant plausible mistakes in copies of the oracle and check the pins catch each.

Each mutant is the oracle's C source with one edit (a flipped sign, a strict
inequality, a wrong head mapping, a dropped term ...), compiled with gcc into a
temporary directory and loaded by a fresh pytest run of ``test_oracle.py``.
The repository's oracle is never modified.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "attn_oracle.c")

MUTANTS = {
    "alibi_sign": ("slope * (double)(j - i)", "slope * (double)(i - j)"),
    "alibi_scaled": ("if (p->alibi) x += slope * (double)(j - i);",
                     "if (p->alibi) x += p->scale * slope * (double)(j - i);"),
    "slope_index": ("-8.0 * (double)(h + 1) / (double)H", "-8.0 * (double)(h) / (double)H"),
    "causal_strict": ("!(j <= i)", "!(j < i)"),
    "window_strict": ("abs(i - j) <= p->window", "abs(i - j) < p->window"),
    "gqa_interleaved": ("const int hk = h / group;", "const int hk = h % p->Hkv;"),
    "no_scale": ("double x = p->scale * dot;", "double x = dot;"),
    "lse_log2": ("*lse = M + log(Lsum);", "*lse = M + log2(Lsum);"),
    "lse_no_max": ("*lse = M + log(Lsum);", "*lse = log(Lsum);"),
    "mask_scaled": ("x += p->add_mask[row * p->mask_ld + j];",
                    "x += p->scale * p->add_mask[row * p->mask_ld + j];"),
    "lens_inclusive": ("j < len;", "j <= len;"),
    "fmix_constant": ("0x85ebca6bu", "0x85ebca6cu"),
    "drop_inverted": ("< threshold;", ">= threshold;"),
    "no_normalise": ("o[d] /= Lsum;", "o[d] /= 1.0;"),
    "full_block_predicated": ("if (blk == 1) {", "if (blk != 0) {"),
    "block_kv_size": ("j / ORACLE_BLOCK_KV];", "j / ORACLE_BLOCK_Q];"),
    "block_empty_kept": ("if (blk == 0) keep = 0;", "if (blk == 3) keep = 0;"),
    "doc_order": ("p->q_doc[b * p->q_doc_sb + i] != p->kv_doc[b * p->kv_doc_sb + j]",
                  "p->q_doc[b * p->q_doc_sb + i] < p->kv_doc[b * p->kv_doc_sb + j]"),
}


# mistakes in the backward, caught by the backward's pins (test_oracle_bwd.py)
MUTANTS_BWD = {
    "bwd_no_row_term": ("const double dsij = pij * (dpij - Di);", "const double dsij = pij * dpij;"),
    "bwd_dk_unscaled": ("dkb[(int64_t)j * D + d] += scale * dsij * qi[d];",
                        "dkb[(int64_t)j * D + d] += dsij * qi[d];"),
    "bwd_dv_from_ds": ("dvb[(int64_t)j * D + d] += pij * doi[d];", "dvb[(int64_t)j * D + d] += dsij * doi[d];"),
    "bwd_dq_from_v": ("dqi[d] += scale * dsij * kb[(int64_t)j * D + d];",
                      "dqi[d] += scale * dsij * vb[(int64_t)j * D + d];"),
    "bwd_group_one_head": ("for (int h = hk * group; h < (hk + 1) * group; ++h) {",
                           "for (int h = hk * group; h < hk * group + 1; ++h) {"),
}


def _run_mutant(name, before, after, tmp_path, test_file):
    src = open(SRC).read()
    assert src.count(before) == 1, name
    c = tmp_path / f"{name}.c"
    so = tmp_path / f"{name}.so"
    c.write_text(src.replace(before, after))
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
                           str(c), "-o", str(so), "-lm"])
    env = dict(os.environ, MASKMODS_ORACLE_LIB=str(so), OMP_NUM_THREADS="2")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", test_file)],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    assert r.returncode != 0, f"mutant {name} survived the pins of {test_file}:\n{r.stdout[-2000:]}"


@pytest.mark.parametrize("name", sorted(MUTANTS_BWD))
def test_backward_pins_catch_planted_mistake(name, tmp_path):
    _run_mutant(name, *MUTANTS_BWD[name], tmp_path, "test_oracle_bwd.py")


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(name, tmp_path):
    before, after = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(before) == 1, name
    c = tmp_path / f"{name}.c"
    so = tmp_path / f"{name}.so"
    c.write_text(src.replace(before, after))
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
                           str(c), "-o", str(so), "-lm"])
    env = dict(os.environ, MASKMODS_ORACLE_LIB=str(so), OMP_NUM_THREADS="2")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    assert r.returncode != 0, f"mutant {name} survived the oracle pins:\n{r.stdout[-2000:]}"
