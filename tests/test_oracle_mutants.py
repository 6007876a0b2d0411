"""Planted mistakes in the CPU oracle are caught by its pins (no GPU).

Each mutant is the committed ``oracle/smla_oracle.c`` with one plausible
mistake substituted in (a dropped term, a wrong sign, a wrong index or
offset, an ignored input, an off-by-one in the mask). It is compiled with gcc
into a temporary directory and must fail at least one pin.
"""

import os
import subprocess

import pytest

import oracle
from tests import cases as C
from tests import pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "smla_oracle.c")

MUTANTS = {
    "drop_scale": ("return p->scale * acc;", "return acc;"),
    "exp_sign": ("exp(score(&p, qrow, g, &ri, j) - (double)lse[g])",
                 "exp((double)lse[g] - score(&p, qrow, g, &ri, j))"),
    "no_div_G": ("psum / (double)G", "psum"),
    "lse_head0": ("(double)lse[g])", "(double)lse[0])"),
    "q_head0": ("const float* qg = qrow + g * p->D;", "const float* qg = qrow;"),
    "tnd_no_col0": ("kwide ? t : ri.col0 + j;", "kwide ? t : j;"),
    "seqused_k_ignored": ("j >= ri->k_used) return -1;", "j >= ri->s2) return -1;"),
    "seqused_q_ignored": ("if (ri->i >= ri->q_used) return 0;", ""),
    "seqused_k_off_by_one": ("clamp64(p->su_k[ri->b], 0, ri->s2)",
                             "clamp64(p->su_k[ri->b] + 1, 0, ri->s2)"),
    "kwide_key_column": ("kwide ? t : ri.col0 + j;", "ri.col0 + j;"),
    "tnd_global_k": ("p->k + (ri->kbase + j) * p->D", "p->k + j * p->D"),
    "causal_off_by_one": ("(j + 1) * r <= ri->i + 1 +", "(j + 1) * r <= ri->i + 2 +"),
    "causal_strict": ("(j + 1) * r <= ri->i", "(j + 1) * r < ri->i"),
    "ignore_residual": ("int64_t res = p->cmp_res ? p->cmp_res[ri->b] : 0;",
                        "int64_t res = 0;"),
    "ignore_cmp_ratio": ("int64_t r = p->cmp_ratio;", "int64_t r = 1;"),
    "ignore_topk_length": ("if (!p->topk_len) {", "if (1) {"),
    "no_visible_cap": ("return nvis < p->K ? nvis : p->K;", "return p->K;"),
    "dense_drops_last_key": ("if (!p->idx) return ri->s2;", "if (!p->idx) return ri->s2 - 1;"),
    "lse_no_max_shift": ("lse = m + log(sum);", "lse = log(sum);"),
    "no_mask": ("if (p->mask_mode == 0) return 1;", "return 1;"),
    "s1_for_s2": ("ri->i + 1 + ri->s2 * r + res - ri->s1",
                  "ri->i + 1 + ri->s1 * r + res - ri->s2"),
}

CASES = C.tiny_cases()


def _build(tmp_path, name, old, new):
    src = open(SRC).read()
    assert src.count(old) >= 1, f"mutant {name}: pattern not found"
    mut = src.replace(old, new)
    cpath = tmp_path / f"{name}.c"
    cpath.write_text(mut)
    so = tmp_path / f"lib{name}.so"
    subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-o", str(so),
                           str(cpath), "-lm"])
    return oracle.COracle(str(so))


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(tmp_path, name):
    old, new = MUTANTS[name]
    orc = _build(tmp_path, name, old, new)
    failed = []
    for pin in pins.ALL_PINS:
        try:
            pin(orc, CASES)
        except (AssertionError, ValueError):  # ValueError: the oracle's own range check
            failed.append(pin.__name__)
    try:
        pins.pin_hand(orc)
    except AssertionError:
        failed.append("pin_hand")
    assert failed, f"mutant {name} passed every pin"
