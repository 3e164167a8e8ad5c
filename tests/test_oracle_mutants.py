"""The oracle's pins catch plausible mistakes.

Each case copies ``oracle/oracle.c`` to a temporary directory, plants one mistake by
a textual substitution (a wrong GQA index, an off-by-one causal bound, a transposed
V layout, a dropped scale or max term, swapped fusion weights, ...), builds it with
gcc and runs the pin checks of ``test_oracle.py`` against it.  Every mutant must
fail at least one pin; the unmodified source must pass all of them.  Nothing here
touches the GPU or the product library.
"""
import math
import os
import shutil
import subprocess

import numpy as np
import pytest

import oracle
import workloads as W
from tests.test_oracle import (_hand_workload, brute_attention, dense_rows, sdpa_reference,
                               tiny_spec, GOLDEN)

SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle.c")

MUTANTS = {
    "gqa_index_modulo": ("int hk = h / g;", "int hk = h % p->num_kv_heads;"),
    "causal_drops_current_token": ("long visible = (long)p->sys_len + pos + 1;",
                                   "long visible = (long)p->sys_len + pos;"),
    "causal_sees_one_future_token": ("long visible = (long)p->sys_len + pos + 1;",
                                     "long visible = (long)p->sys_len + pos + 2;"),
    "multi_token_ignores_position": ("int pos = p->ctx_lens[b] - n_b + (t - p->cu_q_lens[b]);",
                                     "int pos = p->ctx_lens[b] - 1;"),
    "scale_dropped": ("    s *= p->scale;\n", "\n"),
    "lse_without_max": ("*lse = m + log(zv);", "*lse = log(zv);"),
    "ctx_v_read_key_major": (
        "(((size_t)blk * p->num_kv_heads + hk) * d + c) * ORACLE_BLOCK + j % ORACLE_BLOCK",
        "(((size_t)blk * p->num_kv_heads + hk) * ORACLE_BLOCK + j % ORACLE_BLOCK) * d + c"),
    "sys_v_read_key_major": (
        "(((size_t)hk * ntile + j / ORACLE_SYS_TILE) * d + c) * ORACLE_SYS_TILE +\n"
        "                    j % ORACLE_SYS_TILE",
        "((size_t)hk * ntile * ORACLE_SYS_TILE + j) * d + c"),
    "block_table_slot_swapped": (
        "int blk = p->block_tables[(size_t)b * p->max_blocks_per_seq + j / ORACLE_BLOCK];\n"
        "  return elem(p->ctx_k,",
        "int blk = p->block_tables[(size_t)b * p->max_blocks_per_seq + j % ORACLE_BLOCK %"
        " p->max_blocks_per_seq];\n  return elem(p->ctx_k,"),
    "request_lookup_off_by_one": ("p->cu_q_lens[b + 1] <= t", "p->cu_q_lens[b + 1] < t"),
    "fusion_weights_swapped": (
        "out[r * d + c] = as * o_s[r * d + c] + ac * o_c[r * d + c];",
        "out[r * d + c] = ac * o_s[r * d + c] + as * o_c[r * d + c];"),
    "fusion_lse_drops_log1p": ("l = ls + log1p(e);", "l = ls;"),
    "merge_drops_last_part": ("for (int i = 0; i < k; ++i) acc_add(&z,",
                              "for (int i = 0; i + 1 < k; ++i) acc_add(&z,"),
    "value_sum_drops_first_key": (
        "for (long j = lo; j < hi; ++j) acc_add(&o,", "for (long j = lo + 1; j < hi; ++j) acc_add(&o,"),
}


def _build(tmp_path, name, subst):
    src = open(SRC).read()
    if subst is not None:
        old, new = subst
        assert src.count(old) >= 1, f"mutant {name}: pattern not found"
        src = src.replace(old, new, 1)
    d = tmp_path / name
    d.mkdir()
    (d / "oracle.c").write_text(src)
    lib = str(d / "liboracle.so")
    subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-o", lib,
                           str(d / "oracle.c"), "-lm"])
    return oracle.load_library(lib)


def _close(a, b, tol):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    if b.ndim and a.shape != b.shape:
        return False
    same_inf = np.isinf(a) & np.isinf(b) & (np.sign(a) == np.sign(b))
    with np.errstate(invalid="ignore"):
        return bool(np.all(same_inf | (np.abs(a - b) <= tol)))


def pins_pass(lib) -> bool:
    """The pin checks of test_oracle.py, run against an arbitrary oracle build."""
    import json
    # brute force, tiny shapes (GQA, multi-token, zero system)
    for i, kw in enumerate([dict(B=3, Hq=4, Hkv=2, d=4, Ls=2, lo=1, hi=33),
                            dict(B=2, Hq=4, Hkv=1, d=4, Ls=17, lo=3, hi=20, qlo=1, qhi=3),
                            dict(B=2, Hq=4, Hkv=4, d=2, Ls=0, lo=1, hi=17, qlo=1, qhi=2)]):
        w = W.generate(tiny_spec(40 + i, **kw), keep_dense=True)
        P = oracle.Problem(w, lib=lib)
        out, lse = P.attention()
        o_s, l_s = P.system_part()
        o_c, l_c = P.context_part()
        Ls = w.spec.sys_len
        for t, h, qrow, keys, vals in dense_rows(w):
            r, rl = brute_attention(qrow, keys, vals, w.spec.scale)
            rs, rls = brute_attention(qrow, keys[:Ls], vals[:Ls], w.spec.scale)
            rc, rlc = brute_attention(qrow, keys[Ls:], vals[Ls:], w.spec.scale)
            if not (_close(out[t, h], r, 1e-13) and _close(lse[t, h], rl, 1e-13)
                    and _close(o_s[t, h], rs, 1e-13) and _close(l_s[t, h], rls, 1e-13)
                    and _close(o_c[t, h], rc, 1e-13) and _close(l_c[t, h], rlc, 1e-13)):
                return False
    # library routine
    w = W.generate(W.config_spec(5).replace(batch=4, sys_len=130, ctx_lo=20, ctx_hi=70), keep_dense=True)
    out, lse = oracle.Problem(w, lib=lib).attention()
    ref, ref_lse = sdpa_reference(w)
    if not (_close(out, ref, 1e-12) and _close(lse, ref_lse, 1e-12)):
        return False
    # closed forms
    with open(os.path.join(GOLDEN, "closed_form_cases.json")) as f:
        for case in json.load(f)["cases"]:
            w = _hand_workload(case["q"], case["system"], case["context"], None)
            P = oracle.Problem(w, scale=case["scale"], lib=lib)
            out, lse = P.attention()
            if not (_close(out[0, 0], case["out"], 1e-14) and _close(lse[0, 0], case["lse"], 1e-14)):
                return False
    # relay identity: split == unsplit, weights convex, k-way merge
    w = W.generate(tiny_spec(45, B=3, Hq=4, Hkv=2, d=8, Ls=40, lo=5, hi=60, qlo=1, qhi=4))
    P = oracle.Problem(w, lib=lib)
    out, lse = P.attention()
    o_s, l_s = P.system_part()
    o_c, l_c = P.context_part()
    f, fl, alpha = oracle.relay_fuse(o_s, l_s, o_c, l_c, lib=lib)
    if not (_close(f, out, 1e-12) and _close(fl, lse, 1e-12) and np.all(alpha >= 0)
            and _close(alpha.sum(-1), 1.0, 1e-15)):
        return False
    cuts = [0, 3, 17, 40, 52, 1 << 30]
    parts = [P.attention_range(cuts[i], cuts[i + 1]) for i in range(len(cuts) - 1)]
    m, ml = oracle.merge([p[0] for p in parts], [p[1] for p in parts], lib=lib)
    return _close(m, out, 1e-12) and _close(ml, lse, 1e-12)


def test_unmodified_oracle_passes_pins(tmp_path):
    assert pins_pass(_build(tmp_path, "original", None))


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(tmp_path, name):
    assert not pins_pass(_build(tmp_path, name, MUTANTS[name])), f"mutant {name} passed every pin"
