"""The checks catch the mistakes they are there for.

Two kinds of planted mistakes, both on the CPU:
  * traces with a planted breach of an invariant the pages state (a block
    readmitted to Gamma_e after its eviction; a step that completes no block
    but keeps fewer than k_e of the previous step's blocks): the trace
    checker must report exactly that breach;
  * copies of the oracle's source, each with one planted mistake, built on
    their own: the named pin must fail against each of them (in a process of
    its own, pointed at the copy through NOSA_ORACLE_LIB), while it passes
    against the oracle itself (the plain pin run).

Pages: NOSA technical summary, Methodology, "1. Algorithm: NOSA" (bullets
Dual-Selection Mechanism, Locality Guarantee, ED-DMA, Block-Wise
Implementation).
"""
import copy
import os
import subprocess
import sys

import pytest

import oracle
import synth
from harness import oracle_trace, trace_violations

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def trace():
    w = synth.WORKLOADS["small_f32"]
    return w, oracle_trace(w, margins=True, swaps=True)


def _mutable(tr):
    tr2 = copy.copy(tr)
    tr2.step = dict(tr.step)
    tr2.swap = dict(tr.swap)
    return tr2


def _replace(res, **kw):
    r2 = copy.copy(res)
    for k, v in kw.items():
        setattr(r2, k, v)
    return r2


def test_checker_is_quiet_on_the_oracle_trace(trace):
    w, tr = trace
    assert trace_violations(w, tr) == []


def test_checker_flags_a_readmitted_block(trace):
    """Strict eviction: put a block evicted at an earlier step back into
    Gamma_e (in place of one member, so the budget still holds)."""
    w, tr = trace
    r = tr.rows[0]
    evicted_at = {}
    for t in tr.steps:
        res = tr.step[(t, r)]
        for j in set(range(res.n_cand)) - set(res.gamma_e):
            evicted_at.setdefault(j, t)
    # a later step and a block evicted before it that is not selected there
    t = tr.steps[-1]
    res = tr.step[(t, r)]
    j = next(b for b, te in sorted(evicted_at.items())
             if te < t and b not in res.gamma_e and b not in res.gamma_q)
    ge = sorted(res.gamma_e[1:] + [j])
    tr2 = _mutable(tr)
    tr2.step[(t, r)] = _replace(res, gamma_e=ge)
    bad = trace_violations(w, tr2)
    assert ("readmitted", t, r) in bad
    assert all(x[1] == t and x[2] == r for x in bad), bad


def test_checker_flags_a_locality_breach(trace):
    """Locality Guarantee: on a step that completes no block, replace the
    selection by blocks the previous step did not select, so that
    gamma(t) < k_e / k."""
    w, tr = trace
    r = tr.rows[-1]
    t = next(t for t in tr.steps[1:]
             if w.n_cand(t) == w.n_cand(t - 1) and w.n_cand(t) >= w.k + w.k_e)
    prev = set(tr.step[(t - 1, r)].selected)
    res = tr.step[(t, r)]
    fresh = [j for j in range(res.n_cand) if j not in prev]
    ge, gq = sorted(fresh[:w.k_e]), sorted(fresh[w.k_e:w.k])
    assert len(set(ge + gq) & prev) / w.k < w.k_e / w.k
    tr2 = _mutable(tr)
    tr2.step[(t, r)] = _replace(res, gamma_e=ge, gamma_q=gq)
    kinds = {x[0] for x in trace_violations(w, tr2) if x[1:] == (t, r)}
    assert "locality" in kinds
    # and with the gamma of the unmutated step the bound holds there
    assert ("locality", t, r) not in trace_violations(w, tr)


# (name, text in nosa_oracle.c, replacement, pin that must fail)
MUTANTS = [
    ("bias_sign",
     "z[i] = scale * dot + (e ? (double)e[tok[i]] : 0.0);",
     "z[i] = scale * dot - (e ? (double)e[tok[i]] : 0.0);",
     "test_eviction_bias_is_a_log_multiplicity"),
    ("evict_min_pooling",
     "        if (mean > best)\n",
     "        if (mean < best || best == -INFINITY)\n",
     "test_pool_eviction_hand_case"),
    ("newest_token_dropped",
     "for (int u = c * block; u < n_tokens; ++u)",
     "for (int u = c * block; u < n_tokens - 1; ++u)",
     "test_sparse_equals_dense_when_budget_covers_all"),
    ("gamma_q_ignores_gamma_e",
     "    for (int i = 0; i < *n_ge; ++i)\n        rest[ge[i]] = 0;\n",
     "",
     "test_trace_invariants"),
    ("ties_to_higher_index",
     "(x[a] == x[b] && a < b)",
     "(x[a] == x[b] && a > b)",
     "test_topk_tie_rule_lower_index_wins"),
    ("sub_block_mean_over_block",
     "            double mean = s / (double)sub;\n            kbar[i * D + d]",
     "            double mean = s / (double)block;\n            kbar[i * D + d]",
     "test_pool_score_hand_case"),
    ("score_scale_dropped",
     "double a = scale * dot;",
     "double a = dot;",
     "test_pool_score_hand_case"),
]


@pytest.mark.parametrize("name,old,new,pin", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistake_fails_its_pin(tmp_path, name, old, new, pin):
    src = open(os.path.join(ROOT, "oracle", "nosa_oracle.c")).read()
    assert src.count(old) == 1, f"{name}: the text to mutate is not unique"
    mutated = tmp_path / f"oracle_{name}.c"
    mutated.write_text(src.replace(old, new))
    lib = oracle.compile_source(str(mutated), str(tmp_path / f"liboracle_{name}.so"))
    env = dict(os.environ, NOSA_ORACLE_LIB=lib)
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        f"tests/test_oracle_pins.py::{pin}" if "[" in pin else
                        "tests/test_oracle_pins.py", "-k", pin],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    # exit status 1: tests ran and at least one failed (not a crash or a
    # collection error, which would be 2, 3 or 4)
    assert r.returncode == 1, f"{name}: pin {pin} did not fail\n{r.stdout[-2000:]}{r.stderr[-2000:]}"
    assert "failed" in r.stdout
