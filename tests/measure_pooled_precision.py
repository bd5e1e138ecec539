"""How often the query-aware selection depends on the precision of the
pooled keys: exact sub-block means (the oracle's default) against the same
means rounded to the nearest bfloat16 (the model-dtype reading).

Oracle only: both selections come from ``oracle.step_row`` on the same seeded
inputs, drawn WITHOUT the selection-margin filter (a margin filter would hide
exactly the near-ties that rounding can flip). The eviction selection does
not read the pooled keys, so only Gamma_q can differ.

    python tests/measure_pooled_precision.py [--rows N] [--steps T] [--json PATH]

Pages: NOSA technical summary, Methodology, "1. Algorithm: NOSA", bullet
"Block-Wise Implementation" (mean pooling inside sub-blocks, then max pooling
over the block); the pages fix the order of the pooling, not its precision.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import oracle  # noqa: E402
import synth  # noqa: E402


def measure(name: str, rows, steps, workers: int = 8) -> dict:
    w = synth.WORKLOADS[name]
    sc = 1.0 / math.sqrt(w.head_dim)
    G = w.group

    def one_row(r):
        b, g = divmod(r, w.n_kv_heads)
        K = synth.keys_row(w, 0, b, g)
        V = synth.values_row(w, 0, b, g)
        e = synth.evict_row(w, 0, b, g)
        diff_steps, diff_blocks, rel_gap = 0, 0, []
        for t in steps:
            q = synth.queries_step(w, 0, t)[b, g * G:(g + 1) * G]
            n = w.n_tokens(t)
            ex = oracle.step_row(n, q, K, V, e, w.block, w.sub_block, w.k_e, w.k_q, sc,
                                 pooled_bf16=False)
            rb = oracle.step_row(n, q, K, V, e, w.block, w.sub_block, w.k_e, w.k_q, sc,
                                 pooled_bf16=True)
            assert ex.gamma_e == rb.gamma_e
            a, c = set(ex.gamma_q), set(rb.gamma_q)
            if a != c:
                diff_steps += 1
                diff_blocks += len(a - c)
            # score error of the rounded means, relative to the exact score spread
            rest = np.array([j not in set(ex.gamma_e) for j in range(ex.n_cand)], bool)
            s = ex.S[rest]
            if s.size:
                rel_gap.append(float(np.max(np.abs(rb.S[rest] - s)) / (np.std(s) + 1e-300)))
        return diff_steps, diff_blocks, rel_gap

    res = synth.parallel_map(one_row, list(rows), workers)
    n_pairs = len(rows) * len(steps)
    ds = sum(x[0] for x in res)
    db = sum(x[1] for x in res)
    gaps = [g for x in res for g in x[2]]
    return {
        "workload": name, "rows": list(rows), "steps": [min(steps), max(steps)],
        "row_steps": n_pairs, "gamma_q_differs": ds, "rate": ds / n_pairs,
        "blocks_swapped_per_differing_row_step": (db / ds) if ds else 0.0,
        "max_score_error_over_score_std": max(gaps) if gaps else 0.0,
        "median_score_error_over_score_std": float(np.median(gaps)) if gaps else 0.0,
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--rows", type=int, default=16)
    ap.add_argument("--steps", type=int, default=64)
    ap.add_argument("--workers", type=int, default=8)
    ap.add_argument("--json", default=None)
    a = ap.parse_args()
    out = []
    for name in ("bf16_1layer_32k", "bf16_3b_64k"):
        w = synth.WORKLOADS[name]
        rows = np.linspace(0, w.rows - 1, a.rows).round().astype(int).tolist()
        steps = list(range(min(a.steps, w.steps)))
        out.append(measure(name, rows, steps, a.workers))
        print(json.dumps(out[-1]), flush=True)
    if a.json:
        with open(a.json, "w") as f:
            json.dump(out, f, indent=1)


if __name__ == "__main__":
    main()
