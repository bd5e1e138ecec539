"""The algorithmic work that bench.py divides by kernel time, recomputed here
from its definition by counting, with no GPU.

Attention (one partial-attention launch, all rows): every attended token
costs its key and value (2 D elements) and one float32 eviction score; the
selected blocks are attended whole, the newest block up to the newest token;
the queries are read once. Prefill: every (query head, query token, attended
token) triple costs 4 D flops (q.k and p.v), the attended tokens being the
query block's selected blocks and, causally, its own block up to the query.
"""
import numpy as np

import bench
import synth


def test_attention_bytes_by_counting():
    w = synth.WORKLOADS["bf16_1layer_32k"]
    for n_tokens in (w.context + 1, w.context + 6, w.context + 64, w.context + 65):
        newest = n_tokens - 64 * ((n_tokens - 1) // 64)   # tokens of the newest block
        attended = 64 * 64 + newest                       # k = 64 whole blocks + the newest
        per_row = 0
        for _ in range(attended):
            per_row += 2 * w.head_dim * 2 + 4             # bf16 key + value, float32 bias
        q_bytes = w.batch * w.n_q_heads * w.head_dim * 2
        expect = w.rows * per_row + q_bytes
        assert bench.attn_bytes(w, "decode", n_tokens, 64) == expect
    # the query-set launch of a split step covers no newest block
    assert bench.attn_bytes(w, "decode_q", w.context + 6, 16) == \
        w.rows * 16 * 64 * (2 * w.head_dim * 2 + 4) + q_bytes
    # 32k workload, 6 tokens in the newest block: 135,529,984 bytes
    assert bench.attn_bytes(w, "decode", w.context + 6, 64) == 135_529_984


def test_prefill_flops_by_counting_pairs():
    w = synth.WORKLOADS["small_bf16"]
    n_tokens = 64 * 3 + 5                                  # a ragged last query block
    nqb = 4
    rng = np.random.default_rng(1)
    n_sel = rng.integers(0, 3, size=(nqb, w.rows))         # blocks selected per (block, row)
    n_sel[0] = 0                                           # block 0 has no candidates
    pairs = 0
    for i in range(nqb):
        for r in range(w.rows):
            for t in range(64 * i, min(64 * i + 64, n_tokens)):
                pairs += int(n_sel[i, r]) * 64             # whole selected blocks
                pairs += t - 64 * i + 1                    # own block up to itself
    expect = pairs * w.group * 4 * w.head_dim
    assert bench.prefill_flops(w, n_tokens, n_sel) == expect


def test_gamma_stats_by_counting():
    """gamma(t) = |Gamma(t) & Gamma(t-1)| / k per row for t >= 1 (Methodology,
    Locality Guarantee), recomputed with Python sets; the bound is checked on
    the steps that complete no block only."""
    import random
    rng = random.Random(3)
    k, k_e, R, T = 6, 4, 5, 9
    n_cand = [20, 20, 21, 21, 21, 22, 22, 22, 22]
    hist = []
    for t in range(T):
        rows = []
        for r in range(R):
            sel = sorted(rng.sample(range(n_cand[t]), rng.randint(k - 2, k)))
            rows.append(sel + [-1] * (k - len(sel)))
        hist.append(rows)
    want, want_nn = [], []
    for t in range(1, T):
        for r in range(R):
            a = {b for b in hist[t][r] if b >= 0}
            p = {b for b in hist[t - 1][r] if b >= 0}
            g = len(a & p) / k
            want.append(g)
            if n_cand[t] == n_cand[t - 1]:
                want_nn.append(g)
    got = bench.gamma_stats(np.array(hist, np.int32), n_cand, k, k_e)
    assert got["steps"] == T - 1 and got["rows"] == R
    assert abs(got["mean"] - sum(want) / len(want)) < 1e-12
    assert got["min"] == min(want)
    assert got["min_no_new_block"] == min(want_nn)
    assert got["bound_holds"] == (min(want_nn) >= k_e / k)


def test_more_than_one_gpu_is_refused():
    """bench.py measures one GPU's share: --gpus N > 1 exits with status 2 and
    says so, before touching a GPU."""
    import os
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stdout + r.stderr
