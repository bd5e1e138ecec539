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
