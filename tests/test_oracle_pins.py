"""Pins of the fp64 oracle against facts that do not come from the oracle itself.

Each test names what fixes the expected result: a hand-worked case, a textbook
routine, brute force, a closed form, or an invariant the NOSA pages state
(technical summary, Methodology, "1. Algorithm: NOSA").
"""
import itertools
import json
import os

import numpy as np
import pytest
import torch

import oracle
import synth
from harness import oracle_trace, boundary_ok, trace_violations

GOLD = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------------------
# top-k: brute force over tiny inputs, with forced ties
# ---------------------------------------------------------------------------

def test_topk_matches_bruteforce_sort_with_ties():
    rng = np.random.default_rng(7)
    for n in range(0, 11):
        for trial in range(6):
            # few distinct values -> many ties; equal scores must rank the lower index first
            x = rng.integers(-2, 3, size=n).astype(np.float64)
            allowed = rng.integers(0, 2, size=n).astype(bool) if trial % 2 else np.ones(n, bool)
            for k in range(0, n + 2):
                want = sorted(sorted((j for j in range(n) if allowed[j]),
                                     key=lambda j: (-x[j], j))[:k])
                got = oracle.topk(x, k, allowed if trial % 2 else None)
                assert got == want, (n, k, x, allowed)


def test_topk_tie_rule_lower_index_wins():
    assert oracle.topk([5.0, 5.0, 5.0, 1.0], 2) == [0, 1]
    assert oracle.topk([1.0, 5.0, 5.0, 5.0], 1) == [1]
    assert oracle.topk([0.0] * 6, 3, [0, 1, 0, 1, 1, 1]) == [1, 3, 4]


def test_topk_every_subset_small():
    # every subset of n <= 6 candidates, every k: the chosen set is the k best
    x = np.array([0.3, -1.0, 0.3, 2.0, 0.0, 2.0])
    for n in range(1, 7):
        for mask in itertools.product([0, 1], repeat=n):
            for k in range(n + 1):
                got = oracle.topk(x[:n], k, list(mask))
                cand = [j for j in range(n) if mask[j]]
                want = sorted(sorted(cand, key=lambda j: (-x[j], j))[:k])
                assert got == want


def test_select_by_pre_exp_equals_select_by_exp():
    # ED-DMA selects on pre-exponential scores; exp is monotone, so the
    # selected set equals selection on exponentiated scores when both are finite.
    rng = np.random.default_rng(3)
    for _ in range(50):
        x = rng.normal(0, 3, size=40)
        for k in (1, 5, 17, 39):
            assert oracle.topk(x, k) == oracle.topk(np.exp(x), k)


# ---------------------------------------------------------------------------
# two-stage pooling: hand case and reductions to plain routines
# ---------------------------------------------------------------------------

def _hand():
    with open(os.path.join(GOLD, "pool_hand.json")) as f:
        return json.load(f)


def test_pool_eviction_hand_case():
    h = _hand()
    e = np.zeros(64, np.float32)
    e[0] = 16.0
    e[16:32] = 2.0
    e[32:48] = -1.0
    e[48:64:2], e[49:64:2] = 3.0, -3.0
    E = oracle.block_evict(e, h["block"], h["sub_block"], 0)
    assert E == h["expected_E"]
    assert E not in (h["wrong_max_then_mean"], h["wrong_block_mean"], h["wrong_token_max"])


def test_pool_score_hand_case():
    h = _hand()
    a0, a1 = h["keys"]["a0"], h["keys"]["a1"]
    K = np.zeros((64, 2), np.float32)
    for i in range(4):
        K[16 * i:16 * i + 16, 0] = a0[i]
        K[16 * i:16 * i + 16, 1] = a1[i]
    # make sub-block 0 non-constant with the same mean (mean pooling, not max)
    K[0:16:2, 0] += 2.0
    K[1:16:2, 0] -= 2.0
    q = np.array(h["queries"], np.float32)
    S = oracle.block_score(q, K, h["block"], h["sub_block"], 0, h["scale"])
    assert S == h["expected_S"]
    assert S != h["wrong_max_of_sum"]
    kbar = oracle.pool_keys(K, 64, 16, 0)
    np.testing.assert_array_equal(kbar[:, 0], a0)
    np.testing.assert_array_equal(kbar[:, 1], a1)


def test_round_bf16_matches_bit_rounding_of_float32():
    """The oracle's bfloat16 rounding (nearest multiple of the bfloat16
    spacing) against the bit-level round-half-to-even of float32 values."""
    rng = np.random.default_rng(21)
    x = (rng.normal(size=4000) * np.exp2(rng.integers(-140, 60, size=4000))).astype(np.float32)
    # exact ties: float32 values whose dropped half-word is 0x8000
    u = rng.integers(0, 2 ** 31, size=500, dtype=np.uint64).astype(np.uint32)
    u = (u & np.uint32(0xFFFF0000)) | np.uint32(0x8000)
    x = np.concatenate([x, u.view(np.float32), -u.view(np.float32)])
    x = x[np.isfinite(x)]
    want = synth.rne_bf16(x)
    got = np.array([oracle.round_bf16(float(v)) for v in x], dtype=np.float64)
    np.testing.assert_array_equal(got, want.astype(np.float64))


def test_round_bf16_of_doubles():
    """Values that float32 cannot hold: a first rounding to float32 would turn
    1 + 2^-8 + 2^-30 into the tie 1 + 2^-8 and round it down."""
    r = oracle.round_bf16
    assert r(1.0 + 2.0 ** -8 + 2.0 ** -30) == 1.0 + 2.0 ** -7
    assert r(-(1.0 + 2.0 ** -8 + 2.0 ** -30)) == -(1.0 + 2.0 ** -7)
    assert r(1.0 + 2.0 ** -8) == 1.0                      # tie, even mantissa below
    assert r(1.0 + 3 * 2.0 ** -8) == 1.0 + 2.0 ** -6      # tie, even mantissa above
    assert r(1.0 + 2.0 ** -8 - 2.0 ** -40) == 1.0
    assert r(2.0 ** -134) == 0.0                          # half the smallest subnormal
    assert r(3 * 2.0 ** -134) == 2.0 ** -132              # tie between 1 and 2 spacings
    assert r(255.5) == 256.0 and r(254.5) == 254.0        # spacing 1 below 256, 2 above
    assert r(0.0) == 0.0


def test_pool_keys_bf16_rounding_hand_case():
    """Sub-block means of bfloat16 keys, kept in bfloat16: 1 and 1 + 2^-7 are
    neighbours, so a mean of 1 + 2^-9 rounds down, 1 + 2^-8 is a tie (down to
    the even 1) and 1 + 3 * 2^-9 rounds up."""
    hi = 1.0 + 2.0 ** -7
    K = np.ones((64, 1), np.float32)
    K[0:4, 0] = hi          # sub-block 0: mean 1 + 2^-9
    K[16:24, 0] = hi        # sub-block 1: mean 1 + 2^-8
    K[32:44, 0] = hi        # sub-block 2: mean 1 + 3 * 2^-9
    exact = oracle.pool_keys(K, 64, 16, 0)[:, 0]
    np.testing.assert_array_equal(exact, [1 + 2.0 ** -9, 1 + 2.0 ** -8, 1 + 3 * 2.0 ** -9, 1.0])
    kept = oracle.pool_keys(K, 64, 16, 0, pooled_bf16=True)[:, 0]
    np.testing.assert_array_equal(kept, [1.0, 1.0, hi, 1.0])
    q = np.ones((1, 1), np.float32)
    assert oracle.block_score(q, K, 64, 16, 0, 1.0) == 1 + 3 * 2.0 ** -9
    assert oracle.block_score(q, K, 64, 16, 0, 1.0, pooled_bf16=True) == hi
    assert oracle.block_score(-q, K, 64, 16, 0, 1.0, pooled_bf16=True) == -1.0


def test_evict_logit_closed_forms():
    """The eviction head is linear: one-hot inputs pick single weights, the
    bias adds, scaling the input scales the logit, and a hand-made case."""
    rng = np.random.default_rng(31)
    w = rng.normal(size=64).astype(np.float32)
    for i in (0, 17, 63):
        x = np.zeros(64, np.float32)
        x[i] = 1.0
        assert oracle.evict_logit(x, w) == float(w[i])
        assert oracle.evict_logit(x, w, -4.0) == float(w[i]) - 4.0
    x = rng.normal(size=64).astype(np.float32)
    assert oracle.evict_logit(2 * x, w) == 2 * oracle.evict_logit(x, w)
    assert oracle.evict_logit(np.array([1, 2, 3], np.float32),
                              np.array([0.5, -1, 0.25], np.float32), 1.0) == 0.25


def test_qkv_split_order():
    """Query heads, then key heads, then value heads, each head_dim wide."""
    Hq, Hkv, D = 4, 2, 3
    a = np.arange((Hq + 2 * Hkv) * D, dtype=np.float32)
    q, k, v = oracle.qkv_split(a, Hq, Hkv, D)
    assert q.shape == (4, 3) and k.shape == (2, 3) and v.shape == (2, 3)
    assert q[1, 2] == 5 and k[0, 0] == 12 and k[1, 2] == 17 and v[0, 0] == 18 and v[1, 2] == 23


def test_pool_reduces_to_mean_when_sub_block_is_block():
    rng = np.random.default_rng(11)
    K = rng.normal(size=(256, 16)).astype(np.float32)
    e = rng.normal(size=256).astype(np.float32)
    q = rng.normal(size=(1, 16)).astype(np.float32)
    for j in range(4):
        blk = K[64 * j:64 * j + 64].astype(np.float64)
        want = 0.3 * float(q[0].astype(np.float64) @ blk.mean(axis=0))
        assert oracle.block_score(q, K, 64, 64, j, 0.3) == pytest.approx(want, rel=1e-12, abs=1e-12)
        assert oracle.block_evict(e, 64, 64, j) == pytest.approx(
            float(e[64 * j:64 * j + 64].astype(np.float64).mean()), rel=1e-12, abs=1e-13)


def test_pool_reduces_to_token_max_when_sub_block_is_one():
    rng = np.random.default_rng(12)
    K = rng.normal(size=(128, 8)).astype(np.float32)
    e = rng.normal(size=128).astype(np.float32)
    q = rng.normal(size=(2, 8)).astype(np.float32)
    for j in range(2):
        blk = K[64 * j:64 * j + 64].astype(np.float64)
        want = sum(float(np.max(0.5 * (blk @ q[h].astype(np.float64)))) for h in range(2))
        assert oracle.block_score(q, K, 64, 1, j, 0.5) == pytest.approx(want, rel=1e-12)
        assert oracle.block_evict(e, 64, 1, j) == float(e[64 * j:64 * j + 64].max())


# ---------------------------------------------------------------------------
# attention: textbook reductions and closed forms
# ---------------------------------------------------------------------------

def _sdpa(q, K, V, e, n, scale):
    """torch's scaled_dot_product_attention on CPU in float64 with an additive mask."""
    qt = torch.from_numpy(q.astype(np.float64))[None, :, None, :]          # [1, G, 1, D]
    kt = torch.from_numpy(K[:n].astype(np.float64))[None, None].expand(1, q.shape[0], n, -1)
    vt = torch.from_numpy(V[:n].astype(np.float64))[None, None].expand(1, q.shape[0], n, -1)
    mask = torch.from_numpy(e[:n].astype(np.float64))[None, None, None, :]
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask, scale=scale)
    return o[0, :, 0, :].numpy()


@pytest.mark.parametrize("n_tokens", [1, 63, 64, 65, 640, 2000])
def test_sparse_equals_dense_when_budget_covers_all(n_tokens):
    rng = np.random.default_rng(n_tokens)
    D, G = 64, 4
    K = rng.normal(size=(n_tokens, D)).astype(np.float32)
    V = rng.normal(size=(n_tokens, D)).astype(np.float32)
    e = rng.normal(size=n_tokens).astype(np.float32)
    q = rng.normal(size=(G, D)).astype(np.float32)
    c = (n_tokens - 1) // 64
    res = oracle.step_row(n_tokens, q, K, V, e, 64, 16, 4, max(c, 1), 0.125)
    assert res.selected == list(range(c))
    np.testing.assert_allclose(res.out, _sdpa(q, K, V, e, n_tokens, 0.125), rtol=1e-12, atol=1e-13)


def test_constant_values_give_constant_output():
    rng = np.random.default_rng(5)
    n = 1000
    K = rng.normal(size=(n, 32)).astype(np.float32)
    V = np.tile(rng.normal(size=(1, 32)).astype(np.float32), (n, 1))
    e = rng.normal(size=n).astype(np.float32) * 5
    q = rng.normal(size=(3, 32)).astype(np.float32)
    res = oracle.step_row(n, q, K, V, e, 64, 16, 3, 2, 0.2)
    np.testing.assert_allclose(res.out, np.tile(V[:1].astype(np.float64), (3, 1)), rtol=1e-13)


def test_zero_keys_zero_bias_give_mean_of_attended_values():
    rng = np.random.default_rng(6)
    n = 777
    K = np.zeros((n, 16), np.float32)
    V = rng.normal(size=(n, 16)).astype(np.float32)
    e = np.zeros(n, np.float32)
    q = rng.normal(size=(2, 16)).astype(np.float32)
    res = oracle.step_row(n, q, K, V, e, 64, 16, 2, 3, 0.25)
    toks = [t for j in res.selected for t in range(64 * j, 64 * j + 64)] + \
        list(range(64 * res.n_cand, n))
    want = V[toks].astype(np.float64).mean(axis=0)
    np.testing.assert_allclose(res.out, np.tile(want, (2, 1)), rtol=1e-12, atol=1e-14)


def test_eviction_bias_is_a_log_multiplicity():
    # Adding ln(m) to a token's logit weighs it exactly like m copies of that
    # token with no bias: the bias enters inside the exponential (ED-DMA).
    rng = np.random.default_rng(9)
    n, D = 40, 8
    K = rng.normal(size=(n, D)).astype(np.float32)
    V = rng.normal(size=(n, D)).astype(np.float32)
    q = rng.normal(size=(2, D)).astype(np.float32)
    mult = rng.integers(1, 5, size=n)
    e = np.log(mult).astype(np.float32)
    # float32 rounding of ln(m) perturbs weights by < 1e-7 relative
    got = oracle.attend_tokens(q, K, V, e, np.arange(n), 0.3)
    rep = np.repeat(np.arange(n), mult)
    want = oracle.attend_tokens(q, K, V, None, rep, 0.3)
    np.testing.assert_allclose(got, want, rtol=2e-7, atol=2e-7)
    # and the sign matters: a negative bias of ln(m) is not the same
    bad = oracle.attend_tokens(q, K, V, -e, np.arange(n), 0.3)
    assert np.max(np.abs(bad - want)) > 1e-3


def test_large_biases_stay_finite_and_shift_invariant():
    rng = np.random.default_rng(10)
    n = 300
    K = rng.normal(size=(n, 16)).astype(np.float32)
    V = rng.normal(size=(n, 16)).astype(np.float32)
    q = rng.normal(size=(2, 16)).astype(np.float32)
    e = rng.uniform(-100, 100, size=n).astype(np.float32)
    a = oracle.attend_tokens(q, K, V, e, np.arange(n), 0.25)
    b = oracle.attend_tokens(q, K, V, (e - 50).astype(np.float32), np.arange(n), 0.25)
    assert np.all(np.isfinite(a))
    np.testing.assert_allclose(a, b, rtol=1e-9, atol=1e-9)
    # softmax concentrates on the largest logit when it dominates by > 40 nats
    i = int(np.argmax(e))
    z = 0.25 * (K.astype(np.float64) @ q.T.astype(np.float64)) + e[:, None]
    top2 = np.sort(z, axis=0)[-2:]
    for h in range(2):
        if top2[1, h] - top2[0, h] > 40 and int(np.argmax(z[:, h])) == i:
            np.testing.assert_allclose(a[h], V[i], rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------------------
# invariants over traces: strict eviction, locality bound, swap lists
# ---------------------------------------------------------------------------

def _incremental_gamma_e(E_of, counts, k_e):
    """The method's route to Gamma_e: keep k_e blocks; a new candidate replaces
    the lowest-ranked kept block if it ranks above it, else is evicted at once."""
    def above(a, b):
        return E_of[a] > E_of[b] or (E_of[a] == E_of[b] and a < b)
    kept, out, seen = [], [], 0
    for c in counts:
        for x in range(seen, c):
            if len(kept) < k_e:
                kept.append(x)
                continue
            if k_e == 0:
                continue
            low = kept[0]
            for y in kept[1:]:
                if above(low, y):
                    low = y
            if above(x, low):
                kept[kept.index(low)] = x
        seen = c
        out.append(sorted(kept))
    return out


_TRACES = {}


def _trace(name):
    if name not in _TRACES:
        w = synth.WORKLOADS[name]
        _TRACES[name] = (w, oracle_trace(w, steps=list(range(w.steps)), margins=True, swaps=True))
    return _TRACES[name]


@pytest.mark.parametrize("name", ["tiny_f32", "small_f32", "small_offload"])
def test_trace_invariants(name):
    """Strict eviction, the locality bound on steps that complete no block,
    Gamma_q outside Gamma_e, the budgets, and the swap lists (trace_violations)
    hold on every step and row; the stateless top-k_e equals the method's
    incremental eviction; the swap's own gamma agrees."""
    w, tr = _trace(name)
    assert trace_violations(w, tr) == []
    for r in tr.rows:
        counts = [w.n_cand(t) for t in tr.steps]
        E_all = tr.step[(tr.steps[-1], r)].E
        inc = _incremental_gamma_e(E_all, counts, w.k_e)
        prev_sel = None
        for i, t in enumerate(tr.steps):
            res = tr.step[(t, r)]
            # stateless definition == the method's incremental eviction
            assert res.gamma_e == inc[i]
            if prev_sel is not None:
                assert tr.swap[(t, r)].gamma == len(set(res.selected) & set(prev_sel)) / w.k
            prev_sel = res.selected
        # the margin recipe held at every boundary that was used
        for t in tr.steps:
            res = tr.step[(t, r)]
            assert boundary_ok(res.E, w.k_e)[0]
            rest = np.array([j not in set(res.gamma_e) for j in range(res.n_cand)], bool)
            assert boundary_ok(res.S[rest], w.k_q)[0]


def test_swap_cache_bruteforce():
    # random selections; check the slot rule against a direct set computation
    rng = np.random.default_rng(1)
    k = 6
    cache = oracle.SlotCache(k)
    prev = set()
    slots = [-1] * k
    for t in range(200):
        sel = sorted(rng.choice(20, size=rng.integers(0, k + 1), replace=False).tolist())
        res = cache.step(sel)
        fetch = sorted(set(sel) - {b for b in slots if b >= 0})
        free = [s for s in range(k) if slots[s] < 0 or slots[s] not in sel]
        assert res.fetch_block == fetch
        assert res.fetch_slot == free[:len(fetch)]
        for b, s in zip(fetch, free):
            slots[s] = b
        slots = [b if b in sel else -1 for b in slots]
        assert res.slot_block == slots
        assert res.gamma == len(set(sel) & prev) / k
        prev = set(sel)


# ---------------------------------------------------------------------------
# prefill with the selection per query block
# ---------------------------------------------------------------------------

def _np_causal(q, K, V, e, scale, allowed):
    """Textbook softmax attention of q [N, G, D]; allowed(p) -> key positions."""
    N, G, D = q.shape
    out = np.zeros((N, G, D))
    Kd, Vd, ed = K.astype(np.float64), V.astype(np.float64), e.astype(np.float64)
    for p in range(N):
        idx = np.array(sorted(allowed(p)))
        for h in range(G):
            z = scale * (Kd[idx] @ q[p, h].astype(np.float64)) + ed[idx]
            a = np.exp(z - z.max())
            out[p, h] = (a / a.sum()) @ Vd[idx]
    return out


def test_prefill_is_dense_causal_when_the_budget_covers_every_block():
    rng = np.random.default_rng(41)
    N, G, D = 200, 2, 8
    q = rng.normal(size=(N, G, D)).astype(np.float32)
    K = rng.normal(size=(N, D)).astype(np.float32)
    V = rng.normal(size=(N, D)).astype(np.float32)
    e = rng.normal(size=N).astype(np.float32)
    res = oracle.prefill_row(q, K, V, e, 64, 16, 2, 2, 0.35)
    want = _np_causal(q, K, V, e, 0.35, lambda p: range(p + 1))
    np.testing.assert_allclose(res.out, want, rtol=1e-12, atol=1e-12)
    assert res.sel.tolist() == [[-1] * 4, [0, -1, -1, -1], [0, 1, -1, -1], [0, 1, 2, -1]]


def test_prefill_eviction_selection_by_brute_force():
    """k_q = 0: query block i attends the k_e blocks before it with the
    largest max-of-sub-block-mean eviction score, plus its causal own block."""
    rng = np.random.default_rng(42)
    N, G, D, ke = 64 * 6 + 10, 1, 4, 2
    q = rng.normal(size=(N, G, D)).astype(np.float32)
    K = rng.normal(size=(N, D)).astype(np.float32)
    V = rng.normal(size=(N, D)).astype(np.float32)
    e = rng.normal(size=N).astype(np.float32)
    E = [max(float(np.mean(e[64 * j + 16 * i:64 * j + 16 * i + 16].astype(np.float64)))
             for i in range(4)) for j in range(N // 64)]
    res = oracle.prefill_row(q, K, V, e, 64, 16, ke, 0, 0.5)
    for i in range(N // 64 + 1):
        best = sorted(sorted(range(i), key=lambda j: (-E[j], j))[:ke])
        assert res.sel[i][:len(best)].tolist() == best
    sel_of = {i: [j for j in res.sel[i] if j >= 0] for i in range(res.sel.shape[0])}
    want = _np_causal(q, K, V, e, 0.5, lambda p: [64 * j + u for j in sel_of[p // 64]
                                                  for u in range(64)]
                      + list(range(64 * (p // 64), p + 1)))
    np.testing.assert_allclose(res.out, want, rtol=1e-12, atol=1e-12)


def test_prefill_query_selection_by_brute_force():
    """k_e = 0: the k_q blocks with the largest score of the block's pooled
    query (the exact mean of its queries) against the sub-block key means."""
    rng = np.random.default_rng(43)
    N, G, D, kq, sc = 64 * 5 + 30, 2, 4, 2, 0.4
    q = rng.normal(size=(N, G, D)).astype(np.float32)
    K = rng.normal(size=(N, D)).astype(np.float32)
    V = rng.normal(size=(N, D)).astype(np.float32)
    e = rng.normal(size=N).astype(np.float32)
    res = oracle.prefill_row(q, K, V, e, 64, 16, 0, kq, sc)
    Kd = K.astype(np.float64)
    for i in range(1, N // 64 + 1):
        # sums of at most 64 float32 draws are exact in double, so the mean is
        # the exact mean, whatever order numpy adds in
        qb = q[64 * i:64 * i + 64].astype(np.float64).mean(axis=0)
        np.testing.assert_array_equal(oracle.pool_queries(q[64 * i:64 * i + 64]), qb)
        S = []
        for j in range(i):
            kb = Kd[64 * j:64 * j + 64].reshape(4, 16, D).mean(axis=1)
            S.append(sum(max(sc * float(kb[s] @ qb[h]) for s in range(4))
                         for h in range(G)))
        best = sorted(sorted(range(i), key=lambda j: (-S[j], j))[:kq])
        assert res.sel[i][:len(best)].tolist() == best


def test_prefill_qblock_by_brute_force():
    """One query block alone, both parts of the budget: its selection is the
    k_e best eviction blocks plus the k_q best query-scored blocks of the
    rest; its tokens attend those blocks and their own block causally. The
    ragged last query block included."""
    rng = np.random.default_rng(44)
    N, G, D, ke, kq, sc = 64 * 7 + 20, 2, 8, 2, 2, 0.3
    q = rng.normal(size=(N, G, D)).astype(np.float32)
    K = rng.normal(size=(N, D)).astype(np.float32)
    V = rng.normal(size=(N, D)).astype(np.float32)
    e = rng.normal(size=N).astype(np.float32)
    Kd = K.astype(np.float64)
    E = [max(float(np.mean(e[64 * j + 16 * s:64 * j + 16 * s + 16].astype(np.float64)))
             for s in range(4)) for j in range(N // 64)]
    full = oracle.prefill_row(q, K, V, e, 64, 16, ke, kq, sc)
    for i in (0, 1, 4, 7):
        lo, hi = 64 * i, min(64 * i + 64, N)
        qb = q[lo:hi].astype(np.float64).mean(axis=0)
        S = [sum(max(sc * float(Kd[64 * j + 16 * s:64 * j + 16 * s + 16].mean(axis=0)
                                @ qb[h]) for s in range(4))
                 for h in range(G)) for j in range(i)]
        ge = sorted(range(i), key=lambda j: (-E[j], j))[:ke]
        gq = sorted((j for j in range(i) if j not in ge), key=lambda j: (-S[j], j))[:kq]
        want_sel = sorted(ge + gq)
        res = oracle.prefill_qblock(q, K, V, e, i, 64, 16, ke, kq, sc)
        assert res.sel[0][:len(want_sel)].tolist() == want_sel
        assert all(x == -1 for x in res.sel[0][len(want_sel):])
        want = _np_causal(q[lo:hi], K, V, e, sc,
                          lambda p: [64 * j + u for j in want_sel for u in range(64)]
                          + list(range(lo, lo + p + 1)))
        np.testing.assert_allclose(res.out, want, rtol=1e-12, atol=1e-12)
        # the same block of the whole-row call
        np.testing.assert_array_equal(res.out, full.out[lo:hi])
        assert res.sel[0].tolist() == full.sel[i].tolist()


def test_pool_queries_bf16():
    """Integer inputs: the exact means are floats, so rounding them to bf16 is
    the bit-level rounding of those floats."""
    rng = np.random.default_rng(44)
    q = rng.integers(-300, 300, size=(64, 2, 8)).astype(np.float32)
    mean = q.astype(np.float64).mean(axis=0).astype(np.float32)
    np.testing.assert_array_equal(oracle.pool_queries(q, pooled_bf16=True), synth.rne_bf16(mean))
