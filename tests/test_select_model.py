"""Host model of the select kernel's top-k scheme, checked against sorting.

The select kernel (csrc/kernels_select.hip) finds the k best of up to 4096
candidates with 512 threads: candidate j sits in thread j % 512, wave
(j % 512) // 64; each wave finds the smallest key of its own top k by a
most-significant-bit-first search over 64-bit keys (two bits per step when a
lane holds one or two keys, one bit otherwise), keeps its keys at or above it
as survivors, and a survivor is selected when fewer than k survivors exceed
it. This file restates that scheme with Python integers and checks it, with
no GPU, against a plain sort on the same keys: random scores, heavy ties,
waves that hold fewer than k keys, and budgets at the edges. It pins the
scheme, not the kernel's code; the GPU parity tests compare the kernel with
the oracle.

Keys: (orderable(score) << 32) | (2^32 - 1 - j), so a larger key ranks first
and equal scores rank the lower index first (the order of Methodology, "Dual-
Selection Mechanism" with the lower-id tie rule).
"""
import numpy as np
import pytest

THREADS, WAVE = 512, 64


def orderable(f32: np.float32) -> int:
    u = int(np.array(f32, np.float32).view(np.uint32))
    if u == 0x80000000:  # -0 is the same score as +0
        u = 0
    return (~u & 0xFFFFFFFF) if u & 0x80000000 else (u | 0x80000000)


def rank_key(score, j: int) -> int:
    return (orderable(score) << 32) | (0xFFFFFFFF - j)


def wave_kth_key(keys: list, k: int, per_lane: int) -> int:
    """Smallest key of the wave's top k (the wave's keys; 0 = no key)."""
    present = [x for x in keys if x]
    if len(present) <= k:
        return min(present) if present else (1 << 64) - 1
    t = 0
    if per_lane > 2:
        for b in range(63, -1, -1):
            cand = t | (1 << b)
            c = sum(x >= cand for x in present)
            if c >= k:
                t = cand
                if c == k:
                    break
        return t
    for b in range(62, -1, -2):
        c3, c2, c1 = t | (3 << b), t | (2 << b), t | (1 << b)
        n3 = sum(x >= c3 for x in present)
        n2 = sum(x >= c2 for x in present)
        n1 = sum(x >= c1 for x in present)
        if n3 >= k:
            t, c = c3, n3
        elif n2 >= k:
            t, c = c2, n2
        elif n1 >= k:
            t, c = c1, n1
        else:
            c = -1
        if c == k:
            break
    return t


def model_topk(keys: list, k: int) -> set:
    """The kernel's scheme over keys[j] (0 = not a candidate): selected indices."""
    n = len(keys)
    per_lane = 1 if n <= THREADS else 2 if n <= 2 * THREADS else 4 if n <= 4 * THREADS else 8
    waves = [[] for _ in range(THREADS // WAVE)]
    for j, x in enumerate(keys):
        waves[(j % THREADS) // WAVE].append(x)
    surv = []
    for wk in waves:
        t = wave_kth_key(wk, k, per_lane)
        surv += [x for x in wk if x and x >= t]
    assert len(surv) <= (THREADS // WAVE) * k or len(surv) <= THREADS
    sel = {0xFFFFFFFF - (x & 0xFFFFFFFF) for x in surv if sum(y > x for y in surv) < k}
    return sel


def sorted_topk(scores, k: int, eligible=None) -> set:
    idx = [j for j in range(len(scores)) if eligible is None or eligible[j]]
    idx.sort(key=lambda j: (-float(scores[j]), j))
    return set(idx[:k])


def run_case(scores, k, eligible=None):
    keys = [rank_key(s, j) if (eligible is None or eligible[j]) else 0
            for j, s in enumerate(scores)]
    n_elig = len(scores) if eligible is None else int(np.sum(eligible))
    kk = min(k, n_elig)
    got = model_topk(keys, kk) if kk > 0 else set()
    assert got == sorted_topk(scores, kk, eligible)
    assert len(got) == kk


@pytest.mark.parametrize("n,k", [(1, 1), (7, 3), (64, 16), (65, 48), (66, 48), (67, 48),
                                 (512, 16), (513, 48), (1024, 32), (1027, 96 - 64),
                                 (2048, 16), (2051, 48), (4096, 64), (300, 64)])
def test_scheme_matches_sort_random(n, k):
    rng = np.random.default_rng(n * 131 + k)
    for _ in range(3):
        run_case(rng.standard_normal(n).astype(np.float32), k)


@pytest.mark.parametrize("n,k", [(64, 16), (512, 16), (1024, 32), (2048, 48)])
def test_scheme_matches_sort_with_ties(n, k):
    """Scores from a handful of values: the index decides most of the order."""
    rng = np.random.default_rng(7 + n + k)
    for levels in (1, 2, 5):
        scores = rng.integers(0, levels, n).astype(np.float32) - 1.5
        run_case(scores, k)


def test_scheme_with_excluded_candidates():
    """Gamma_q's keys: the members of Gamma_e are not candidates (key 0)."""
    rng = np.random.default_rng(11)
    for n, k, n_ex in ((512, 16, 48), (1024, 32, 96), (2051, 16, 48), (70, 16, 48)):
        scores = rng.standard_normal(n).astype(np.float32)
        elig = np.ones(n, bool)
        elig[rng.choice(n, n_ex, replace=False)] = False
        run_case(scores, k, elig)


def test_scheme_when_one_wave_holds_few_keys():
    """65-67 candidates: wave 1 holds 1-3 keys, fewer than the budget; keys
    that wave 0 leaves out must not be taken (the case that once selected 52
    blocks for a budget of 48)."""
    rng = np.random.default_rng(5)
    for n in (65, 66, 67):
        for k in (16, 48, 64):
            for _ in range(5):
                run_case(rng.standard_normal(n).astype(np.float32), k)


def test_negative_and_signed_zero_scores_order():
    """Keys sort negative scores below positive ones, and treat -0 and +0 as
    one score, so the lower index of the two ranks first, as a float sort."""
    scores = np.array([-1.0, -0.0, 0.0, 2.0, -3.5, 1e-30, -1e-30, -0.0], np.float32)
    ks = [rank_key(s, j) for j, s in enumerate(scores)]
    by_key = sorted(range(len(scores)), key=lambda j: -ks[j])
    assert by_key == [3, 5, 1, 2, 7, 6, 0, 4]
    assert by_key == sorted(range(len(scores)), key=lambda j: (-float(scores[j]), j))
    run_case(scores, 3)
