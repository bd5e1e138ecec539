"""Test-side helpers: seeded inputs per row, selection margins, oracle traces.

Inputs come from ``synth`` (keyed Philox streams). Selection margins are
enforced here, with the oracle's pooled scores: at every selection boundary
the k-th and (k+1)-th ranked scores must differ by at least 1e-4 relative
(relative to the larger magnitude, floored by the rms of the ranked set). A
row that fails is redrawn: the 64 eviction logits of the lower-ranked block
for a Gamma_e boundary, the group's query vectors for a Gamma_q boundary.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

import oracle
import synth
from synth import Overrides, Workload

MARGIN_REL = 1e-4


def workload(name: str) -> Workload:
    """A named workload; the suffix ":pbf16" selects its variant with pooled
    keys (and pooled queries) kept in bfloat16."""
    base, _, variant = name.partition(":")
    w = synth.WORKLOADS[base]
    if variant == "pbf16":
        return w.scaled(name=base + "_pbf16", pooled="bf16")
    if variant:
        raise ValueError(name)
    return w


def scale_of(w: Workload) -> float:
    return 1.0 / math.sqrt(w.head_dim)


def row_kv(w: Workload, layer: int, b: int, g: int):
    slab = layer % w.kv_slabs
    return synth.keys_row(w, slab, b, g), synth.values_row(w, slab, b, g)


def group_q(w: Workload, layer: int, t: int, b: int, g: int, ov: Overrides | None) -> np.ndarray:
    G = w.group
    return synth.queries_step(w, layer, t, ov)[b, g * G:(g + 1) * G]


def boundary_ok(x: np.ndarray, k: int, rel: float = MARGIN_REL) -> tuple[bool, int]:
    """Margin test between ranks k and k+1 of x (descending, ties by index).

    Returns (ok, index of the (k+1)-th ranked entry). Sets of at most k entries,
    and k = 0, have no boundary.
    """
    n = x.shape[0]
    if k == 0 or n <= k:
        return True, -1
    order = sorted(range(n), key=lambda j: (-x[j], j))
    a, b = x[order[k - 1]], x[order[k]]
    rms = math.sqrt(float(np.mean(np.square(x))))
    ok = abs(a - b) >= rel * max(abs(a), abs(b), rms)
    return ok, order[k]


def enforce_evict_margins(w: Workload, layer: int, b: int, g: int, steps, ov: Overrides,
                          max_attempts: int = 64, evict_tail=None):
    """Redraw eviction-logit blocks until every Gamma_e boundary has its margin.
    evict_tail(b, g, e) may replace the logits of the decoded tokens."""
    counts = sorted({w.n_cand(t) for t in range(max(steps) + 1)})
    for _ in range(max_attempts * max(1, len(counts))):
        e = synth.evict_row(w, layer, b, g, ov)
        if evict_tail is not None:
            e = evict_tail(b, g, e)
        cmax = counts[-1]
        E = np.array([oracle.block_evict(e, w.block, w.sub_block, j) for j in range(cmax)])
        bad = None
        for c in counts:
            ok, lower = boundary_ok(E[:c], w.k_e)
            if not ok:
                bad = lower
                break
        if bad is None:
            return e
        key = (layer, b, g, bad)
        ov.evict[key] = ov.evict.get(key, 0) + 1
    raise RuntimeError("could not enforce eviction margins")


@dataclass
class OracleTrace:
    """Oracle results for some rows of one layer over some steps."""
    w: Workload
    layer: int
    steps: list
    rows: list
    ov: Overrides
    step: dict = field(default_factory=dict)     # (t, row) -> oracle.RowStep
    swap: dict = field(default_factory=dict)     # (t, row) -> oracle.SwapResult
    # magnitude of the terms a pooled score sums: scale * sum_h |q_h| * max_token |k|
    term_scale: dict = field(default_factory=dict)  # (t, row) -> float


def oracle_trace(w: Workload, layer: int = 0, rows=None, steps=None, ov: Overrides | None = None,
                 margins: bool = True, swaps: bool = True, workers: int = 8,
                 evict_tail=None) -> OracleTrace:
    """Run the oracle on the given rows and steps, enforcing margins first.

    With ``swaps`` the steps must be 0..T-1 in order so the slot cache can be
    replayed from its empty start.
    """
    ov = ov if ov is not None else Overrides()
    rows = list(range(w.rows)) if rows is None else list(rows)
    steps = list(range(w.steps)) if steps is None else list(steps)
    if swaps:
        assert steps == list(range(len(steps))), "swap replay needs steps 0..T-1"
    tr = OracleTrace(w, layer, steps, rows, ov)
    sc = scale_of(w)

    def one_row(r):
        b, g = divmod(r, w.n_kv_heads)
        K, V = row_kv(w, layer, b, g)
        if margins:
            e = enforce_evict_margins(w, layer, b, g, steps, ov, evict_tail=evict_tail)
        else:
            e = synth.evict_row(w, layer, b, g, ov)
            if evict_tail is not None:
                e = evict_tail(b, g, e)
        cache = oracle.SlotCache(w.k)
        kmax = float(np.sqrt(np.max(np.sum(K.astype(np.float64) ** 2, axis=1))))
        out_step, out_swap, out_scale = {}, {}, {}
        for t in steps:
            for _ in range(64):
                q = group_q(w, layer, t, b, g, ov)
                res = oracle.step_row(w.n_tokens(t), q, K, V, e, w.block, w.sub_block,
                                      w.k_e, w.k_q, sc, pooled_bf16=w.pooled == "bf16")
                if not margins:
                    break
                rest = np.array([j not in set(res.gamma_e) for j in range(res.n_cand)], bool)
                ok, _ = boundary_ok(res.S[rest], w.k_q)
                if ok:
                    break
                key = (layer, t, b, g)
                ov.query[key] = ov.query.get(key, 0) + 1
            else:
                raise RuntimeError("could not enforce query margins")
            out_step[(t, r)] = res
            qn = float(np.sum(np.sqrt(np.sum(q.astype(np.float64) ** 2, axis=1))))
            out_scale[(t, r)] = sc * qn * kmax
            if swaps:
                out_swap[(t, r)] = cache.step(res.selected)
        return out_step, out_swap, out_scale

    # rows are independent; the oracle's C calls release the GIL
    for st, sw, ts in synth.parallel_map(one_row, rows, min(workers, max(1, len(rows)))):
        tr.step.update(st)
        tr.swap.update(sw)
        tr.term_scale.update(ts)
    return tr


def trace_violations(w: Workload, tr: OracleTrace) -> list:
    """Invariants the pages state, checked over the steps of a trace (an
    oracle trace, or a copy with a planted mistake). Returns (kind, t, row)
    for every breach:

    readmitted  a block that left Gamma_e is back in it (strict eviction:
                Methodology, Dual-Selection Mechanism)
    locality    gamma(t) = |Gamma(t) & Gamma(t-1)| / k below k_e / k on a step
                that completes no new block (Locality Guarantee)
    overlap     Gamma_q shares a block with Gamma_e (it ranks the rest)
    size        |Gamma_e| != min(k_e, c) or |Gamma| != min(k, c)
    cache       after the swap the cache does not hold exactly Gamma(t)
    fetch       the fetch list is not Gamma(t) minus the blocks cached before
    """
    out = []
    for r in tr.rows:
        evicted, prev = set(), None
        for t in tr.steps:
            res = tr.step[(t, r)]
            ge, gq = set(res.gamma_e), set(res.gamma_q)
            sel = sorted(ge | gq)
            if ge & evicted:
                out.append(("readmitted", t, r))
            evicted |= set(range(res.n_cand)) - ge
            if ge & gq:
                out.append(("overlap", t, r))
            if len(ge) != min(w.k_e, res.n_cand) or len(sel) != min(w.k, res.n_cand):
                out.append(("size", t, r))
            if prev is not None and w.n_cand(t) == w.n_cand(t - 1) and res.n_cand >= w.k:
                if len(set(sel) & set(prev)) / w.k < w.k_e / w.k:
                    out.append(("locality", t, r))
            sw = tr.swap.get((t, r))
            if sw is not None:
                if sorted(b for b in sw.slot_block if b >= 0) != sel:
                    out.append(("cache", t, r))
                if sw.fetch_block != sorted(set(sel) - set(prev or [])):
                    out.append(("fetch", t, r))
            prev = sel
    return out
