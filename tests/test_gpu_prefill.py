"""Prefill (training-time forward) with NOSA's selection per query block:
the HIP path (pooled queries, per-block selection, causal block-sparse MFMA
attention) against the fp64 oracle through the C ABI. Selections bit-exact,
outputs within the bf16 tolerance. Pooled keys and queries are float32 (the
exact means rounded once) unless a workload name carries ":pbf16", the
variant that keeps them in bfloat16."""
import math

import numpy as np
import pytest

import oracle
import synth
from harness import boundary_ok, row_kv
from synth import Overrides, Workload

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

TOL = dict(rtol=2e-2, atol=2e-3)

# sequence length = context; one extra token keeps n_max above it
PREFILL = {
    # 16 query blocks (the last one 40 tokens), GQA 4, D 128
    "prefill_bf16": Workload("prefill_bf16", 3001, 2, 8, 2, 128, 1000, 1, 3, 2, "bf16",
                             key_offset_std=0.5),
    # GQA 3, D 64, a k_q larger than k_e
    "prefill_g3_d64": Workload("prefill_g3_d64", 3002, 1, 6, 2, 64, 700, 1, 2, 3, "bf16",
                               key_offset_std=0.5),
    # the budget covers every earlier block: dense causal attention
    "prefill_dense": Workload("prefill_dense", 3003, 1, 4, 1, 128, 200, 1, 4, 4, "bf16"),
    # GQA 8: a query block's 512 query rows take two workgroups of the kernel
    "prefill_g8": Workload("prefill_g8", 3004, 1, 8, 1, 128, 600, 1, 2, 3, "bf16",
                           key_offset_std=0.5),
    # no grouping (G 1, D 64): one 16-column tile per wave, four waves
    "prefill_g1_d64": Workload("prefill_g1_d64", 3005, 2, 2, 2, 64, 450, 1, 3, 2, "bf16",
                               key_offset_std=0.5),
    # GQA 2: four waves of two tiles
    "prefill_g2": Workload("prefill_g2", 3006, 1, 4, 2, 128, 330, 1, 2, 2, "bf16",
                           key_offset_std=0.5),
}


def _w(name: str) -> Workload:
    base, _, variant = name.partition(":")
    w = PREFILL[base]
    return w.scaled(name=base + "_pbf16", pooled="bf16") if variant == "pbf16" else w


def _prefill_trace(w: Workload, e_scale: float = 1.0):
    """Oracle prefill of every row, with the 1e-4 margins enforced at every
    selection boundary (eviction blocks and query blocks redrawn as needed);
    the eviction logits are the seeded ones times e_scale."""
    N, D, G = w.context, w.head_dim, w.group
    nqb = -(-N // 64)
    sc = 1.0 / math.sqrt(D)
    pb = w.pooled == "bf16"
    ov = Overrides()
    out = {}
    for r in range(w.rows):
        b, g = divmod(r, w.n_kv_heads)
        K, V = row_kv(w, 0, b, g)
        K, V = K[:N], V[:N]
        for _ in range(256):
            e = (synth.evict_row(w, 0, b, g, ov) * np.float32(e_scale)).astype(np.float32)
            E = [oracle.block_evict(e, 64, 16, j) for j in range(max(nqb - 1, 0))]
            bad = None
            for c in range(1, nqb):
                ok, lower = boundary_ok(np.array(E[:c]), w.k_e)
                if not ok:
                    bad = lower
                    break
            if bad is None:
                break
            key = (0, b, g, bad)
            ov.evict[key] = ov.evict.get(key, 0) + 1
        else:
            raise RuntimeError("eviction margins")
        for i in range(1, nqb):
            ge = sorted(sorted(range(i), key=lambda j: (-E[j], j))[:w.k_e])
            for _ in range(64):
                q = synth.prefill_queries(w, 0, N, ov)[b, :, g * G:(g + 1) * G]
                qb = oracle.pool_queries(q[64 * i:64 * i + 64], pooled_bf16=pb)
                S = np.array([oracle.block_score(qb, K, 64, 16, j, sc, pooled_bf16=pb)
                              for j in range(i)])
                rest = np.array([j not in ge for j in range(i)], bool)
                ok, _ = boundary_ok(S[rest], w.k_q)
                if ok:
                    break
                key = ("prefill", 0, b, g, i)
                ov.query[key] = ov.query.get(key, 0) + 1
            else:
                raise RuntimeError("query margins")
        q = synth.prefill_queries(w, 0, N, ov)[b, :, g * G:(g + 1) * G]
        out[r] = oracle.prefill_row(q, K, V, e[:N], 64, 16, w.k_e, w.k_q, sc, pooled_bf16=pb)
    return ov, out


@pytest.mark.parametrize("name,e_scale", [(n, 1.0) for n in PREFILL] + [
    ("prefill_bf16", 40.0), ("prefill_g8", 40.0), ("prefill_bf16:pbf16", 1.0),
    ("prefill_g3_d64:pbf16", 1.0)])
def test_prefill_parity(name, e_scale):
    """e_scale 40: eviction logits up to ~150 in magnitude, past float32's exp
    range; the softmax's running base keeps every exponential bounded, and a
    few tokens dominate each softmax, so the probabilities' own rounding no
    longer averages out: the bf16 tolerance holds there too."""
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gpu_harness as gh
    w = _w(name)
    N, G = w.context, w.group
    ov, ref = _prefill_trace(w, e_scale)
    inp = gh.upload(w, ov=ov, steps=1)
    if e_scale != 1.0:
        e = inp.e_tok.cpu().numpy()
        for r in range(w.rows):
            b, g = divmod(r, w.n_kv_heads)
            e[r, :w.n_max] = synth.evict_row(w, 0, b, g, ov) * np.float32(e_scale)
        assert np.abs(e).max() > 100.0
        inp.e_tok.copy_(torch.from_numpy(e))
    q_all = gh.to_device(gh.storage(synth.prefill_queries(w, 0, N, ov), w), w)
    layer = gh.make_layer(w, inp)
    out, sel, n_sel = layer.prefill(q_all, N)
    torch.cuda.synchronize()
    out = out.float().cpu().numpy()
    sel, n_sel = sel.cpu().numpy(), n_sel.cpu().numpy()
    for r in range(w.rows):
        b, g = divmod(r, w.n_kv_heads)
        for i in range(ref[r].sel.shape[0]):
            want = [j for j in ref[r].sel[i] if j >= 0]
            n = int(n_sel[i, r])
            assert sel[i, r, :n].tolist() == want, f"{name} row {r} query block {i}"
        assert np.isfinite(out[b, :, g * G:(g + 1) * G]).all()
        np.testing.assert_allclose(out[b, :, g * G:(g + 1) * G], ref[r].out,
                                   err_msg=f"{name} row {r}", **TOL)


# Full size: the 32k-token context of the 8-sequence, 32/8-head, D 128
# workload (k = 48 + 16), in the launch configuration the benchmark times.
# Every (query block, row) is checked for properties that hold at any size;
# sampled rows and query blocks (first, small, around k, middle, last) are
# checked against the oracle, with their selection margins enforced.
FULL_ROWS = (0, 29, 63)
FULL_QBLOCKS = (0, 1, 47, 64, 65, 200, 511)


def _fullsize_margins(w: Workload):
    N, G = w.context, w.group
    sc = 1.0 / math.sqrt(w.head_dim)
    pb = w.pooled == "bf16"
    ov = Overrides()
    cmax = max(FULL_QBLOCKS)
    for r in FULL_ROWS:
        b, g = divmod(r, w.n_kv_heads)
        K, _ = row_kv(w, 0, b, g)
        for _ in range(256):
            e = synth.evict_row(w, 0, b, g, ov)
            E = np.array([oracle.block_evict(e, 64, 16, j) for j in range(cmax)])
            bad = None
            for i in FULL_QBLOCKS:
                ok, lower = boundary_ok(E[:i], w.k_e)
                if not ok:
                    bad = lower
                    break
            if bad is None:
                break
            key = (0, b, g, bad)
            ov.evict[key] = ov.evict.get(key, 0) + 1
        else:
            raise RuntimeError("eviction margins")
        qrow = synth.prefill_queries(w, 0, N, ov, batch=b)
        for i in FULL_QBLOCKS:
            if i <= w.k:
                continue  # every candidate is selected
            ge = set(sorted(range(i), key=lambda j: (-E[j], j))[:w.k_e])
            rest = [j for j in range(i) if j not in ge]
            for _ in range(64):
                q = qrow[64 * i:64 * i + 64, g * G:(g + 1) * G]
                qb = oracle.pool_queries(q, pooled_bf16=pb)
                S = np.array([oracle.block_score(qb, K, 64, 16, j, sc, pooled_bf16=pb)
                              for j in rest])
                if boundary_ok(S, w.k_q)[0]:
                    break
                key = ("prefill", 0, b, g, i)
                ov.query[key] = ov.query.get(key, 0) + 1
                qrow = synth.prefill_queries(w, 0, N, ov, batch=b)
            else:
                raise RuntimeError("query margins")
    return ov


def test_prefill_fullsize_sampled():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gpu_harness as gh
    w = synth.WORKLOADS["bf16_1layer_32k"]
    N, G, k = w.context, w.group, w.k
    sc = 1.0 / math.sqrt(w.head_dim)
    ov = _fullsize_margins(w)
    inp = gh.upload(w, ov=ov, steps=1)
    q_all = gh.to_device(gh.storage(synth.prefill_queries(w, 0, N, ov), w), w)
    layer = gh.make_layer(w, inp)
    out, sel, n_sel = layer.prefill(q_all, N)
    torch.cuda.synchronize()
    sel, n_sel = sel.cpu().numpy(), n_sel.cpu().numpy()
    nqb = N // 64
    # any size: query block i selects min(k, i) distinct earlier blocks, ascending
    for i in range(nqb):
        want_n = min(k, i)
        assert (n_sel[i] == want_n).all(), f"query block {i}"
        s = sel[i]
        if want_n:
            assert (s[:, :want_n] >= 0).all() and (s[:, :want_n] < i).all()
            assert (np.diff(s[:, :want_n], axis=1) > 0).all()
        assert (s[:, want_n:] == -1).all()
    assert torch.isfinite(out).all()
    for r in FULL_ROWS:
        b, g = divmod(r, w.n_kv_heads)
        K, V = row_kv(w, 0, b, g)
        e = synth.evict_row(w, 0, b, g, ov)
        q = synth.prefill_queries(w, 0, N, ov, batch=b)[:, g * G:(g + 1) * G]
        for i in FULL_QBLOCKS:
            ref = oracle.prefill_qblock(q, K[:N], V[:N], e[:N], i, 64, 16, w.k_e, w.k_q, sc,
                                        pooled_bf16=w.pooled == "bf16")
            want = [j for j in ref.sel[0] if j >= 0]
            assert sel[i, r, :len(want)].tolist() == want, f"row {r} query block {i}"
            got = out[b, 64 * i:64 * i + 64, g * G:(g + 1) * G].float().cpu().numpy()
            np.testing.assert_allclose(got, ref.out, err_msg=f"row {r} query block {i}", **TOL)


@pytest.mark.parametrize("name", ["prefill_bf16", "prefill_g3_d64", "prefill_g8",
                                  "prefill_bf16:pbf16", "prefill_g3_d64:pbf16"])
def test_pooled_queries_bit_exact(name):
    """nosa_prefill_pool_queries against the oracle's pooled query of every
    (query block, sequence, head), the last block ragged: bit for bit (the
    mean of bf16 values is exact in double and rounded once to the pooled
    dtype)."""
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gpu_harness as gh
    from trainable_block_sparse_nosa_amd import _lib as L
    w = _w(name)
    N = w.context
    nqb = -(-N // 64)
    pb = w.pooled == "bf16"
    qh = synth.prefill_queries(w, 0, N)                     # [batch][N][Hq][D]
    q_all = gh.to_device(gh.storage(qh, w), w)
    qbar = torch.empty(nqb, w.batch, w.n_q_heads, w.head_dim,
                       dtype=torch.bfloat16 if pb else torch.float32, device="cuda")
    shape = L.make_shape(w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.k_e, w.k_q,
                         -(-w.n_max // 64), L.NOSA_BF16, pooled_dtype=gh.pooled_dtype(w))
    L.nosa_prefill_pool_queries(shape, q_all, N, qbar, None)
    torch.cuda.synchronize()
    got = qbar.float().cpu().numpy()
    for i in range(nqb):
        for b in range(w.batch):
            ref = oracle.pool_queries(qh[b, 64 * i:64 * i + 64], pooled_bf16=pb)
            np.testing.assert_array_equal(got[i, b], ref.astype(np.float32),
                                          err_msg=f"{name} block {i} b {b}")


def test_prefill_large_values():
    """Large values in a few blocks, three whole blocks times 2^17 (one of them
    the ragged last block, attended causally by its own queries) and one token
    times 2^40: P enters P.V as a bf16 hi + lo pair over the full float32
    exponent range, so a small weight on a huge value keeps its ~16 bits and
    each output matches the oracle within the bf16 tolerance plus 2^-14 of the
    size of its terms (sum_t p_t |v_t| / l). (A single fp16 P, tried, loses
    such a weight below fp16's normal range and fails this case.)"""
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gpu_harness as gh
    w = PREFILL["prefill_bf16"]
    N, G, D = w.context, w.group, w.head_dim
    nqb = -(-N // 64)
    big_blocks, big_token = (2, 9, nqb - 1), 64 * 5 + 7
    sc = 1.0 / math.sqrt(D)
    ov, _ = _prefill_trace(w)

    def scaled_v(V):
        V = V.copy()
        for j in big_blocks:
            V[64 * j:64 * j + 64] *= np.float32(2.0 ** 17)
        V[big_token] *= np.float32(2.0 ** 40)
        return V

    inp = gh.upload(w, ov=ov, steps=1)
    kv = inp.kv.cpu()
    v_off = torch.from_numpy(gh.block_offsets(D, 2)[1])   # V[token][d] in a block
    for r in range(w.rows):
        for j in big_blocks:
            kv[r, j, v_off.reshape(-1)] *= 2.0 ** 17
        j, u = divmod(big_token, 64)
        kv[r, j, v_off[u]] *= 2.0 ** 40
    inp.kv.copy_(kv.to(inp.kv.device))
    q_all = gh.to_device(gh.storage(synth.prefill_queries(w, 0, N, ov), w), w)
    layer = gh.make_layer(w, inp)
    out, sel, n_sel = layer.prefill(q_all, N)
    torch.cuda.synchronize()
    out = out.float().cpu().numpy()
    for r in range(w.rows):
        b, g = divmod(r, w.n_kv_heads)
        K, V = row_kv(w, 0, b, g)
        e = synth.evict_row(w, 0, b, g, ov)
        q = synth.prefill_queries(w, 0, N, ov)[b, :, g * G:(g + 1) * G]
        Vs = scaled_v(V[:N])
        ref = oracle.prefill_row(q, K[:N], Vs, e[:N], 64, 16, w.k_e, w.k_q, sc)
        # the size of the terms behind each output, sum_t p_t |v_t| / l: where
        # large terms cancel, P's error (about 2^-18 of each weight, hi + lo)
        # is bounded by this, not by the small result
        mag = oracle.prefill_row(q, K[:N], np.abs(Vs), e[:N], 64, 16, w.k_e, w.k_q, sc).out
        got = out[b, :, g * G:(g + 1) * G]
        assert np.isfinite(got).all()
        bound = TOL["atol"] + TOL["rtol"] * np.abs(ref.out) + 2.0 ** -14 * mag
        bad = np.abs(got - ref.out) > bound
        assert not bad.any(), (f"row {r}: {int(bad.sum())} outputs, worst excess "
                               f"{float(np.max((np.abs(got - ref.out) - bound)[bad]))}")
        assert np.abs(ref.out).max() > 2.0 ** 16     # the planted values reach the outputs
