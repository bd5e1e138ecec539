"""HIP path vs the fp64 oracle, element by element, through the C ABI.

Bar: selections (Gamma_e, Gamma_q, their union), swap lists and slot tables
bit-exact; attention outputs within rtol 1e-5 / atol 1e-6 for float32 inputs
and rtol 2e-2 / atol 2e-3 for bfloat16 inputs; pooled scores within the
float32 accumulation error (well inside the 1e-4 selection margin).
"""
import numpy as np
import pytest

import synth
from harness import oracle_trace, workload

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

TOL = {"f32": dict(rtol=1e-5, atol=1e-6), "bf16": dict(rtol=2e-2, atol=2e-3)}


def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gpu_harness
    return gpu_harness


def _compare_step(w, tr, t, r, got, check_swap=True, check_slots=True):
    """Compare one (step, row) of the GPU snapshot `got` with the oracle."""
    import gpu_harness as gh
    ref = tr.step[(t, r)]
    c = ref.n_cand
    where = f"{w.name} t={t} row={r}"
    # pooled scores: float32 accumulation. A D-term float32 dot product errs by
    # about sqrt(D) * 2^-24 times the magnitude of its terms; 2e-6 of the term
    # scale covers D = 128 with room, and stays far inside the 1e-4 selection
    # margin the inputs are drawn with. The eviction scores are float32 means
    # of 16 logits: 2e-6 of the row's largest pooled magnitude (at least 1).
    # With certified scoring (bf16 keys, float32 pooled keys, nosa_score_select)
    # s_q holds the scores of the pooled keys' bf16 copy, within
    # scale * sum_h |q_h| * |copy - mean| <= 2^-8 of the term scale of the
    # float32 ones; the selection itself is settled on float32 scores.
    if c:
        e_scale = max(1.0, float(np.max(np.abs(ref.E))))
        np.testing.assert_allclose(got["e_blk"][r, :c], ref.E, rtol=0, atol=2e-6 * e_scale,
                                   err_msg=where)
        s_tol = 2.0 ** -8 if got.get("s_q_certified") else 2e-6
        np.testing.assert_allclose(got["s_q"][r, :c], ref.S, rtol=0,
                                   atol=s_tol * tr.term_scale[(t, r)], err_msg=where)
    # selections: bit-exact
    assert gh.bits_to_list(got["ge_bits"][r]) == ref.gamma_e, where
    n = int(got["n_sel"][r])
    assert got["sel"][r, :n].tolist() == ref.selected, where
    assert (got["sel"][r, n:] == -1).all(), where
    assert gh.bits_to_list(got["sel_bits"][r]) == ref.selected, where
    # strict eviction bookkeeping: evicted = candidates outside Gamma_e
    assert gh.bits_to_list(got["ev_bits"][r]) == sorted(set(range(c)) - set(ref.gamma_e)), where
    if check_swap:
        sw = tr.swap[(t, r)]
        nf = int(got["n_fetch"][r])
        assert got["fetch_block"][r, :nf].tolist() == sw.fetch_block, where
        if check_slots:
            assert got["fetch_slot"][r, :nf].tolist() == sw.fetch_slot, where
            assert got["slot_block"][r].tolist() == sw.slot_block, where
    # attention output of the row's G query heads
    b, g = divmod(r, w.n_kv_heads)
    G = w.group
    out = got["out"][b, g * G:(g + 1) * G]
    np.testing.assert_allclose(out, ref.out, err_msg=where, **TOL[w.dtype])


@pytest.mark.parametrize("name", ["small_f32", "small_bf16", "small_offload",
                                  "small_bf16:pbf16", "small_offload:pbf16"])
def test_pooled_keys(name):
    """Pooled sub-block means after the prefill pooling and the steps that
    complete further blocks, bit for bit: the oracle's exact mean rounded once
    to the pooled dtype (float32 by default, bfloat16 in the variant)."""
    import oracle
    from harness import row_kv
    gh = _gpu()
    w = workload(name)
    inp = gh.upload(w)
    steps = 72 if w.steps >= 72 else w.steps
    layer, _ = gh.run(w, inp, list(range(steps)))
    c = w.n_cand(steps - 1)
    assert c > w.n_cand(0), "the steps complete at least one block"
    D = w.head_dim
    kb = layer.kbar.float().cpu().numpy()          # [rows][quads][D/V][16][V]
    kb = kb.transpose(0, 1, 3, 2, 4).reshape(w.rows, -1, D)  # [rows][sub-block][D]
    for r in range(w.rows):
        b, g = divmod(r, w.n_kv_heads)
        K, _ = row_kv(w, 0, b, g)
        for j in range(c):
            ref = oracle.pool_keys(K, w.block, w.sub_block, j, pooled_bf16=w.pooled == "bf16")
            got = kb[r, 4 * j:4 * j + 4].astype(np.float64)
            where = f"{name} row={r} block={j}"
            np.testing.assert_array_equal(got, ref.astype(np.float32).astype(np.float64),
                                          err_msg=where)
    if layer.scores_certified:
        check_certificate(layer.kbar_buf, w.rows, layer.max_blocks, w.head_dim, c)


def check_certificate(kbar_buf, rows, max_blocks, D, c):
    """The stored certificate of certified scoring (bf16 keys, float32 pooled
    keys): the bf16 copy is each float32 mean rounded to the nearest bf16
    (ties to even), and each block's radius is at least max over its
    sub-blocks of ||copy - mean||_2 + 2^-14 ||mean||_2, the bound the
    selection's scoring intervals rest on."""
    quads = (max_blocks + 3) // 4
    n = rows * quads * 16 * D  # float32 means
    buf = kbar_buf.view(torch.int32).cpu().numpy().view(np.uint32)  # float32 words
    mean = buf[:n].view(np.float32).reshape(rows, quads, D // 4, 16, 4)
    mean = mean.transpose(0, 1, 3, 2, 4).reshape(rows, -1, D).astype(np.float64)
    sh16 = buf[n:n + n // 2].view(np.uint16).reshape(rows, quads, D // 8, 16, 8)
    sh = (sh16.astype(np.uint32) << 16).view(np.float32)
    sh = sh.transpose(0, 1, 3, 2, 4).reshape(rows, -1, D).astype(np.float64)
    rad = buf[n + n // 2:n + n // 2 + rows * max_blocks].view(np.float32)
    rad = rad.reshape(rows, max_blocks).astype(np.float64)
    want_sh = synth.rne_bf16(mean[:, :4 * c].astype(np.float32)).astype(np.float64)
    np.testing.assert_array_equal(sh[:, :4 * c], want_sh, err_msg="bf16 copy of the means")
    need = (np.sqrt(((sh[:, :4 * c] - mean[:, :4 * c]) ** 2).sum(-1))
            + 2.0 ** -14 * np.sqrt((mean[:, :4 * c] ** 2).sum(-1)))
    need = need.reshape(rows, c, 4).max(-1)
    assert (rad[:, :c] >= need).all(), float(np.max(need - rad[:, :c]))
    # and not loose: within 2^-9 of the bound (the enlargement is 2^-10)
    assert (rad[:, :c] <= need * (1 + 2.0 ** -9) + 1e-30).all()


@pytest.mark.parametrize("name", ["tiny_f32", "small_f32", "small_bf16", "small_offload",
                                  "small_bf16:pbf16", "small_offload:pbf16"])
def test_parity_all_steps_all_rows(name):
    gh = _gpu()
    w = workload(name)
    tr = oracle_trace(w)
    inp = gh.upload(w, ov=tr.ov)
    _, res = gh.run(w, inp, list(range(w.steps)))
    for t in range(w.steps):
        for r in range(w.rows):
            _compare_step(w, tr, t, r, res[t])


@pytest.mark.parametrize("name", ["small_bf16", "small_offload", "d64"])
def test_parity_valu_kernel_bf16(name):
    """The VALU decode kernel on bf16 inputs (the default there is MFMA); at
    head_dim 64 too, where a block's K and V^T vectors map back to the LDS
    tiles with two dimension groups per fragment row instead of four."""
    gh = _gpu()
    from trainable_block_sparse_nosa_amd import _lib as L
    if name == "d64":
        w = synth.WORKLOADS["small_bf16"].scaled(name="valu_bf16_d64", seed=3200, n_q_heads=6,
                                                 n_kv_heads=2, head_dim=64, context=1300,
                                                 steps=12)
    else:
        w = synth.WORKLOADS[name]
    tr = oracle_trace(w)
    inp = gh.upload(w, ov=tr.ov)
    _, res = gh.run(w, inp, list(range(w.steps)), decode_kernel=L.NOSA_DECODE_VALU)
    for t in range(w.steps):
        for r in range(w.rows):
            _compare_step(w, tr, t, r, res[t])


@pytest.mark.parametrize("name", ["small_f32", "small_bf16", "small_offload"])
def test_parity_device_append(name):
    """The KV holds the context only; every step's token enters on the GPU
    through nosa_append_tokens. Offloaded, a block completed during the run is
    written back to host memory (and fetched from there when selected), so the
    host bytes are checked against the tokens as well."""
    from harness import row_kv
    gh = _gpu()
    w = synth.WORKLOADS[name]
    tr = oracle_trace(w)
    inp = gh.upload(w, ov=tr.ov, prefix_only=True)
    layer, res = gh.run(w, inp, list(range(w.steps)))
    for t in range(w.steps):
        for r in range(w.rows):
            _compare_step(w, tr, t, r, res[t])
    c0, c1 = w.n_cand(0), w.n_cand(w.steps - 1)
    assert c1 > c0, "the run completes a block"
    if not w.offload:
        return
    D = w.head_dim
    host = inp.kv.array(np.uint16, (w.rows, inp.nb, 2 * 64 * D))
    for r in range(w.rows):
        b, g = divmod(r, w.n_kv_heads)
        K, V = row_kv(w, 0, b, g)
        for j in range(c0, c1):
            k_tile, v_tile = gh.unpack_blocks(host[r, j:j + 1], D)
            np.testing.assert_array_equal(k_tile, synth.bf16_bits(K[64 * j:64 * j + 64]),
                                          err_msg=f"row {r} block {j} K")
            np.testing.assert_array_equal(v_tile, synth.bf16_bits(V[64 * j:64 * j + 64]),
                                          err_msg=f"row {r} block {j} V")


@pytest.mark.parametrize("name", ["small_bf16", "small_offload", "small_bf16:pbf16"])
def test_parity_separate_score_kernel(name):
    """nosa_score_blocks then nosa_select_swap as two launches (the pipeline
    scores and selects through nosa_score_select)."""
    gh = _gpu()
    w = workload(name)
    tr = oracle_trace(w)
    inp = gh.upload(w, ov=tr.ov)
    _, res = gh.run(w, inp, list(range(w.steps)), fuse_score=False)
    for t in range(w.steps):
        for r in range(w.rows):
            _compare_step(w, tr, t, r, res[t])


@pytest.mark.parametrize("name", ["tiny_f32", "small_f32"])
def test_parity_fused_score_select_f32(name):
    """nosa_score_select on float32 inputs (its VALU scoring; the pipeline
    fuses by default only for bf16, where the scores run on MFMA)."""
    gh = _gpu()
    w = synth.WORKLOADS[name]
    tr = oracle_trace(w)
    inp = gh.upload(w, ov=tr.ov)
    _, res = gh.run(w, inp, list(range(w.steps)), fuse_score=True)
    for t in range(w.steps):
        for r in range(w.rows):
            _compare_step(w, tr, t, r, res[t])


@pytest.mark.parametrize("name", ["small_f32", "small_offload"])
def test_parity_separate_select_and_swap(name):
    """nosa_score_blocks, nosa_select, then nosa_swap_diff as three calls."""
    gh = _gpu()
    w = synth.WORKLOADS[name]
    tr = oracle_trace(w)
    inp = gh.upload(w, ov=tr.ov)
    _, res = gh.run(w, inp, list(range(w.steps)), fuse_select_swap=False)
    for t in range(w.steps):
        for r in range(w.rows):
            _compare_step(w, tr, t, r, res[t])


@pytest.mark.parametrize("name", ["tiny_f32", "small_f32", "small_bf16"])
def test_parity_overlapped_decode(name):
    """Eviction-set attention on a side stream, query-set attention after the
    selection, then the merge (nosa_select_parts, nosa_decode_partial x2,
    nosa_decode_combine)."""
    gh = _gpu()
    w = synth.WORKLOADS[name]
    tr = oracle_trace(w)
    inp = gh.upload(w, ov=tr.ov)
    _, res = gh.run(w, inp, list(range(w.steps)), overlap=True)
    for t in range(w.steps):
        for r in range(w.rows):
            _compare_step(w, tr, t, r, res[t])


@pytest.mark.parametrize("append", [False, True])
def test_parity_offload_overlap(append):
    """Offloaded KV in two batch halves: the second half's fetch overlaps the
    first half's attention; every step and row against the oracle, with
    pre-generated tokens and with the device-side append and write-back."""
    gh = _gpu()
    w = synth.WORKLOADS["small_offload"]
    tr = oracle_trace(w)
    inp = gh.upload(w, ov=tr.ov, prefix_only=append)
    layer = gh.make_layer(w, inp, overlap=True, device_append=append)
    assert layer.overlap_fetch
    _, res = gh.run(w, inp, list(range(w.steps)), layer=layer)
    for t in range(w.steps):
        for r in range(w.rows):
            _compare_step(w, tr, t, r, res[t])


EDGE = {
    # fewer tokens than one block at the start: no candidates, then one
    "short_context": dict(context=10, steps=70, k_e=2, k_q=2),
    # the budget covers every candidate: sparse == dense over all tokens
    "budget_covers_all": dict(context=500, steps=30, k_e=4, k_q=8),
    # query-aware only / eviction only
    "no_eviction_budget": dict(context=1500, steps=20, k_e=0, k_q=6),
    "no_query_budget": dict(context=1500, steps=20, k_e=6, k_q=0),
    # GQA extremes and head_dim 64 in bf16
    "gqa1_d64": dict(n_q_heads=3, n_kv_heads=3, head_dim=64, context=1300, steps=20),
    "gqa8": dict(n_q_heads=16, n_kv_heads=2, context=1300, steps=20),
    # the other group sizes: 2, 5 (640 query elements: the certified
    # rescoring's second query pass is partial) and 6 at head_dim 64
    "gqa2": dict(n_q_heads=4, n_kv_heads=2, context=1300, steps=12),
    "gqa5": dict(n_q_heads=10, n_kv_heads=2, context=1300, steps=12),
    "gqa6_d64": dict(n_q_heads=12, n_kv_heads=2, head_dim=64, context=1300, steps=12),
    "gqa8_d64": dict(n_q_heads=16, n_kv_heads=2, head_dim=64, context=1300, steps=12),
    # ragged: context ends one token before a block boundary
    "ragged_boundary": dict(context=2047, steps=3, k_e=5, k_q=5),
    # the largest supported budget (eviction budget above 64: LDS top-k at start)
    "k128": dict(context=9000, steps=4, k_e=96, k_q=32),
    # query-aware budget above 64: LDS top-k every step
    "kq_large": dict(context=9000, steps=70, k_e=20, k_q=80),
    # 65..67 candidates: the second wave of the select kernel holds one to
    # three keys, fewer than the budget, while the first holds more than it;
    # the threshold must still be the exact k-th key
    "wave_tail_evict": dict(context=4161, steps=3, k_e=40, k_q=16, n_q_heads=16,
                            n_kv_heads=8),
    "wave_tail_query": dict(context=4161, steps=130, k_e=8, k_q=40),
    # near the capacity: 4093 blocks per row, 4091 then (a block completes at
    # step 2) 4092 candidates, 128 bitmap words in use, the largest budget
    # 96 + 32
    "max_capacity": dict(context=4092 * 64 - 2, steps=4, k_e=96, k_q=32),
}


@pytest.mark.parametrize("overlap", [False, True])
@pytest.mark.parametrize("edge", sorted(EDGE))
def test_parity_edge_cases(edge, overlap):
    gh = _gpu()
    base = synth.WORKLOADS["small_bf16"]
    w = base.scaled(name="edge_" + edge, seed=3000 + sorted(EDGE).index(edge), **EDGE[edge])
    tr = oracle_trace(w)
    inp = gh.upload(w, ov=tr.ov)
    _, res = gh.run(w, inp, list(range(w.steps)), overlap=overlap)
    for t in range(w.steps):
        for r in range(w.rows):
            _compare_step(w, tr, t, r, res[t])


# Near-ties under certified scoring (bf16 keys, float32 pooled keys): every
# key element carries a common offset of 64, so each pooled key's bf16 copy
# sits up to 0.25 per element from its float32 mean, while the blocks' scores
# differ by far less than the bound that follows from it. The copy's intervals
# then cover nearly every candidate: the exact rescoring runs over all of them
# (two passes of 128 blocks), and the copy's own top k_q is wrong at most steps.
NEAR_TIES = {
    # 4 rows: scores on the split grid, then the selection
    "split": dict(context=10000, steps=12, key_common=64.0),
    # 260 rows: scores inside the selecting workgroup
    "fused": dict(batch=65, n_q_heads=8, n_kv_heads=4, context=10000, steps=4, key_common=64.0),
    # head_dim 64 (a quarter of D is four 16-byte loads per lane), one query head per
    # KV head; split and fused
    "d64_g1": dict(n_q_heads=3, n_kv_heads=3, head_dim=64, context=10000, steps=6,
                   key_common=64.0),
    "d64_g1_fused": dict(batch=86, n_q_heads=3, n_kv_heads=3, head_dim=64, context=10000,
                         steps=3, key_common=64.0),
    # eight query heads per KV head
    "gqa8": dict(n_q_heads=16, n_kv_heads=2, context=10000, steps=6, key_common=64.0),
}


@pytest.mark.parametrize("case", sorted(NEAR_TIES))
def test_certified_scoring_near_ties(case):
    gh = _gpu()
    base = synth.WORKLOADS["small_bf16"]
    w = base.scaled(name="ties_" + case, seed=3400 + sorted(NEAR_TIES).index(case),
                    **NEAR_TIES[case])
    tr = oracle_trace(w)
    inp = gh.upload(w, ov=tr.ov)
    _, res = gh.run(w, inp, list(range(w.steps)))
    copy_wrong = 0
    for t in range(w.steps):
        assert res[t]["s_q_certified"]
        for r in range(w.rows):
            _compare_step(w, tr, t, r, res[t])
            ref = tr.step[(t, r)]
            ge = set(ref.gamma_e)
            s = res[t]["s_q"][r]
            rest = [j for j in range(ref.n_cand) if j not in ge]
            top = sorted(sorted(rest, key=lambda j: (-s[j], j))[:w.k_q])
            copy_wrong += top != sorted(ref.gamma_q)
    # the bf16 copy alone would have selected wrongly at most (step, row)s
    assert copy_wrong >= w.steps * w.rows // 2, copy_wrong


@pytest.mark.parametrize("edge", ["gqa1_d64", "gqa8", "k128", "kq_large", "max_capacity"])
def test_parity_edge_cases_pooled_bf16(edge):
    """Edge cases of the scoring shapes with pooled keys kept in bfloat16
    (scores on the matrix cores)."""
    gh = _gpu()
    base = synth.WORKLOADS["small_bf16"]
    w = base.scaled(name="edge_pbf16_" + edge, seed=3200 + sorted(EDGE).index(edge),
                    pooled="bf16", **EDGE[edge])
    tr = oracle_trace(w)
    inp = gh.upload(w, ov=tr.ov)
    _, res = gh.run(w, inp, list(range(w.steps)), overlap=False)
    for t in range(w.steps):
        for r in range(w.rows):
            _compare_step(w, tr, t, r, res[t])


OFFLOAD_EDGE = {
    # fewer tokens than two blocks at the start, one query head per KV head
    "gqa1_short": dict(seed=3100, n_q_heads=2, n_kv_heads=2, context=100, steps=40, k_e=2,
                       k_q=3),
    # head_dim 64 (16 KiB blocks) with eight query heads per KV head
    "d64_gqa8": dict(seed=3101, n_q_heads=16, n_kv_heads=2, head_dim=64, context=1500,
                     steps=20),
    # float32 KV over the HBM cache (the VALU attention kernel)
    "f32_d64": dict(seed=3102, dtype="f32", head_dim=64, context=1200, steps=20),
}


@pytest.mark.parametrize("edge", sorted(OFFLOAD_EDGE))
def test_offload_edge_cases(edge):
    gh = _gpu()
    w = synth.WORKLOADS["small_offload"].scaled(name="edge_offload_" + edge,
                                               **OFFLOAD_EDGE[edge])
    tr = oracle_trace(w)
    inp = gh.upload(w, ov=tr.ov)
    _, res = gh.run(w, inp, list(range(w.steps)))
    for t in range(w.steps):
        for r in range(w.rows):
            _compare_step(w, tr, t, r, res[t])


@pytest.mark.parametrize("name", ["small_bf16", "small_offload", "small_f32"])
def test_one_call_decode_matches_split_calls(name):
    """nosa_sparse_decode (partial + merge in one call) gives the same bits as
    the pipeline's attention call."""
    gh = _gpu()
    from trainable_block_sparse_nosa_amd import _lib as L
    w = synth.WORKLOADS[name]
    inp = gh.upload(w)
    layer, _ = gh.run(w, inp, list(range(w.steps)), collect=[])
    t = w.steps - 1
    c = w.n_cand(t)
    st = L.make_step(w.n_tokens(t), c)
    ref = layer.out.clone()
    out = torch.empty_like(ref)
    if w.offload:
        L.nosa_sparse_decode(layer.shape, inp.q[t], layer.cache, layer.k, L.NOSA_KV_CACHE,
                             layer.slot_block, None, layer.cur, 1, st, layer.e_tok,
                             layer.e_stride, out, layer.ws, layer.ws_bytes)
    else:
        L.nosa_sparse_decode(layer.shape, inp.q[t], layer.kv, layer.kv_row_blocks,
                             L.NOSA_KV_FULL, layer.sel, layer.n_sel, layer._kv_ptr(c),
                             layer.kv_row_blocks, st, layer.e_tok, layer.e_stride, out, layer.ws,
                             layer.ws_bytes)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16 if w.dtype == "bf16" else torch.int32),
                       ref.view(torch.int16 if w.dtype == "bf16" else torch.int32))


def test_deterministic_rerun():
    gh = _gpu()
    w = synth.WORKLOADS["small_bf16"]
    inp = gh.upload(w)
    _, a = gh.run(w, inp, list(range(w.steps)))
    _, b = gh.run(w, inp, list(range(w.steps)))
    for t in a:
        for key in a[t]:
            np.testing.assert_array_equal(a[t][key], b[t][key], err_msg=f"{key} t={t}")


def test_select_signed_zero_ties():
    """Scores of exactly +0 and -0 at both budget boundaries. The oracle
    compares them as equal numbers, so the lower block id ranks first; the
    kernel's integer keys must order them the same way (Gamma_e from the
    eviction scores, then Gamma_q from the query scores of the rest)."""
    _gpu()
    import oracle
    from trainable_block_sparse_nosa_amd import _lib as L
    n_cand, k_e, k_q, nb = 12, 3, 3, 16
    shape = L.make_shape(1, 4, 1, 128, k_e, k_q, nb, L.NOSA_BF16)
    e = np.zeros(nb, np.float32)
    s = np.zeros(nb, np.float32)
    e[:n_cand] = [-1.0, 0.0, -0.0, 0.0, -0.0, 0.0, -0.0, -1.0, -2.0, 0.0, -3.0, -4.0]
    s[:n_cand] = [-0.0, 0.0, 0.0, 0.0, 0.0, -0.0, 0.0, -5.0, -5.0, 0.0, -5.0, -5.0]
    ge_ref = oracle.topk(e[:n_cand], k_e)
    allowed = np.ones(n_cand, np.uint8)
    allowed[ge_ref] = 0
    gq_ref = oracle.topk(s[:n_cand], k_q, allowed)
    assert ge_ref == [1, 2, 3] and gq_ref == [0, 4, 5]
    dev = "cuda"
    e_d = torch.from_numpy(e).to(dev)[None]
    s_d = torch.from_numpy(s).to(dev)[None]
    ge = torch.zeros(1, 1, dtype=torch.int32, device=dev)
    ev = torch.zeros_like(ge)
    bits = torch.zeros_like(ge)
    sel = torch.full((1, k_e + k_q), -7, dtype=torch.int32, device=dev)
    n_sel = torch.zeros(1, dtype=torch.int32, device=dev)
    st = L.make_step(64 * n_cand + 1, -1)
    L.nosa_select(shape, s_d, e_d, st, ge, ev, sel, n_sel, bits, None)
    torch.cuda.synchronize()
    assert int(n_sel[0]) == k_e + k_q
    assert sel[0].tolist() == sorted(ge_ref + gq_ref)
    ge_bits = int(ge[0, 0].item()) & 0xFFFFFFFF
    assert [j for j in range(n_cand) if (ge_bits >> j) & 1] == ge_ref


def test_timed_partial_matches_untimed():
    """The attention call with events recorded at its kernel's own start and
    end (nosa_decode_attend with events; nosa_decode_partial_timed for a
    split step) writes the same bits as without them, and the events give a
    positive duration per call."""
    gh = _gpu()
    import bench
    from trainable_block_sparse_nosa_amd import _lib as L
    w = synth.WORKLOADS["small_bf16"]
    tr = oracle_trace(w)
    inp = gh.upload(w, ov=tr.ov)
    outs = []
    for timed in (False, True):
        layer = gh.make_layer(w, inp)
        ev = bench.HipTimingEvents(2 * w.steps)
        n = [0]

        def hook(name, fn, *a):
            if timed and fn in (L.nosa_decode_partial, L.nosa_decode_attend):
                bench.bracket(ev, 2 * n[0], 0, fn, a)
                n[0] += 1
            else:
                fn(*a)
        layer.stage_hook = hook
        layer.start(w.n_tokens(0))
        res = []
        for t in range(w.steps):
            layer.step(inp.q[t], w.n_tokens(t))
            res.append(layer.out.clone())
        torch.cuda.synchronize()
        outs.append(torch.stack(res).cpu())
        if timed:
            assert n[0] == w.steps
            assert all(ev.elapsed_ms(2 * i, 2 * i + 1) > 0 for i in range(n[0]))
        ev.close()
    assert torch.equal(outs[0], outs[1])


@pytest.mark.parametrize("name", ["small_bf16", "small_f32"])
def test_parity_large_eviction_logits(name):
    """Eviction logits scaled by 40 (|e| up to ~150, past where exp overflows
    float32 at ~88.7): the logit enters the softmax as an additive term, so
    the GPU path stays finite and matches the oracle; selections exact."""
    gh = _gpu()
    w = synth.WORKLOADS[name].scaled(name=name + "_large_e", steps=20)

    def tail(b, g, e):
        return (e * np.float32(40.0)).astype(np.float32)

    tr = oracle_trace(w, evict_tail=tail)
    inp = gh.upload(w, ov=tr.ov)
    e = inp.e_tok.cpu().numpy()
    for r in range(w.rows):
        b, g = divmod(r, w.n_kv_heads)
        e[r, :w.n_max] = tail(b, g, synth.evict_row(w, 0, b, g, tr.ov))
    assert np.abs(e).max() > 100.0
    inp.e_tok.copy_(torch.from_numpy(e))
    _, res = gh.run(w, inp, list(range(w.steps)))
    for t in range(w.steps):
        assert np.isfinite(res[t]["out"]).all()
        for r in range(w.rows):
            _compare_step(w, tr, t, r, res[t])


@pytest.mark.gpu
@pytest.mark.parametrize("name", ["bf16_1layer_32k", "bf16_3b_64k", "small_f32"])
def test_attend_matches_partial_then_merge(name):
    """nosa_decode_attend against nosa_decode_partial + nosa_decode_combine on
    the same selection: 64k (256 rows, one chunk per row: the matrix-
    core workgroup writes the output itself, in one launch), 32k (4 chunks
    per row: partials, then the merge kernel) and float32. With one chunk the
    merge's weight is exp(0) = 1, so the direct write is the same division of
    the same values: every case must agree bit for bit. Two calls, the second
    over the eviction set only (fewer chunks), each also with its two timing
    events (the bench's timed form). The one-call nosa_sparse_decode
    takes the same single launch on one chunk per row: checked on the full
    list."""
    gh = _gpu()
    from trainable_block_sparse_nosa_amd import _lib as L
    w = synth.WORKLOADS[name]
    inp = gh.upload(w, steps=1)
    layer = gh.make_layer(w, inp)
    layer.start(w.n_tokens(0))
    layer.step(inp.q[0], w.n_tokens(0))
    torch.cuda.synchronize()
    c = (w.n_tokens(0) - 1) // 64
    st = L.make_step(w.n_tokens(0), c)
    for list_len in (layer.k, w.k_e):
        args = (layer.shape, inp.q[0], layer.kv, layer.kv_row_blocks, L.NOSA_KV_FULL, layer.sel,
                layer.n_sel, layer.k, list_len, 1, layer._kv_ptr(c), layer.kv_row_blocks, st,
                layer.e_tok, layer.e_stride, layer.ws, layer.ws_bytes)
        got = torch.full_like(layer.out, 7)
        L.nosa_decode_attend(*args, got)
        want = torch.full_like(layer.out, 7)
        L.nosa_decode_partial(*args, 0)
        L.nosa_decode_combine(layer.shape, L.nosa_decode_chunks(layer.shape, list_len, 1), want,
                              layer.ws, layer.ws_bytes)
        torch.cuda.synchronize()
        g, x = got.cpu(), want.cpu()
        assert torch.isfinite(g.float()).all()
        assert torch.equal(g, x)
        # the same call with its two events (the bench's timed form)
        import bench
        ev = bench.HipTimingEvents(2)
        timed = torch.full_like(layer.out, 7)
        L.nosa_decode_attend(*args, timed, ev.handle(0), ev.handle(1))
        torch.cuda.synchronize()
        assert ev.elapsed_ms(0, 1) > 0
        ev.close()
        assert torch.equal(timed.cpu(), x)
        if list_len == layer.k:
            one = torch.full_like(layer.out, 7)
            L.nosa_sparse_decode(layer.shape, inp.q[0], layer.kv, layer.kv_row_blocks,
                                 L.NOSA_KV_FULL, layer.sel, layer.n_sel, layer._kv_ptr(c),
                                 layer.kv_row_blocks, st, layer.e_tok, layer.e_stride, one,
                                 layer.ws, layer.ws_bytes)
            torch.cuda.synchronize()
            assert torch.equal(one.cpu(), x)


@pytest.mark.parametrize("kernel", ["mfma", "valu"])
@pytest.mark.parametrize("base", ["small_bf16", "small_f32"])
def test_newest_block_tail_not_finite(base, kernel):
    """The newest block's slots past the last token hold NaN and infinities
    (keys, values and eviction scores): storage past n_tokens is whatever the
    buffer held before (torch.empty, a recycled block, tokens appended one at
    a time). Attention covers tokens [S * n_cand, n_tokens) only (ED-DMA,
    Methodology), so the outputs stay finite and match the oracle, which
    never reads those slots."""
    gh = _gpu()
    from trainable_block_sparse_nosa_amd import _lib as L
    if kernel == "mfma" and base == "small_f32":
        pytest.skip("the matrix-core attention is the bf16 kernel")
    w = synth.WORKLOADS[base]
    w = w.scaled(name=w.name + "_tail", context=64 * 46 + 6 if w.dtype == "bf16" else 64 * 14 + 3,
                 steps=4)
    tr = oracle_trace(w)
    inp = gh.upload(w, ov=tr.ov)
    T = w.steps
    c = w.n_cand(T - 1)
    assert c == w.n_cand(0), "every step attends the same partial newest block"
    lo = w.n_tokens(T - 1) - 64 * c          # first slot no step reads
    D = w.head_dim
    kv = inp.kv.cpu()
    bits = kv.view(torch.int16 if w.dtype == "bf16" else torch.int32)
    k_off, v_off = gh.block_offsets(D, 2 if w.dtype == "bf16" else 4)
    if w.dtype == "bf16":
        bad = [0x7FC0, 0x7F80, -128]           # NaN, +inf, -inf (0xFF80)
    else:
        bad = [0x7FC00000, 0x7F800000, -8388608]  # NaN, +inf, -inf (0xFF800000)
    for r in range(w.rows):
        for u in range(lo, 64):
            x = bad[u % 3]
            bits[r, c, torch.from_numpy(k_off[u])] = x
            bits[r, c, torch.from_numpy(v_off[u])] = x
    inp.kv.copy_(kv.to(inp.kv.device))
    e = inp.e_tok.cpu()
    e[:, 64 * c + lo:64 * c + 64] = float("nan")
    inp.e_tok.copy_(e.to(inp.e_tok.device))
    dk = L.NOSA_DECODE_MFMA if kernel == "mfma" else L.NOSA_DECODE_VALU
    _, res = gh.run(w, inp, list(range(T)), decode_kernel=dk)
    for t in range(T):
        assert np.isfinite(res[t]["out"]).all(), f"t={t}"
        for r in range(w.rows):
            _compare_step(w, tr, t, r, res[t])


@pytest.mark.parametrize("name,append", [("small_offload", False), ("small_offload", True),
                                         ("small_bf16", False), ("small_f32", True)])
def test_resume_from_state_dict(name, append):
    """Checkpoint / resume: the decode state after step t copied out
    (state_dict), a fresh layer built with the same arguments loads it and
    continues; every later step is bit for bit the uninterrupted run's
    (selections, eviction state, swap lists and slot tables, counters,
    outputs). t sits before a block boundary so the continuation pools a
    block and, offloaded, writes it back and fetches it."""
    gh = _gpu()
    w = synth.WORKLOADS[name]
    T = w.steps
    inp = gh.upload(w, prefix_only=append)
    steps = list(range(T))
    _, ref = gh.run(w, inp, steps)
    t_cut = next(t for t in steps if w.n_cand(t + 3) > w.n_cand(t)) - 1
    assert 0 < t_cut < T - 4
    first = gh.make_layer(w, inp, device_append=append)
    first.start(w.n_tokens(0))

    def step(layer, t):
        if append:
            layer.step(inp.q[t], w.n_tokens(t), k_new=inp.k_new[t], v_new=inp.v_new[t])
        else:
            layer.step(inp.q[t], w.n_tokens(t))

    for t in range(t_cut + 1):
        step(first, t)
    state = first.state_dict()
    del first
    torch.cuda.synchronize()
    second = gh.make_layer(w, inp, device_append=append)
    second.load_state_dict(state)
    for t in range(t_cut + 1, T):
        step(second, t)
        got = gh.snapshot(second, w)
        for key, want in ref[t].items():
            np.testing.assert_array_equal(got[key], want, err_msg=f"{name} t={t} {key}")


@pytest.mark.parametrize("case", ["rows4", "rows64"])
def test_attend_any_list_length(case):
    """nosa_decode_attend over the first n candidate blocks of every row, with
    and without the newest block, for list lengths that split unevenly over
    the chunks (4 rows: up to n + 1 chunks of one block per wave; 64 rows:
    4 chunks, the newest joining the last), against the oracle's softmax over
    exactly those tokens: every entry is attended once, whatever the length."""
    import math
    import oracle
    from harness import row_kv
    gh = _gpu()
    from trainable_block_sparse_nosa_amd import _lib as L
    base = synth.WORKLOADS["small_bf16"]
    w = base if case == "rows4" else base.scaled(name="attend_rows64", seed=3600, batch=32,
                                                 context=1500, steps=1)
    inp = gh.upload(w, steps=1)
    layer = gh.make_layer(w, inp)
    n_tok = w.n_tokens(0)
    c = (n_tok - 1) // 64
    k = layer.k
    assert c >= k
    st = L.make_step(n_tok, c)
    blocks = torch.arange(k, dtype=torch.int32, device="cuda").repeat(w.rows, 1).contiguous()
    q = inp.q[0].float().cpu().numpy()
    G, D = w.group, w.head_dim
    rows = {}
    for r in range(w.rows):
        b, g = divmod(r, w.n_kv_heads)
        K, V = row_kv(w, 0, b, g)
        rows[r] = (q[b, g * G:(g + 1) * G], K, V, synth.evict_row(w, 0, b, g))
    for n in sorted({1, 2, 7, 8, 9, k // 2, k - 1, k}):
        for newest in (1, 0):
            n_list = torch.full((w.rows,), n, dtype=torch.int32, device="cuda")
            out = torch.full_like(layer.out, 7)
            L.nosa_decode_attend(layer.shape, inp.q[0], layer.kv, layer.kv_row_blocks,
                                 L.NOSA_KV_FULL, blocks, n_list, k, n, newest,
                                 layer._kv_ptr(c), layer.kv_row_blocks, st, layer.e_tok,
                                 layer.e_stride, layer.ws, layer.ws_bytes, out)
            torch.cuda.synchronize()
            got = out.float().cpu().numpy()
            tokens = list(range(64 * n)) + (list(range(64 * c, n_tok)) if newest else [])
            for r, (qr, K, V, e) in rows.items():
                b, g = divmod(r, w.n_kv_heads)
                ref = oracle.attend_tokens(qr, K, V, e, tokens, 1.0 / math.sqrt(D))
                np.testing.assert_allclose(got[b, g * G:(g + 1) * G], ref, rtol=2e-2, atol=2e-3,
                                           err_msg=f"{case} n={n} newest={newest} row {r}")
