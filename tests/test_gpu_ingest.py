"""The fused step before the path (nosa_ingest_tokens: QKV split, eviction
head, pooling of a completed block) against the oracle, through the C ABI:
the launch's outputs one by one, and whole decode steps fed by it."""
import numpy as np
import pytest

import synth
from harness import oracle_trace, row_kv
from test_gpu_parity import _compare_step, _gpu

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dtype,D,G,pos,pooled,hidden", [
    ("bf16", 128, 4, 10, "f32", 384), ("bf16", 128, 4, 63, "f32", 384),
    ("bf16", 64, 3, 63, "f32", 384), ("f32", 64, 2, 63, "f32", 384),
    ("bf16", 128, 4, 63, "bf16", 384), ("bf16", 64, 3, 63, "bf16", 384),
    ("bf16", 128, 8, 63, "f32", 384), ("bf16", 64, 1, 63, "f32", 384),
    # hidden sizes that are not a whole number of 16-byte vectors: the
    # eviction head's element-wise loop
    ("bf16", 128, 4, 63, "f32", 389), ("f32", 64, 2, 30, "f32", 390)])
def test_ingest_outputs(dtype, D, G, pos, pooled, hidden):
    """One launch: q split and the K/V slot bit for bit, the eviction logit
    within float32 summation error of the double sum, and (pos 63) the block's
    pooled keys bit for bit (the oracle's exact means rounded once to the
    pooled dtype) and its pooled eviction score."""
    import oracle
    gh = _gpu()
    from trainable_block_sparse_nosa_amd import _lib as L
    B, Hkv, nb = 2, 2, 8
    Hq = G * Hkv
    rows = B * Hkv
    w = synth.Workload("ingest_probe", 77, B, Hq, Hkv, D, 0, 1, 2, 2, dtype)
    rng = np.random.default_rng(5)
    cast = synth.rne_bf16 if dtype == "bf16" else (lambda a: a.astype(np.float32))
    j = 3
    tok = 64 * j + pos
    # the block's earlier tokens, already in the KV buffer and in e_tok
    K = cast(rng.normal(size=(rows, 64, D)).astype(np.float32))
    V = cast(rng.normal(size=(rows, 64, D)).astype(np.float32))
    e_tok = np.zeros((rows, nb * 64), np.float32)
    e_tok[:, 64 * j:64 * j + 64] = rng.normal(size=(rows, 64)).astype(np.float32)
    conv = (lambda a: a) if dtype == "f32" else synth.bf16_bits
    kv_host = np.zeros((rows, nb, 2 * 64 * D), np.float32 if dtype == "f32" else np.uint16)
    for r in range(rows):
        Kp, Vp = K[r].copy(), V[r].copy()
        Kp[pos:], Vp[pos:] = 0, 0               # slots from pos on are not written yet
        kv_host[r, j] = gh.pack_blocks(conv(Kp), conv(Vp), 1)[0]
    qkv = cast(rng.normal(size=(B, (Hq + 2 * Hkv) * D)).astype(np.float32))
    x = cast(rng.normal(size=(B, hidden)).astype(np.float32))
    W = cast((rng.normal(size=(Hkv, hidden)) / np.sqrt(hidden)).astype(np.float32))
    bias = np.array([0.25, -1.5], np.float32)
    dev = lambda a: gh.to_device(np.ascontiguousarray(a), w)
    kv = dev(kv_host)
    q_out = torch.zeros(B, Hq, D, dtype=kv.dtype, device="cuda")
    e_dev = torch.from_numpy(e_tok).cuda()
    V8 = 16 // (4 if pooled == "f32" else 2)
    e_blk = torch.zeros(rows, nb, dtype=torch.float32, device="cuda")
    shape = L.make_shape(B, Hq, Hkv, D, 2, 2, nb, L.NOSA_F32 if dtype == "f32" else L.NOSA_BF16,
                         pooled_dtype=L.NOSA_F32 if pooled == "f32" else L.NOSA_BF16)
    kdt = torch.float32 if pooled == "f32" else torch.bfloat16
    esz = 4 if pooled == "f32" else 2
    kbar_buf = torch.zeros(L.nosa_kbar_bytes(shape) // esz, dtype=kdt, device="cuda")
    kbar = kbar_buf[:rows * (nb // 4) * D * 16].view(rows, nb // 4, D // V8, 16, V8)
    L.nosa_ingest_tokens(shape, dev(conv(qkv)), dev(conv(x)), dev(conv(W)),
                         torch.from_numpy(bias).cuda(), hidden, tok + 1, q_out, kv, nb, j, e_dev,
                         nb * 64, kbar, e_blk)
    torch.cuda.synchronize()
    if dtype == "bf16" and pooled == "f32" and pos == 63:
        # the certificate of certified scoring, written by the same launch
        from test_gpu_parity import check_certificate
        check_certificate(kbar_buf, rows, nb, D, j + 1)
    got_q = q_out.float().cpu().numpy()
    got_kv = kv.float().cpu().numpy()
    got_e = e_dev.cpu().numpy()
    kb = kbar.float().cpu().numpy().transpose(0, 1, 3, 2, 4).reshape(rows, -1, D)
    got_eb = e_blk.cpu().numpy()
    k_off, v_off = gh.block_offsets(D, 4 if dtype == "f32" else 2)
    for b in range(B):
        q, k, v = oracle.qkv_split(qkv[b], Hq, Hkv, D)
        np.testing.assert_array_equal(got_q[b], q)
        for g in range(Hkv):
            r = b * Hkv + g
            blk = got_kv[r, j]
            np.testing.assert_array_equal(blk[k_off[pos]], k[g])
            np.testing.assert_array_equal(blk[v_off[pos]], v[g])
            e_ref = oracle.evict_logit(x[b], W[g], bias[g])
            scale = float(np.sum(np.abs(x[b].astype(np.float64) * W[g].astype(np.float64))))
            assert abs(got_e[r, tok] - e_ref) <= 1e-6 * max(scale, 1.0)
            if pos == 63:
                Kfull = K[r].copy()
                Kfull[63] = k[g]
                ref = oracle.pool_keys(Kfull, 64, 16, 0, pooled_bf16=pooled == "bf16")
                # float32 pooled keys: the exact mean rounded once to float32
                np.testing.assert_array_equal(kb[r, 4 * j:4 * j + 4], ref.astype(np.float32))
                e_blockrow = e_tok[r, 64 * j:64 * j + 64].copy()
                e_blockrow[63] = np.float32(e_ref)
                assert abs(got_eb[r, j] - oracle.block_evict(e_blockrow, 64, 16, 0)) <= 2e-6
            else:
                assert got_eb[r, j] == 0.0          # nothing pooled before the block completes


@pytest.mark.parametrize("name", ["small_bf16", "small_offload"])
def test_parity_device_ingest(name):
    """Whole decode steps whose q, new K/V and eviction logits come from the
    ingest launch (hidden states and the eviction head are synthetic, bias
    -4: decoded blocks rank far below the eviction set, so float32 and double
    sums of the head agree on every selection); offloaded, completed blocks
    are written back to host memory."""
    import oracle
    gh = _gpu()
    w = synth.WORKLOADS[name]
    T = w.steps
    W = synth.evict_head_weights(w, 0)
    bias = np.full(w.n_kv_heads, -4.0, np.float32)
    X = [synth.hidden_step(w, 0, t) for t in range(T)]

    def tail(b, g, e):
        e = e.copy()
        for t in range(T):
            e[w.context + t] = np.float32(oracle.evict_logit(X[t][b], W[g], bias[g]))
        return e

    tr = oracle_trace(w, evict_tail=tail)
    inp = gh.upload(w, ov=tr.ov, prefix_only=True)
    # the fused projection output of each step: [q heads | k heads | v heads] per batch
    qs = inp.q.view(T, w.batch, w.n_q_heads * w.head_dim)
    kn = inp.k_new.view(T, w.batch, w.n_kv_heads * w.head_dim)
    vn = inp.v_new.view(T, w.batch, w.n_kv_heads * w.head_dim)
    qkv = torch.cat([qs, kn, vn], dim=2).contiguous()
    x_dev = gh.to_device(np.stack([gh.storage(x, w) for x in X]), w)
    w_dev = gh.to_device(gh.storage(W, w), w)
    from trainable_block_sparse_nosa_amd.pipeline import DecodeLayer
    layer_ing = DecodeLayer(batch=w.batch, n_q_heads=w.n_q_heads, n_kv_heads=w.n_kv_heads,
                            head_dim=w.head_dim, k_e=w.k_e, k_q=w.k_q, max_blocks=inp.nb,
                            dtype=gh.nosa_dtype(w), kv=inp.kv_ptr, kv_row_blocks=inp.nb,
                            e_tok=inp.e_tok, offload=w.offload,
                            evict_head=(w_dev, torch.from_numpy(bias).cuda()))
    layer_ing.start(w.n_tokens(0))
    for t in range(T):
        layer_ing.step(None, w.n_tokens(t), qkv=qkv[t], x=x_dev[t])
        got = gh.snapshot(layer_ing, w)
        for r in range(w.rows):
            _compare_step(w, tr, t, r, got)
    assert w.n_cand(T - 1) > w.n_cand(0), "the run completes a block"
