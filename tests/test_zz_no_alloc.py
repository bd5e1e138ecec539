"""nosa_sparse_decode_noalloc (for callers that cannot allocate: graph
capture, tight serving loops) against nosa_sparse_decode with a caller
workspace, through the C ABI: the same bits, on two calls in a row, the
second with a smaller input, for the matrix-core kernel with several chunks
per row (partials in the library's scratch), with one chunk per row (no
partials) and for the float32 VALU kernel; and a shape whose partials would
not fit the scratch is refused before any launch."""
import numpy as np
import pytest

import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gpu_harness
    return gpu_harness


def _both(gh, L, w, steps=3):
    """Run the pipeline for a few steps, then the last step's attention both
    ways; returns (with workspace, without)."""
    inp = gh.upload(w, steps=steps)
    layer, _ = gh.run(w, inp, list(range(steps)), collect=[])
    t = steps - 1
    c = w.n_cand(t)
    st = L.make_step(w.n_tokens(t), c)
    if w.offload:
        args = (layer.shape, inp.q[t], layer.cache, layer.k, L.NOSA_KV_CACHE, layer.slot_block,
                None, layer.cur, 1, st, layer.e_tok, layer.e_stride)
    else:
        args = (layer.shape, inp.q[t], layer.kv, layer.kv_row_blocks, L.NOSA_KV_FULL, layer.sel,
                layer.n_sel, layer._kv_ptr(c), layer.kv_row_blocks, st, layer.e_tok,
                layer.e_stride)
    ref = torch.full_like(layer.out, 7)
    L.nosa_sparse_decode(*args, ref, layer.ws, layer.ws_bytes)
    got = torch.full_like(layer.out, 9)
    L.nosa_sparse_decode_noalloc(*args, got)
    torch.cuda.synchronize()
    return layer, ref, got


def _same(a, b):
    it = torch.int16 if a.dtype == torch.bfloat16 else torch.int32
    return torch.equal(a.view(it).cpu(), b.view(it).cpu())


@pytest.mark.parametrize("base,smaller", [
    ("small_bf16", dict(batch=1, context=1200)),          # MFMA, several chunks per row
    ("small_offload", dict(batch=1, context=700)),        # MFMA over the HBM cache
    ("small_f32", dict(n_q_heads=3, n_kv_heads=1, context=500)),  # VALU, float32
])
def test_noalloc_matches_workspace_call(base, smaller):
    gh = _gpu()
    from trainable_block_sparse_nosa_amd import _lib as L
    w1 = synth.WORKLOADS[base]
    w2 = w1.scaled(name=w1.name + "_smaller", seed=w1.seed + 50, **smaller)
    assert w2.rows * w2.n_max < w1.rows * w1.n_max
    for w in (w1, w2):
        layer, ref, got = _both(gh, L, w)
        assert torch.isfinite(ref.float()).all()
        assert _same(ref, got), w.name
        if w.dtype == "bf16":
            assert L.nosa_decode_chunks(layer.shape, layer.k, 1) > 1  # partials in the scratch


def test_noalloc_one_chunk_per_row():
    gh = _gpu()
    from trainable_block_sparse_nosa_amd import _lib as L
    w = synth.WORKLOADS["small_bf16"].scaled(name="noalloc_256rows", seed=2301, batch=128,
                                             context=1500)
    layer, ref, got = _both(gh, L, w, steps=2)
    assert L.nosa_decode_chunks(layer.shape, layer.k, 1) == 1
    assert _same(ref, got)
    # and a multi-chunk call right after it on the same GPU
    w2 = synth.WORKLOADS["small_bf16"].scaled(name="noalloc_after", seed=2302, batch=1,
                                              context=900)
    layer2, ref2, got2 = _both(gh, L, w2, steps=2)
    assert L.nosa_decode_chunks(layer2.shape, layer2.k, 1) > 1
    assert _same(ref2, got2)


def test_noalloc_refuses_a_shape_beyond_its_scratch():
    """float32, 4096 rows, G = 8, k = 128: the VALU plan's partials need far
    more than the scratch holds; the host check refuses the call (no launch:
    the buffers passed are never read)."""
    _gpu()
    from trainable_block_sparse_nosa_amd import _lib as L
    shape = L.make_shape(512, 64, 8, 64, 96, 32, 4096, L.NOSA_F32)
    chunks = L.nosa_decode_chunks(shape, 128, 1)
    need = 512 * 8 * chunks * 8 * (64 + 2) * 4
    assert need > L.NOSA_NOALLOC_SCRATCH_BYTES
    buf = torch.zeros(1 << 16, dtype=torch.float32, device="cuda")
    ids = torch.zeros(512 * 8 * 128, dtype=torch.int32, device="cuda")
    st = L.make_step(64 * 200 + 5, 200)
    with pytest.raises(L.NosaError) as ei:
        L.nosa_sparse_decode_noalloc(shape, buf, buf, 4096, L.NOSA_KV_FULL, ids, ids, buf, 4096,
                                     st, buf, 64 * 4096, buf)
    assert ei.value.status == L.NOSA_ERR_WORKSPACE
