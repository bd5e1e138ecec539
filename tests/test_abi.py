"""The C-ABI library loads, exports every entry point its header declares,
and rejects bad arguments on the host before launching anything (no GPU
needed for these checks)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _no_gpu_visible():
    try:
        import torch
        return torch.cuda.device_count() == 0
    except Exception:
        return True


# These tests hand made-up pointers to the entry points to check that host-side
# validation rejects them; they must never run where a kernel could launch.
fake_pointers = pytest.mark.skipif(not _no_gpu_visible(),
                                   reason="made-up pointers are only passed where no GPU exists")


def _declared():
    with open(os.path.join(ROOT, "include", "nosa.h")) as f:
        text = f.read()
    return sorted(set(re.findall(r"\b(nosa_[a-z_]+)\s*\(", text)))


def test_header_declares_the_path_entry_points():
    names = _declared()
    for n in ("nosa_score_blocks", "nosa_select", "nosa_swap_diff", "nosa_fetch_blocks",
              "nosa_sparse_decode", "nosa_pool_blocks"):
        assert n in names


def test_library_exports_every_declared_symbol():
    from trainable_block_sparse_nosa_amd import _lib
    lib = ctypes.CDLL(_lib.LIB_PATH)
    missing = [n for n in _declared() if not hasattr(lib, n)]
    assert not missing, missing
    assert set(_lib.EXPORTS) == set(_declared())


def _shape(**kw):
    from trainable_block_sparse_nosa_amd import _lib as L
    a = dict(batch=2, n_q_heads=8, n_kv_heads=2, head_dim=128, k_e=4, k_q=4, max_blocks=64,
             dtype=L.NOSA_BF16)
    a.update(kw)
    return L.make_shape(**a)


@fake_pointers
@pytest.mark.parametrize("bad,status", [
    (dict(n_q_heads=7), 1),           # heads not a multiple of KV heads
    (dict(head_dim=96), 2),           # unsupported head_dim
    (dict(k_e=100, k_q=100), 2),      # budget above 128 blocks
    (dict(k_e=0, k_q=0), 1),          # empty budget
    (dict(dtype=5), 1),
    (dict(block_size=48), 2),
    (dict(sub_block=24), 1),          # block not a multiple of sub-block
    (dict(n_q_heads=32, n_kv_heads=2), 2),  # G = 16 > 8
    (dict(max_blocks=5000, k_e=4), 2),
    (dict(dtype=0, head_dim=128), 2),  # float32 supports head_dim 64 only
])
def test_invalid_shapes_rejected(bad, status):
    from trainable_block_sparse_nosa_amd import _lib as L
    sh = _shape(**bad)
    assert L.lib().nosa_decode_workspace_size(ctypes.byref(sh)) == 0
    st = L.make_step(100, -1)
    rc = L.lib().nosa_score_blocks(ctypes.byref(sh), 16, 16, ctypes.byref(st), 16, None)
    assert rc == status


@fake_pointers
def test_invalid_pointers_and_steps_rejected():
    from trainable_block_sparse_nosa_amd import _lib as L
    lib = L.lib()
    # the VALU plan needs the largest workspace, so a short one fails its check
    sh = _shape(decode_kernel=L.NOSA_DECODE_VALU)
    ok_step = L.make_step(100, -1)
    # null pointers
    assert lib.nosa_score_blocks(ctypes.byref(sh), None, 16, ctypes.byref(ok_step), 16, None) == 1
    assert lib.nosa_select(ctypes.byref(sh), 16, 16, ctypes.byref(ok_step), None, 16, 16, 16, 16,
                           None) == 1
    # fused score + select: null inputs, cache pointers given only in part
    P = [16] * 12
    assert lib.nosa_score_select(ctypes.byref(sh), None, 16, 16, ctypes.byref(ok_step), *P,
                                 None) == 1
    part = [16] * 6 + [16, 16, 16, None, 16, 16]
    assert lib.nosa_score_select(ctypes.byref(sh), 16, 16, 16, ctypes.byref(ok_step), *part,
                                 None) == 1
    # append: token slot and block out of range, null buffer
    assert lib.nosa_append_tokens(ctypes.byref(sh), 16, 16, 64, 16, 4, 0, None) == 1
    assert lib.nosa_append_tokens(ctypes.byref(sh), 16, 16, 3, 16, 4, 4, None) == 1
    assert lib.nosa_append_tokens(ctypes.byref(sh), 16, 16, -1, 16, 4, 0, None) == 1
    assert lib.nosa_append_tokens(ctypes.byref(sh), 16, 16, 3, None, 4, 0, None) == 1
    # merge that advances the device step record, without the record
    assert lib.nosa_decode_combine_step(ctypes.byref(sh), 1, 16, 16, 1 << 30, None, None) == 1
    # timed partial decode without its two events
    args = [ctypes.byref(sh), 16, 16, 64, L.NOSA_KV_FULL, 16, 16, 64, 64, 1, 16, 64,
            ctypes.byref(ok_step), 16, 64 * 64, 16, 1 << 30, 0]
    assert lib.nosa_decode_partial_timed(*args, None, 16, None) == 1
    assert lib.nosa_decode_partial_timed(*args, 16, None, None) == 1
    # attention with its merge: no out, one event without the other, an
    # empty list with no newest block
    a17 = args[:-1]
    assert lib.nosa_decode_attend(*a17, None, None, None, None) == 1
    assert lib.nosa_decode_attend(*a17, 16, 16, None, None) == 1
    assert lib.nosa_decode_attend(*a17, 16, None, 16, None) == 1
    empty = list(a17)
    empty[8], empty[9] = 0, 0
    assert lib.nosa_decode_attend(*empty, 16, None, None, None) == 1
    # a step beyond the block capacity
    big = L.make_step(64 * 64 + 1, -1)
    assert lib.nosa_score_blocks(ctypes.byref(sh), 16, 16, ctypes.byref(big), 16, None) == 1
    # previous candidate count above the current one
    back = L.make_step(200, 10)
    assert lib.nosa_select(ctypes.byref(sh), 16, 16, ctypes.byref(back), 16, 16, 16, 16, 16,
                           None) == 1
    # pooling outside the capacity / inconsistent strides
    assert lib.nosa_pool_blocks(ctypes.byref(sh), 16, 64, 0, 16, 64 * 64, 0, 65, 16, 16, None) == 1
    assert lib.nosa_pool_blocks(ctypes.byref(sh), 16, 4, 2, 16, 64 * 64, 0, 3, 16, 16, None) == 1
    assert lib.nosa_pool_blocks(ctypes.byref(sh), 16, 64, 0, 16, 100, 0, 3, 16, 16, None) == 1
    # fetch list longer than the budget
    assert lib.nosa_fetch_blocks(ctypes.byref(sh), 16, 64, 16, 16, 16, 9, 16, 8, None) == 1
    # decode: small workspace, misaligned pointers, bad mode, e stride too short
    ws = lib.nosa_decode_workspace_size(ctypes.byref(sh))
    assert ws > 0
    st = L.make_step(100, 0)
    args = lambda **o: dict(dict(q=16, kv=16, rb=64, mode=0, lst=16, nl=16, cur=16, crb=64,
                                 e=16, es=4096, out=16, ws=16, wsb=ws), **o)
    def call(a):
        return lib.nosa_sparse_decode(ctypes.byref(sh), a["q"], a["kv"], a["rb"], a["mode"],
                                      a["lst"], a["nl"], a["cur"], a["crb"], ctypes.byref(st),
                                      a["e"], a["es"], a["out"], a["ws"], a["wsb"], None)
    assert call(args(wsb=ws - 4)) == 4
    assert call(args(q=17)) == 1
    assert call(args(mode=3)) == 1
    assert call(args(es=99)) == 1             # shorter than the blocks present
    assert call(args(es=130)) == 1            # not a multiple of 4
    assert call(args(e=20)) == 1              # not 16-byte aligned
    assert call(args(mode=1, rb=7)) == 1      # cache smaller than k slots
    assert call(args(nl=None)) == 1           # full mode needs the list length
    # host allocation needs a size
    h, d = ctypes.c_void_p(), ctypes.c_void_p()
    assert lib.nosa_host_alloc(0, 0, ctypes.byref(h), ctypes.byref(d)) == 1
    assert lib.nosa_status_string(2) == b"unsupported shape"
    # MFMA decode is bf16 only
    f32 = _shape(dtype=L.NOSA_F32, head_dim=64, decode_kernel=L.NOSA_DECODE_MFMA)
    assert lib.nosa_sparse_decode(ctypes.byref(f32), 16, 16, 64, 0, 16, 16, 16, 64,
                                  ctypes.byref(st), 16, 4096, 16, 16, 1 << 30, None) == 2


@fake_pointers
def test_device_step_calls_validate_against_the_capacity():
    """The *_step calls cannot read the record on the host: they check their
    buffers against the shape's capacity (max_blocks) before any launch."""
    from trainable_block_sparse_nosa_amd import _lib as L
    lib = L.lib()
    sh = _shape()
    mb = sh.max_blocks
    # null record
    assert lib.nosa_step_advance(ctypes.byref(sh), None, None) == 1
    assert lib.nosa_pool_step(ctypes.byref(sh), 16, mb, 16, mb * 64, None, 16, 16, None) == 1
    # KV rows or eviction rows shorter than the capacity
    assert lib.nosa_pool_step(ctypes.byref(sh), 16, mb - 1, 16, mb * 64, 16, 16, 16, None) == 1
    assert lib.nosa_pool_step(ctypes.byref(sh), 16, mb, 16, mb * 64 - 4, 16, 16, 16, None) == 1
    assert lib.nosa_append_step(ctypes.byref(sh), 16, 16, 16, mb - 1, 16, None) == 1
    assert lib.nosa_append_step(ctypes.byref(sh), None, 16, 16, mb, 16, None) == 1
    # fused score + select: null record, cache pointers given only in part
    P = [16] * 12
    assert lib.nosa_score_select_step(ctypes.byref(sh), 16, 16, 16, None, *P, None) == 1
    part = [16] * 6 + [16, 16, 16, None, 16, 16]
    assert lib.nosa_score_select_step(ctypes.byref(sh), 16, 16, 16, 16, *part, None) == 1
    # decode: newest block taken from a full KV shorter than the capacity, e
    # stride shorter than the capacity, null record
    ws = lib.nosa_decode_workspace_size(ctypes.byref(sh))
    args = lambda **o: dict(dict(q=16, kv=16, rb=mb, mode=0, lst=16, nl=16, cur=16, crb=mb,
                                 st=16, e=16, es=mb * 64, ws=16, wsb=ws), **o)

    def call(a):
        return lib.nosa_decode_partial_step(ctypes.byref(sh), a["q"], a["kv"], a["rb"],
                                            a["mode"], a["lst"], a["nl"], sh.k_e + sh.k_q,
                                            sh.k_e + sh.k_q, 1, a["cur"], a["crb"], a["st"],
                                            a["e"], a["es"], a["ws"], a["wsb"], 0, None)
    assert call(args(crb=mb - 1)) == 1
    assert call(args(es=mb * 64 - 4)) == 1
    assert call(args(st=None)) == 1
    assert call(args(rb=mb - 1)) == 1


def test_decode_chunk_plan():
    """The attention plan, host logic only: about one 8-wave workgroup per CU
    (256), so ceil(256 / rows) chunks per row, at least one block per wave;
    one chunk per row from 256 rows on, where nosa_decode_attend writes the
    output in the attention launch with no merge launch. The list splits
    evenly over the chunks and the newest block joins the last one."""
    from trainable_block_sparse_nosa_amd import _lib as L
    # 64 rows (batch 8 x 8 KV heads), 64 + 1 entries: 4 chunks
    sh = _shape(batch=8, n_q_heads=32, n_kv_heads=8, k_e=48, k_q=16, max_blocks=1024)
    assert L.nosa_decode_chunks(sh, 64, 1) == 4
    # few entries cap the chunks at one block per wave: 9 entries -> 2 chunks
    assert L.nosa_decode_chunks(sh, 8, 1) == 2
    # the query-aware part alone (16 blocks, no newest): 2 chunks of 8
    assert L.nosa_decode_chunks(sh, 16, 0) == 2
    # the newest block alone, or with one listed block: one chunk
    assert L.nosa_decode_chunks(sh, 0, 1) == 1
    assert L.nosa_decode_chunks(sh, 1, 1) == 1
    # 17 + 1 entries: 3 chunks (6, 6 and 5 + the newest)
    assert L.nosa_decode_chunks(sh, 17, 1) == 3
    assert L.nosa_decode_chunks(sh, 0, 0) == 0
    # 256 rows (batch 32 x 8 KV heads), 128 + 1 entries: one chunk per row
    sh = _shape(batch=32, n_q_heads=24, n_kv_heads=8, k_e=96, k_q=32, max_blocks=1024)
    assert L.nosa_decode_chunks(sh, 128, 1) == 1
    # 128 rows: 2 chunks
    sh = _shape(batch=16, n_q_heads=32, n_kv_heads=8, k_e=48, k_q=16, max_blocks=2048)
    assert L.nosa_decode_chunks(sh, 64, 1) == 2


def test_kbar_bytes_by_dtype():
    """Size of the pooled-key buffer per row and quad of 4 blocks (16 sub-blocks
    x D means): float32 keys and means 4 bytes each; bf16 keys with bf16 means
    2 bytes; bf16 keys with float32 means (certified scoring) the float32 means,
    then their bf16 copy in the same layout, then a float32 radius per block.
    The radius region sits after whole quads, so a max_blocks that is not a
    multiple of 4 still rounds the means up."""
    from trainable_block_sparse_nosa_amd import _lib as L
    rows, D = 2 * 2, 128
    for nb in (64, 63):
        quads = (nb + 3) // 4
        means = rows * quads * 16 * D
        assert L.nosa_kbar_bytes(_shape(max_blocks=nb, pooled_dtype=L.NOSA_BF16)) == 2 * means
        assert (L.nosa_kbar_bytes(_shape(max_blocks=nb, pooled_dtype=L.NOSA_F32))
                == 4 * means + 2 * means + 4 * rows * nb)
        f32 = _shape(max_blocks=nb, dtype=L.NOSA_F32, head_dim=64, pooled_dtype=L.NOSA_F32)
        assert L.nosa_kbar_bytes(f32) == 4 * rows * quads * 16 * 64
    # an invalid shape has no buffer: the C call returns 0, the binding raises
    import ctypes
    bad = _shape(n_q_heads=7)
    assert L.lib().nosa_kbar_bytes(ctypes.byref(bad)) == 0
    with pytest.raises(L.NosaError):
        L.nosa_kbar_bytes(bad)


def test_plan_and_sizes_over_random_shapes():
    """Host-side sizing over random valid shapes: every split-K plan fits the
    workspace the library asks for, including the two partial calls of an
    overlapped step (the eviction set with the newest block, then the
    query-aware set) in one workspace; a plan has at least one chunk when
    anything is attended and never more chunks than entries; with the
    matrix-core kernel at most ceil(256 / rows) chunks per row."""
    hypothesis = pytest.importorskip("hypothesis")
    from hypothesis import given, settings, strategies as st
    from trainable_block_sparse_nosa_amd import _lib as L

    @st.composite
    def shapes(draw):
        D = draw(st.sampled_from([64, 128]))
        dtype = L.NOSA_F32 if D == 64 and draw(st.booleans()) else L.NOSA_BF16
        kind = draw(st.sampled_from([L.NOSA_DECODE_AUTO, L.NOSA_DECODE_VALU]
                                    + ([L.NOSA_DECODE_MFMA] if dtype == L.NOSA_BF16 else [])))
        k_e = draw(st.integers(0, 128))
        k_q = draw(st.integers(1 if k_e == 0 else 0, 128 - k_e))
        hkv = draw(st.integers(1, 8))
        G = draw(st.integers(1, 8))
        return L.make_shape(draw(st.integers(1, 64)), G * hkv, hkv, D, k_e, k_q,
                            draw(st.integers(k_e + k_q, 4096)), dtype, decode_kernel=kind)

    @settings(max_examples=300, deadline=None)
    @given(shapes(), st.data())
    def check(sh, data):
        k = sh.k_e + sh.k_q
        rows, G, D = sh.batch * sh.n_kv_heads, sh.n_q_heads // sh.n_kv_heads, sh.head_dim
        cap = k + 2
        assert L.nosa_decode_workspace_size(sh) >= rows * cap * G * (D + 2) * 4
        mfma = sh.decode_kernel == L.NOSA_DECODE_MFMA or (
            sh.decode_kernel == L.NOSA_DECODE_AUTO and sh.dtype == L.NOSA_BF16)
        n = data.draw(st.integers(0, k))
        for newest in (0, 1):
            c = L.nosa_decode_chunks(sh, n, newest)
            if n + newest == 0:
                assert c == 0
                continue
            assert 1 <= c <= min(n + newest, cap)
            if mfma:
                assert c <= max(1, -(-256 // rows))
        assert L.nosa_decode_chunks(sh, sh.k_e, 1) + L.nosa_decode_chunks(sh, sh.k_q, 0) <= cap
        assert L.lib().nosa_decode_chunks(ctypes.byref(sh), k + 1, 1) == -1

    check()


@pytest.mark.parametrize("D,dt", [(64, "bf16"), (128, "bf16"), (64, "f32")])
def test_block_layout(D, dt):
    """The block layout the library reports equals the packing the Python layer
    uses, places every element once, and makes each bf16 fragment exactly the
    A operand of v_mfma_f32_16x16x32_bf16 (lane l: row l % 16, k-elements
    8 (l / 16) .. + 7 of a 32-wide step), for K and for the transposed V."""
    import numpy as np
    from trainable_block_sparse_nosa_amd import _lib as L
    from trainable_block_sparse_nosa_amd.pipeline import (VT_TOKEN_AT, block_offsets, pack_blocks,
                                                          unpack_blocks)
    dtype = L.NOSA_BF16 if dt == "bf16" else L.NOSA_F32
    itemsize = 2 if dt == "bf16" else 4
    k_off, v_off = L.nosa_block_offsets(_shape(head_dim=D, dtype=dtype))
    k_py, v_py = block_offsets(D, itemsize)
    np.testing.assert_array_equal(k_off, k_py)
    np.testing.assert_array_equal(v_off, v_py)
    every = np.sort(np.concatenate([k_off.ravel(), v_off.ravel()]))
    np.testing.assert_array_equal(every, np.arange(2 * 64 * D))
    assert k_off.max() < 64 * D <= v_off.min()
    # pack / unpack agree with the offsets and invert each other
    rng = np.random.default_rng(7)
    npt = np.uint16 if dt == "bf16" else np.float32
    K = rng.integers(1, 1 << 15, (130, D)).astype(npt)
    V = rng.integers(1, 1 << 15, (130, D)).astype(npt)
    P = pack_blocks(K, V, 3)
    for b in range(2):
        np.testing.assert_array_equal(P[b][k_off], K[64 * b:64 * b + 64])
        np.testing.assert_array_equal(P[b][v_off], V[64 * b:64 * b + 64])
    K2, V2 = unpack_blocks(P, D)
    np.testing.assert_array_equal(K2[:130], K)
    np.testing.assert_array_equal(V2[:130], V)
    assert not K2[130:].any() and not V2[130:].any()
    if dt != "bf16":
        return
    # fragment f, lane l = the 8 elements at 8 (64 f + l)
    for t in range(4):
        for s in range(D // 32):
            for lane in range(64):
                at = 8 * (64 * (t * (D // 32) + s) + lane)
                row, k0 = 16 * t + lane % 16, 32 * s + 8 * (lane // 16)
                np.testing.assert_array_equal(P[0][at:at + 8], K[row, k0:k0 + 8])
    for dtile in range(D // 16):
        for s in range(2):
            for lane in range(64):
                at = 64 * D + 8 * (64 * (2 * dtile + s) + lane)
                d, p0 = 16 * dtile + lane % 16, 32 * s + 8 * (lane // 16)
                np.testing.assert_array_equal(P[0][at:at + 8], V[VT_TOKEN_AT[p0:p0 + 8], d])


def test_block_offsets_rejects_bad_arguments():
    """nosa_block_offsets is host only: NULL arrays and unsupported shapes come
    back as errors before anything is written."""
    import numpy as np
    from trainable_block_sparse_nosa_amd import _lib as L
    lib = L.lib()
    good = np.zeros(64 * 128, np.int64)
    sh = _shape()
    assert lib.nosa_block_offsets(ctypes.byref(sh), None, good.ctypes.data) == L.NOSA_ERR_INVALID_ARGUMENT
    assert lib.nosa_block_offsets(ctypes.byref(sh), good.ctypes.data, None) == L.NOSA_ERR_INVALID_ARGUMENT
    bad = _shape(head_dim=96)
    k = np.full(64 * 96, -7, np.int64)
    v = np.full(64 * 96, -7, np.int64)
    assert lib.nosa_block_offsets(ctypes.byref(bad), k.ctypes.data, v.ctypes.data) == L.NOSA_ERR_UNSUPPORTED
    assert (k == -7).all() and (v == -7).all()
    with pytest.raises(L.NosaError):
        L.nosa_block_offsets(_shape(head_dim=128, dtype=L.NOSA_F32))   # float32 supports D = 64
