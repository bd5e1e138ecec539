"""ctypes binding of libnosa.so: the C ABI declared in include/nosa.h.

Argument marshalling only. Pointers may be given as torch tensors (their
data_ptr is passed), plain integers, or None for NULL; streams as
torch.cuda.Stream, an integer handle, or None for the current torch stream.
Every function raises NosaError on a non-zero status. There is no fallback:
if libnosa.so is missing, importing this module fails.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
# NOSA_LIB_PATH may point at another build of the same library (same ABI)
LIB_PATH = os.environ.get("NOSA_LIB_PATH") or os.path.join(_PKG, "libnosa.so")

NOSA_OK = 0
NOSA_ERR_INVALID_ARGUMENT = 1
NOSA_ERR_UNSUPPORTED = 2
NOSA_ERR_HIP = 3
NOSA_ERR_WORKSPACE = 4
NOSA_F32 = 0
NOSA_BF16 = 1
NOSA_KV_FULL = 0
NOSA_KV_CACHE = 1
NOSA_DECODE_AUTO = 0
NOSA_DECODE_VALU = 1
NOSA_DECODE_MFMA = 2

EXPORTS = (
    "nosa_pool_blocks", "nosa_score_blocks", "nosa_select", "nosa_select_swap", "nosa_swap_diff",
    "nosa_select_parts", "nosa_score_select", "nosa_fetch_blocks", "nosa_append_tokens",
    "nosa_ingest_tokens", "nosa_prefill_pool_queries", "nosa_prefill_select",
    "nosa_prefill_attention", "nosa_kbar_bytes", "nosa_decode_workspace_size",
    "nosa_decode_chunks", "nosa_block_offsets",
    "nosa_sparse_decode", "nosa_sparse_decode_noalloc", "nosa_decode_partial", "nosa_decode_partial_timed",
    "nosa_decode_combine", "nosa_decode_combine_step", "nosa_decode_attend",
    "nosa_step_advance", "nosa_pool_step", "nosa_append_step", "nosa_score_select_step",
    "nosa_decode_partial_step",
    "nosa_host_alloc", "nosa_host_free", "nosa_read_probe", "nosa_status_string",
    "nosa_last_error", "nosa_version",
)


class NosaError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        msg = _L.nosa_status_string(status).decode()
        detail = _L.nosa_last_error().decode()
        super().__init__(f"{fn}: {msg}" + (f" ({detail})" if detail and status == NOSA_ERR_HIP else ""))


class nosa_shape(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "batch", "n_q_heads", "n_kv_heads", "head_dim", "block_size", "sub_block", "k_e", "k_q",
        "max_blocks", "dtype", "decode_kernel")] + [("scale", ctypes.c_float),
                                                     ("pooled_dtype", ctypes.c_int32)]


class nosa_step(ctypes.Structure):
    _fields_ = [("n_tokens", ctypes.c_int32), ("n_cand_prev", ctypes.c_int32)]


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python trainable_block_sparse_nosa_amd/build.py`")
    L = ctypes.CDLL(LIB_PATH)
    P, I32, I64, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    SH, ST = ctypes.POINTER(nosa_shape), ctypes.POINTER(nosa_step)
    sig = {
        "nosa_pool_blocks": [SH, P, I64, I32, P, I64, I32, I32, P, P, P],
        "nosa_score_blocks": [SH, P, P, ST, P, P],
        "nosa_select": [SH, P, P, ST, P, P, P, P, P, P],
        "nosa_select_swap": [SH, P, P, ST, P, P, P, P, P, P, P, P, P, P, P, P],
        "nosa_swap_diff": [SH, P, P, P, P, P, P, P, P, P, P],
        "nosa_fetch_blocks": [SH, P, I64, P, P, P, I32, P, I64, P],
        "nosa_sparse_decode": [SH, P, P, I64, I32, P, P, P, I64, ST, P, I64, P, P, SZ, P],
        "nosa_sparse_decode_noalloc": [SH, P, P, I64, I32, P, P, P, I64, ST, P, I64, P, P],
        "nosa_select_parts": [SH, P, P, ST] + [P] * 15 + [P],
        "nosa_score_select": [SH, P, P, P, ST] + [P] * 12 + [P],
        "nosa_decode_chunks": [SH, I32, I32],
        "nosa_append_tokens": [SH, P, P, I32, P, I64, I32, P],
        "nosa_ingest_tokens": [SH, P, P, P, P, I32, I32, P, P, I64, I32, P, I64, P, P, P],
        "nosa_prefill_pool_queries": [SH, P, I32, P, P],
        "nosa_prefill_select": [SH, P, P, P, I32, P, P, P],
        "nosa_prefill_attention": [SH, P, I32, P, I64, P, I64, P, P, P, P],
        "nosa_decode_partial": [SH, P, P, I64, I32, P, P, I32, I32, I32, P, I64, ST, P, I64, P, SZ,
                                I32, P],
        "nosa_decode_partial_timed": [SH, P, P, I64, I32, P, P, I32, I32, I32, P, I64, ST, P, I64,
                                      P, SZ, I32, P, P, P],
        "nosa_decode_attend": [SH, P, P, I64, I32, P, P, I32, I32, I32, P, I64, ST, P, I64,
                               P, SZ, P, P, P, P],
        "nosa_decode_combine": [SH, I32, P, P, SZ, P],
        "nosa_decode_combine_step": [SH, I32, P, P, SZ, P, P],
        "nosa_host_alloc": [SZ, I32, ctypes.POINTER(P), ctypes.POINTER(P)],
        "nosa_host_free": [P],
        "nosa_read_probe": [P, I64, P, I32, P],
        "nosa_step_advance": [SH, P, P],
        "nosa_block_offsets": [SH, P, P],
        "nosa_pool_step": [SH, P, I64, P, I64, P, P, P, P],
        "nosa_append_step": [SH, P, P, P, I64, P, P],
        "nosa_score_select_step": [SH, P, P, P, P] + [P] * 12 + [P],
        "nosa_decode_partial_step": [SH, P, P, I64, I32, P, P, I32, I32, I32, P, I64, P, P, I64,
                                     P, SZ, I32, P],
    }
    for name, args in sig.items():
        f = getattr(L, name)
        f.argtypes = args
        f.restype = ctypes.c_int32
    L.nosa_decode_chunks.restype = ctypes.c_int32
    L.nosa_decode_workspace_size.argtypes = [SH]
    L.nosa_decode_workspace_size.restype = SZ
    L.nosa_kbar_bytes.argtypes = [SH]
    L.nosa_kbar_bytes.restype = SZ
    L.nosa_status_string.argtypes = [ctypes.c_int32]
    L.nosa_status_string.restype = ctypes.c_char_p
    L.nosa_last_error.argtypes = []
    L.nosa_last_error.restype = ctypes.c_char_p
    L.nosa_version.argtypes = []
    L.nosa_version.restype = ctypes.c_int32
    return L


_L = _load()


def lib() -> ctypes.CDLL:
    return _L


def _p(x):
    if x is None:
        return None
    if hasattr(x, "data_ptr"):
        return x.data_ptr()
    return int(x)


def _s(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if hasattr(stream, "cuda_stream"):
        return stream.cuda_stream
    return int(stream)


def _chk(fn: str, status: int):
    if status != NOSA_OK:
        raise NosaError(fn, status)


def make_shape(batch, n_q_heads, n_kv_heads, head_dim, k_e, k_q, max_blocks, dtype,
               block_size=64, sub_block=16, decode_kernel=NOSA_DECODE_AUTO, scale=0.0,
               pooled_dtype=NOSA_F32) -> nosa_shape:
    return nosa_shape(batch, n_q_heads, n_kv_heads, head_dim, block_size, sub_block, k_e, k_q,
                      max_blocks, dtype, decode_kernel, scale, pooled_dtype)


def make_step(n_tokens: int, n_cand_prev: int) -> nosa_step:
    return nosa_step(n_tokens, n_cand_prev)


def nosa_pool_blocks(shape, kv, kv_row_blocks, kv_first_block, e_tok, e_row_stride, blk_begin,
                     blk_end, kbar, e_blk, stream=None):
    _chk("nosa_pool_blocks", _L.nosa_pool_blocks(
        ctypes.byref(shape), _p(kv), kv_row_blocks, kv_first_block, _p(e_tok), e_row_stride,
        blk_begin, blk_end, _p(kbar), _p(e_blk), _s(stream)))


def nosa_score_blocks(shape, q, kbar, step, s_q, stream=None):
    _chk("nosa_score_blocks", _L.nosa_score_blocks(
        ctypes.byref(shape), _p(q), _p(kbar), ctypes.byref(step), _p(s_q), _s(stream)))


def nosa_select(shape, s_q, e_blk, step, ge_bits, ev_bits, sel, n_sel, sel_bits, stream=None):
    _chk("nosa_select", _L.nosa_select(
        ctypes.byref(shape), _p(s_q), _p(e_blk), ctypes.byref(step), _p(ge_bits), _p(ev_bits),
        _p(sel), _p(n_sel), _p(sel_bits), _s(stream)))


def nosa_select_swap(shape, s_q, e_blk, step, ge_bits, ev_bits, sel, n_sel, sel_bits, slot_block,
                     block_slot, fetch_block, fetch_slot, n_fetch, counters, stream=None):
    _chk("nosa_select_swap", _L.nosa_select_swap(
        ctypes.byref(shape), _p(s_q), _p(e_blk), ctypes.byref(step), _p(ge_bits), _p(ev_bits),
        _p(sel), _p(n_sel), _p(sel_bits), _p(slot_block), _p(block_slot), _p(fetch_block),
        _p(fetch_slot), _p(n_fetch), _p(counters), _s(stream)))


def nosa_select_parts(shape, s_q, e_blk, step, ge_bits, ev_bits, sel, n_sel, sel_bits, ge_list,
                      n_ge, gq_list, n_gq, slot_block=None, block_slot=None, fetch_block=None,
                      fetch_slot=None, n_fetch=None, counters=None, stream=None):
    _chk("nosa_select_parts", _L.nosa_select_parts(
        ctypes.byref(shape), _p(s_q), _p(e_blk), ctypes.byref(step), _p(ge_bits), _p(ev_bits),
        _p(sel), _p(n_sel), _p(sel_bits), _p(ge_list), _p(n_ge), _p(gq_list), _p(n_gq),
        _p(slot_block), _p(block_slot), _p(fetch_block), _p(fetch_slot), _p(n_fetch),
        _p(counters), _s(stream)))


def nosa_score_select(shape, q, kbar, e_blk, step, s_q, ge_bits, ev_bits, sel, n_sel, sel_bits,
                      slot_block=None, block_slot=None, fetch_block=None, fetch_slot=None,
                      n_fetch=None, counters=None, stream=None):
    _chk("nosa_score_select", _L.nosa_score_select(
        ctypes.byref(shape), _p(q), _p(kbar), _p(e_blk), ctypes.byref(step), _p(s_q),
        _p(ge_bits), _p(ev_bits), _p(sel), _p(n_sel), _p(sel_bits), _p(slot_block),
        _p(block_slot), _p(fetch_block), _p(fetch_slot), _p(n_fetch), _p(counters),
        _s(stream)))


def nosa_decode_chunks(shape, list_len, with_newest) -> int:
    n = _L.nosa_decode_chunks(ctypes.byref(shape), list_len, with_newest)
    if n < 0:
        raise NosaError("nosa_decode_chunks", NOSA_ERR_INVALID_ARGUMENT)
    return n


def nosa_decode_partial(shape, q, kv, kv_row_blocks, kv_mode, list_, n_list, list_stride,
                        list_len, with_newest, cur_kv, cur_row_blocks, step, e_tok, e_row_stride,
                        ws, ws_bytes, chunk0, stream=None):
    _chk("nosa_decode_partial", _L.nosa_decode_partial(
        ctypes.byref(shape), _p(q), _p(kv), kv_row_blocks, kv_mode, _p(list_), _p(n_list),
        list_stride, list_len, with_newest, _p(cur_kv), cur_row_blocks, ctypes.byref(step),
        _p(e_tok), e_row_stride, _p(ws), ws_bytes, chunk0, _s(stream)))


def nosa_decode_partial_timed(shape, q, kv, kv_row_blocks, kv_mode, list_, n_list, list_stride,
                              list_len, with_newest, cur_kv, cur_row_blocks, step, e_tok,
                              e_row_stride, ws, ws_bytes, chunk0, start_event, stop_event,
                              stream=None):
    """start_event / stop_event: hipEvent_t handles (ints or ctypes pointers)."""
    _chk("nosa_decode_partial_timed", _L.nosa_decode_partial_timed(
        ctypes.byref(shape), _p(q), _p(kv), kv_row_blocks, kv_mode, _p(list_), _p(n_list),
        list_stride, list_len, with_newest, _p(cur_kv), cur_row_blocks, ctypes.byref(step),
        _p(e_tok), e_row_stride, _p(ws), ws_bytes, chunk0, _p(start_event), _p(stop_event),
        _s(stream)))


def nosa_decode_attend(shape, q, kv, kv_row_blocks, kv_mode, list_, n_list, list_stride,
                       list_len, with_newest, cur_kv, cur_row_blocks, step, e_tok, e_row_stride,
                       ws, ws_bytes, out, start_event=None, stop_event=None, stream=None):
    """start_event / stop_event: both None, or hipEvent_t handles."""
    _chk("nosa_decode_attend", _L.nosa_decode_attend(
        ctypes.byref(shape), _p(q), _p(kv), kv_row_blocks, kv_mode, _p(list_), _p(n_list),
        list_stride, list_len, with_newest, _p(cur_kv), cur_row_blocks, ctypes.byref(step),
        _p(e_tok), e_row_stride, _p(ws), ws_bytes, _p(out), _p(start_event),
        _p(stop_event), _s(stream)))


def nosa_decode_combine(shape, n_chunks, out, ws, ws_bytes, stream=None):
    _chk("nosa_decode_combine", _L.nosa_decode_combine(
        ctypes.byref(shape), n_chunks, _p(out), _p(ws), ws_bytes, _s(stream)))


def nosa_decode_combine_step(shape, n_chunks, out, ws, ws_bytes, step_dev, stream=None):
    _chk("nosa_decode_combine_step", _L.nosa_decode_combine_step(
        ctypes.byref(shape), n_chunks, _p(out), _p(ws), ws_bytes, _p(step_dev), _s(stream)))


def nosa_swap_diff(shape, sel, n_sel, sel_bits, slot_block, block_slot, fetch_block, fetch_slot,
                   n_fetch, counters, stream=None):
    _chk("nosa_swap_diff", _L.nosa_swap_diff(
        ctypes.byref(shape), _p(sel), _p(n_sel), _p(sel_bits), _p(slot_block), _p(block_slot),
        _p(fetch_block), _p(fetch_slot), _p(n_fetch), _p(counters), _s(stream)))


def nosa_fetch_blocks(shape, src_kv, src_row_blocks, fetch_block, fetch_slot, n_fetch, max_fetch,
                      dst_kv, dst_row_blocks, stream=None):
    _chk("nosa_fetch_blocks", _L.nosa_fetch_blocks(
        ctypes.byref(shape), _p(src_kv), src_row_blocks, _p(fetch_block), _p(fetch_slot),
        _p(n_fetch), max_fetch, _p(dst_kv), dst_row_blocks, _s(stream)))


def nosa_append_tokens(shape, k_new, v_new, pos, kv, kv_row_blocks, block, stream=None):
    _chk("nosa_append_tokens", _L.nosa_append_tokens(
        ctypes.byref(shape), _p(k_new), _p(v_new), pos, _p(kv), kv_row_blocks, block, _s(stream)))


def nosa_ingest_tokens(shape, qkv, x, w_evict, b_evict, hidden, n_tokens, q_out, kv,
                       kv_row_blocks, block, e_tok, e_row_stride, kbar, e_blk, stream=None):
    _chk("nosa_ingest_tokens", _L.nosa_ingest_tokens(
        ctypes.byref(shape), _p(qkv), _p(x), _p(w_evict), _p(b_evict), hidden, n_tokens,
        _p(q_out), _p(kv), kv_row_blocks, block, _p(e_tok), e_row_stride, _p(kbar), _p(e_blk),
        _s(stream)))


def nosa_prefill_pool_queries(shape, q, n_tokens, qbar, stream=None):
    _chk("nosa_prefill_pool_queries", _L.nosa_prefill_pool_queries(
        ctypes.byref(shape), _p(q), n_tokens, _p(qbar), _s(stream)))


def nosa_prefill_select(shape, qbar, kbar, e_blk, n_tokens, sel, n_sel, stream=None):
    _chk("nosa_prefill_select", _L.nosa_prefill_select(
        ctypes.byref(shape), _p(qbar), _p(kbar), _p(e_blk), n_tokens, _p(sel), _p(n_sel),
        _s(stream)))


def nosa_prefill_attention(shape, q, n_tokens, kv, kv_row_blocks, e_tok, e_row_stride, sel, n_sel,
                           out, stream=None):
    _chk("nosa_prefill_attention", _L.nosa_prefill_attention(
        ctypes.byref(shape), _p(q), n_tokens, _p(kv), kv_row_blocks, _p(e_tok), e_row_stride,
        _p(sel), _p(n_sel), _p(out), _s(stream)))


def nosa_kbar_bytes(shape) -> int:
    n = _L.nosa_kbar_bytes(ctypes.byref(shape))
    if n == 0:
        raise NosaError("nosa_kbar_bytes", NOSA_ERR_INVALID_ARGUMENT)
    return n


def nosa_block_offsets(shape):
    """(k_off, v_off): int64 arrays [64, head_dim], the element offsets of
    K[tok][d] and V[tok][d] inside one KV block-unit (host only)."""
    D = shape.head_dim
    k_off = np.zeros((64, D), np.int64)
    v_off = np.zeros((64, D), np.int64)
    _chk("nosa_block_offsets", _L.nosa_block_offsets(
        ctypes.byref(shape), k_off.ctypes.data, v_off.ctypes.data))
    return k_off, v_off


def nosa_decode_workspace_size(shape) -> int:
    n = _L.nosa_decode_workspace_size(ctypes.byref(shape))
    if n == 0:
        raise NosaError("nosa_decode_workspace_size", NOSA_ERR_INVALID_ARGUMENT)
    return n


def nosa_sparse_decode(shape, q, kv, kv_row_blocks, kv_mode, list_, n_list, cur_kv,
                       cur_row_blocks, step, e_tok, e_row_stride, out, ws, ws_bytes, stream=None):
    _chk("nosa_sparse_decode", _L.nosa_sparse_decode(
        ctypes.byref(shape), _p(q), _p(kv), kv_row_blocks, kv_mode, _p(list_), _p(n_list),
        _p(cur_kv), cur_row_blocks, ctypes.byref(step), _p(e_tok), e_row_stride, _p(out), _p(ws),
        ws_bytes, _s(stream)))


def nosa_sparse_decode_noalloc(shape, q, kv, kv_row_blocks, kv_mode, list_, n_list, cur_kv,
                               cur_row_blocks, step, e_tok, e_row_stride, out, stream=None):
    _chk("nosa_sparse_decode_noalloc", _L.nosa_sparse_decode_noalloc(
        ctypes.byref(shape), _p(q), _p(kv), kv_row_blocks, kv_mode, _p(list_), _p(n_list),
        _p(cur_kv), cur_row_blocks, ctypes.byref(step), _p(e_tok), e_row_stride, _p(out),
        _s(stream)))


NOSA_NOALLOC_SCRATCH_BYTES = 16 << 20


def nosa_host_alloc(nbytes: int, coherent: bool = True) -> tuple[int, int]:
    h, d = ctypes.c_void_p(), ctypes.c_void_p()
    _chk("nosa_host_alloc", _L.nosa_host_alloc(nbytes, 1 if coherent else 0,
                                               ctypes.byref(h), ctypes.byref(d)))
    return h.value, d.value


def nosa_host_free(host: int):
    _chk("nosa_host_free", _L.nosa_host_free(host))


# Steps replayed from a captured graph: `step_dev` is a device buffer holding a
# nosa_step (int32 n_tokens, n_cand_prev), e.g. torch.int32 tensor of 2.

def nosa_step_advance(shape, step_dev, stream=None):
    _chk("nosa_step_advance", _L.nosa_step_advance(ctypes.byref(shape), _p(step_dev), _s(stream)))


def nosa_pool_step(shape, kv, kv_row_blocks, e_tok, e_row_stride, step_dev, kbar, e_blk,
                   stream=None):
    _chk("nosa_pool_step", _L.nosa_pool_step(
        ctypes.byref(shape), _p(kv), kv_row_blocks, _p(e_tok), e_row_stride, _p(step_dev),
        _p(kbar), _p(e_blk), _s(stream)))


def nosa_append_step(shape, k_new, v_new, kv, kv_row_blocks, step_dev, stream=None):
    _chk("nosa_append_step", _L.nosa_append_step(
        ctypes.byref(shape), _p(k_new), _p(v_new), _p(kv), kv_row_blocks, _p(step_dev),
        _s(stream)))


def nosa_score_select_step(shape, q, kbar, e_blk, step_dev, s_q, ge_bits, ev_bits, sel, n_sel,
                           sel_bits, slot_block=None, block_slot=None, fetch_block=None,
                           fetch_slot=None, n_fetch=None, counters=None, stream=None):
    _chk("nosa_score_select_step", _L.nosa_score_select_step(
        ctypes.byref(shape), _p(q), _p(kbar), _p(e_blk), _p(step_dev), _p(s_q), _p(ge_bits),
        _p(ev_bits), _p(sel), _p(n_sel), _p(sel_bits), _p(slot_block), _p(block_slot),
        _p(fetch_block), _p(fetch_slot), _p(n_fetch), _p(counters), _s(stream)))


def nosa_decode_partial_step(shape, q, kv, kv_row_blocks, kv_mode, list_, n_list, list_stride,
                             list_len, with_newest, cur_kv, cur_row_blocks, step_dev, e_tok,
                             e_row_stride, ws, ws_bytes, chunk0, stream=None):
    _chk("nosa_decode_partial_step", _L.nosa_decode_partial_step(
        ctypes.byref(shape), _p(q), _p(kv), kv_row_blocks, kv_mode, _p(list_), _p(n_list),
        list_stride, list_len, with_newest, _p(cur_kv), cur_row_blocks, _p(step_dev), _p(e_tok),
        e_row_stride, _p(ws), ws_bytes, chunk0, _s(stream)))


def nosa_read_probe(src, nbytes: int, sink, workgroups: int = 2048, stream=None):
    _chk("nosa_read_probe", _L.nosa_read_probe(_p(src), nbytes, _p(sink), workgroups,
                                               _s(stream)))


def nosa_version() -> int:
    return _L.nosa_version()
