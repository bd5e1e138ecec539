"""GPU-side helpers for the parity tests: upload seeded inputs, run the HIP
path step by step through the C ABI, and copy results back for comparison.

Inputs come from ``synth`` only; nothing here computes any of the method's
arithmetic.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np
import torch

import synth
from synth import Overrides, Workload
from trainable_block_sparse_nosa_amd import _lib as L
from trainable_block_sparse_nosa_amd.hostmem import PinnedBuffer
from trainable_block_sparse_nosa_amd.pipeline import (DecodeLayer, block_offsets,  # noqa: F401
                                                      pack_blocks, unpack_blocks)


def nosa_dtype(w: Workload) -> int:
    return L.NOSA_F32 if w.dtype == "f32" else L.NOSA_BF16


def pooled_dtype(w: Workload) -> int:
    return L.NOSA_BF16 if w.pooled == "bf16" else L.NOSA_F32


def storage(x: np.ndarray, w: Workload) -> np.ndarray:
    """float32 values (already in the input dtype) -> storage array."""
    return np.ascontiguousarray(x, np.float32) if w.dtype == "f32" else synth.bf16_bits(x)


def to_device(a: np.ndarray, w: Workload, device="cuda") -> torch.Tensor:
    if w.dtype == "f32":
        return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(device)
    return torch.from_numpy(a.view(np.int16)).to(device).view(torch.bfloat16)


@dataclass
class GpuInputs:
    w: Workload
    kv: object            # device tensor [rows, nb, BE] or PinnedBuffer
    kv_ptr: object        # tensor (resident) or device alias int (offload)
    nb: int
    e_tok: torch.Tensor   # [rows, n_max] float32
    q: torch.Tensor       # [T, batch, n_q_heads, D]
    k_new: torch.Tensor = None  # [T, rows, D]: token context + t of every row (prefix_only)
    v_new: torch.Tensor = None


def _row_blocks(w: Workload, layer: int, r: int, nb: int, n_tokens: int | None = None) -> np.ndarray:
    """Block-unit KV of one row; with n_tokens, only its first n_tokens tokens."""
    b, g = divmod(r, w.n_kv_heads)
    slab = layer % w.kv_slabs
    K = storage(synth.keys_row(w, slab, b, g), w)
    V = storage(synth.values_row(w, slab, b, g), w)
    if n_tokens is not None:
        K, V = K[:n_tokens], V[:n_tokens]
    return pack_blocks(K, V, nb)


def upload(w: Workload, layer: int = 0, ov: Overrides | None = None, steps: int | None = None,
           device="cuda", workers: int = 16, prefix_only: bool = False) -> GpuInputs:
    """Seeded inputs on the GPU. prefix_only: the KV holds the context tokens
    only, and each step's token comes as k_new[t] / v_new[t] [rows][D]."""
    T = w.steps if steps is None else steps
    nb = w.nb_max
    BE = 2 * 64 * w.head_dim
    rows = w.rows
    if w.offload:
        elem = 4 if w.dtype == "f32" else 2
        buf = PinnedBuffer(rows * nb * BE * elem)
        view = buf.array(np.float32 if w.dtype == "f32" else np.uint16, (rows, nb, BE))

        def fill(r):
            view[r] = _row_blocks(w, layer, r, nb, w.context if prefix_only else None)
        synth.parallel_map(fill, range(rows), workers)
        kv, kv_ptr = buf, buf.dev
    else:
        tdt = torch.float32 if w.dtype == "f32" else torch.bfloat16
        kv = torch.empty(rows, nb, BE, dtype=tdt, device=device)
        chunk = max(1, workers)
        for r0 in range(0, rows, chunk):
            rr = list(range(r0, min(rows, r0 + chunk)))
            parts = synth.parallel_map(
                lambda r: _row_blocks(w, layer, r, nb, w.context if prefix_only else None), rr,
                workers)
            for r, p in zip(rr, parts):
                kv[r].copy_(to_device(p, w, device))
        kv_ptr = kv
    e = np.zeros((rows, nb * 64), np.float32)   # rows padded to whole blocks
    e[:, :w.n_max] = np.stack(synth.parallel_map(
        lambda r: synth.evict_row(w, layer, *divmod(r, w.n_kv_heads), ov), range(rows), workers))
    e_tok = torch.from_numpy(e).to(device)
    qs = synth.parallel_map(lambda t: storage(synth.queries_step(w, layer, t, ov), w), range(T),
                            workers)
    q = to_device(np.stack(qs), w, device)
    inp = GpuInputs(w, kv, kv_ptr, nb, e_tok, q)
    if prefix_only:
        def new_tokens(r):
            b, g = divmod(r, w.n_kv_heads)
            slab = layer % w.kv_slabs
            lo, hi = w.context, w.context + T
            return (storage(synth.keys_row(w, slab, b, g)[lo:hi], w),
                    storage(synth.values_row(w, slab, b, g)[lo:hi], w))
        kvn = synth.parallel_map(new_tokens, range(rows), workers)
        inp.k_new = to_device(np.ascontiguousarray(np.stack([k for k, _ in kvn], 1)), w, device)
        inp.v_new = to_device(np.ascontiguousarray(np.stack([v for _, v in kvn], 1)), w, device)
    return inp


def upload_slabs(w: Workload, workers: int = 16) -> list:
    """Pinned host KV of every slab: [(PinnedBuffer, device alias)]."""
    nb = w.nb_max
    BE = 2 * 64 * w.head_dim
    out = []
    for slab in range(w.kv_slabs):
        buf = PinnedBuffer(w.rows * nb * BE * 2)
        view = buf.array(np.uint16, (w.rows, nb, BE))

        def fill(r, slab=slab, view=view):
            view[r] = _row_blocks(w, slab, r, nb)
        synth.parallel_map(fill, range(w.rows), workers)
        out.append((buf, buf.dev))
    return out


def upload_layer(w: Workload, layer: int, kv, ov: Overrides | None, steps: int,
                 device="cuda", workers: int = 16) -> GpuInputs:
    """Eviction scores and queries of one layer; KV from an existing slab."""
    nb = w.nb_max
    e = np.zeros((w.rows, nb * 64), np.float32)
    e[:, :w.n_max] = np.stack(synth.parallel_map(
        lambda r: synth.evict_row(w, layer, *divmod(r, w.n_kv_heads), ov), range(w.rows), workers))
    e_tok = torch.from_numpy(e).to(device)
    qs = synth.parallel_map(lambda t: storage(synth.queries_step(w, layer, t, ov), w), range(steps),
                            workers)
    q = to_device(np.stack(qs), w, device)
    return GpuInputs(w, kv[0], kv[1], nb, e_tok, q)


def make_layer(w: Workload, inp: GpuInputs, decode_kernel=L.NOSA_DECODE_AUTO,
               fuse_select_swap=True, overlap=False, fuse_score=None,
               device_append=False) -> DecodeLayer:
    return DecodeLayer(batch=w.batch, n_q_heads=w.n_q_heads, n_kv_heads=w.n_kv_heads,
                       head_dim=w.head_dim, k_e=w.k_e, k_q=w.k_q, max_blocks=inp.nb,
                       dtype=nosa_dtype(w), kv=inp.kv_ptr, kv_row_blocks=inp.nb,
                       e_tok=inp.e_tok, offload=w.offload, decode_kernel=decode_kernel,
                       fuse_select_swap=fuse_select_swap, fuse_score=fuse_score,
                       overlap=overlap, device_append=device_append,
                       pooled_dtype=pooled_dtype(w))


def bits_to_list(words: np.ndarray) -> list:
    u = words.astype(np.uint32)
    return [i * 32 + j for i, x in enumerate(u) for j in range(32) if (int(x) >> j) & 1]


def snapshot(layer: DecodeLayer, w: Workload) -> dict:
    """Copy the per-step results of every row to host memory."""
    torch.cuda.synchronize()
    return {
        "sel": layer.sel.cpu().numpy().copy(),
        "n_sel": layer.n_sel.cpu().numpy().copy(),
        "ge_bits": layer.ge_bits.cpu().numpy().copy(),
        "ev_bits": layer.ev_bits.cpu().numpy().copy(),
        "sel_bits": layer.sel_bits.cpu().numpy().copy(),
        "s_q": layer.s_q.cpu().numpy().copy(),
        "e_blk": layer.e_blk.cpu().numpy().copy(),
        "fetch_block": layer.fetch_block.cpu().numpy().copy(),
        "fetch_slot": layer.fetch_slot.cpu().numpy().copy(),
        "n_fetch": layer.n_fetch.cpu().numpy().copy(),
        "slot_block": layer.slot_block.cpu().numpy().copy(),
        "counters": layer.counters.cpu().numpy().copy(),
        "s_q_certified": bool(getattr(layer, "scores_certified", False)),
        "out": layer.out.float().cpu().numpy().astype(np.float64),
    }


def run(w: Workload, inp: GpuInputs, steps, layer: DecodeLayer | None = None,
        collect=None, swap=True, decode_kernel=L.NOSA_DECODE_AUTO, fuse_select_swap=True,
        overlap=False, fuse_score=None):
    """Run steps 0..max(steps) in order; snapshot the steps listed in ``collect``.
    Inputs uploaded with prefix_only feed each step's token through the
    device-side append."""
    append = inp.k_new is not None
    layer = layer or make_layer(w, inp, decode_kernel, fuse_select_swap, overlap, fuse_score,
                                device_append=append)
    T = max(steps) + 1
    collect = set(steps if collect is None else collect)
    layer.start(w.n_tokens(0))
    res = {}
    for t in range(T):
        if append:
            layer.step(inp.q[t], w.n_tokens(t), swap=swap, k_new=inp.k_new[t], v_new=inp.v_new[t])
        else:
            layer.step(inp.q[t], w.n_tokens(t), swap=swap)
        if t in collect:
            res[t] = snapshot(layer, w)
    torch.cuda.synchronize()
    return layer, res
