"""Host-side sequencing of the NOSA decode path for one layer.

Every stage of a step runs in the library's kernels; this module allocates
the device buffers (through torch) and issues the C-ABI calls in order, all
on one stream with no host synchronisation inside a step.

Per decode step (NOSA technical summary, Methodology):
  pool      a block that just became complete joins the candidates: its
            sub-block mean keys and pooled eviction score are computed once
  score     query-aware pooled score of every candidate block
  select    Gamma_e (eviction budget, strict eviction) and Gamma_q (top k_q)
  swap      set difference against the blocks cached in HBM
  fetch     (offloaded KV) copy of the missing blocks from pinned host memory
  decode    attention over the selection plus the newest block, eviction
            score as an additive logit
"""
from __future__ import annotations

import math

import numpy as np
import torch

from . import _lib as L

BLOCK = 64
SUB_BLOCK = 16


# Token held at each position of a stored V^T row: inside each half of 32,
# positions 8j..8j+7 hold tokens 4j..4j+3 and 16+4j..16+4j+3.
VT_TOKEN_AT = np.array([32 * (p // 32) + 16 * ((p % 8) // 4) + 4 * ((p % 32) // 8) + p % 4
                        for p in range(BLOCK)])
VT_POS_OF = np.argsort(VT_TOKEN_AT)


def _geometry(D: int, itemsize: int):
    e = 16 // itemsize  # elements per 16-byte vector
    if D % (4 * e) or D % 16:
        raise ValueError("head_dim must be a multiple of 16 and of 4 vectors")
    return e, D // (4 * e), BLOCK // (4 * e), D // 16


def pack_blocks(K: np.ndarray, V: np.ndarray, n_blocks: int) -> np.ndarray:
    """Block-unit layout of one row (include/nosa.h): [n_blocks, 2*64*D] with,
    per block, the K tile and then the V^T tile (positions in the VT_TOKEN_AT
    token order), both as 1 KiB fragments of 16-byte vectors: K fragment
    t*NS + s, vector col + 16 grp holds token 16t + col, dimensions
    (4s + grp)E .. + E-1; V^T fragment dt*NP + s, vector col + 16 grp holds
    dimension 16dt + col, positions (4s + grp)E .. + E-1 (E elements per
    vector, NS = D/4E, NP = 64/4E). Tokens beyond the input are zero. Works
    on float32 or bfloat16-bit (uint16) arrays."""
    n, D = K.shape
    pad = n_blocks * BLOCK - n
    if pad < 0:
        raise ValueError("more tokens than blocks")
    if pad:
        K = np.concatenate([K, np.zeros((pad, D), K.dtype)])
        V = np.concatenate([V, np.zeros((pad, D), V.dtype)])
    e, ns, npos, dt = _geometry(D, K.dtype.itemsize)
    # K[tok = 16t + col][d = (4s + grp)e + x] -> (t, s, grp, col, x)
    Kf = K.reshape(n_blocks, 4, 16, ns, 4, e).transpose(0, 1, 3, 4, 2, 5)
    # V^T[d = 16dt + col][pos = (4s + grp)e + x] -> (dt, s, grp, col, x)
    Vp = V.reshape(n_blocks, BLOCK, D)[:, VT_TOKEN_AT, :]
    Vf = Vp.reshape(n_blocks, npos, 4, e, dt, 16).transpose(0, 4, 1, 2, 5, 3)
    return np.ascontiguousarray(np.concatenate(
        [Kf.reshape(n_blocks, BLOCK * D), Vf.reshape(n_blocks, BLOCK * D)], axis=1))


def unpack_blocks(packed: np.ndarray, D: int):
    """The inverse of pack_blocks: (K, V), each [n_blocks * 64, D], from
    packed [n_blocks, 2*64*D]."""
    packed = np.asarray(packed)
    n = packed.shape[0]
    e, ns, npos, dt = _geometry(D, packed.dtype.itemsize)
    K = packed[:, :BLOCK * D].reshape(n, 4, ns, 4, 16, e).transpose(0, 1, 4, 2, 3, 5)
    Vp = packed[:, BLOCK * D:].reshape(n, dt, npos, 4, 16, e).transpose(0, 2, 3, 5, 1, 4)
    V = Vp.reshape(n, BLOCK, D)[:, VT_POS_OF, :]
    return K.reshape(n * BLOCK, D), V.reshape(n * BLOCK, D)


def block_offsets(D: int, itemsize: int):
    """Element offsets inside one packed block of K[tok][d] and of V[tok][d]:
    two int64 arrays [64, D] (the formulas of include/nosa.h)."""
    e, ns, npos, _ = _geometry(D, itemsize)
    tok = np.arange(BLOCK)[:, None]
    d = np.arange(D)[None, :]
    k_off = (((tok // 16) * ns + d // (4 * e)) * 64 + tok % 16 + 16 * ((d // e) % 4)) * e + d % e
    p = VT_POS_OF[tok]
    v_off = BLOCK * D + (((d // 16) * npos + p // (4 * e)) * 64 + d % 16
                         + 16 * ((p // e) % 4)) * e + p % e
    return k_off.astype(np.int64), v_off.astype(np.int64)


def torch_dtype(dtype: int):
    return torch.float32 if dtype == L.NOSA_F32 else torch.bfloat16


class DecodeLayer:
    """Device state and call sequence of one layer.

    kv:     resident mode: device tensor [rows, kv_row_blocks, 2*64*D];
            offload mode: integer device alias of pinned host memory with the
            same layout.
    e_tok:  device float32 tensor [rows, e_row_stride].
    """

    def __init__(self, *, batch, n_q_heads, n_kv_heads, head_dim, k_e, k_q, max_blocks, dtype,
                 kv, kv_row_blocks, e_tok, offload=False, decode_kernel=L.NOSA_DECODE_AUTO,
                 scale=0.0, device="cuda", fuse_select_swap=True, fuse_score=None,
                 overlap=False, device_append=False, evict_head=None, pooled_dtype=L.NOSA_F32):
        self.shape = L.make_shape(batch, n_q_heads, n_kv_heads, head_dim, k_e, k_q, max_blocks,
                                  dtype, decode_kernel=decode_kernel, scale=scale,
                                  pooled_dtype=pooled_dtype)
        self.pooled_dtype = pooled_dtype
        self.rows = batch * n_kv_heads
        self.k = k_e + k_q
        self.D = head_dim
        self.G = n_q_heads // n_kv_heads
        self.max_blocks = max_blocks
        self.W = (max_blocks + 31) // 32
        self.dtype = dtype
        self.offload = offload
        self.kv = kv
        self.kv_row_blocks = kv_row_blocks
        self.e_tok = e_tok
        self.e_stride = e_tok.shape[1]
        self.block_elems = 2 * BLOCK * head_dim
        self.elem_bytes = 4 if dtype == L.NOSA_F32 else 2
        dev = torch.device(device)
        R, k, W = self.rows, self.k, self.W
        f32, i32 = torch.float32, torch.int32
        # pooled keys in the pooled dtype (float32 unless bfloat16 is asked
        # for): quads of 4 blocks (16 sub-blocks), each [D / V][16][V] with V
        # dimensions per 16-byte vector
        # (with bf16 keys and float32 pooled keys the buffer goes on with the
        # bf16 copy and the radii of certified scoring; self.kbar views the
        # float32 means at its start)
        V = 16 // (4 if pooled_dtype == L.NOSA_F32 else 2)
        kdt = torch_dtype(pooled_dtype)
        kshape = (R, (max_blocks + 3) // 4, head_dim // V, 16, V)
        n_kbar = int(np.prod(kshape))
        esz = 4 if pooled_dtype == L.NOSA_F32 else 2
        self.kbar_buf = torch.zeros(-(-L.nosa_kbar_bytes(self.shape) // esz), dtype=kdt,
                                    device=dev)
        self.kbar = self.kbar_buf[:n_kbar].view(kshape)
        # scores in s_q come from the bf16 copy on the nosa_score_select path
        self.scores_certified = dtype == L.NOSA_BF16 and pooled_dtype == L.NOSA_F32
        self.e_blk = torch.zeros(R, max_blocks, dtype=f32, device=dev)
        self.s_q = torch.zeros(R, max_blocks, dtype=f32, device=dev)
        self.ge_bits = torch.zeros(R, W, dtype=i32, device=dev)
        self.ev_bits = torch.zeros(R, W, dtype=i32, device=dev)
        self.sel_bits = torch.zeros(R, W, dtype=i32, device=dev)
        self.sel = torch.full((R, k), -1, dtype=i32, device=dev)
        self.n_sel = torch.zeros(R, dtype=i32, device=dev)
        self.slot_block = torch.full((R, k), -1, dtype=i32, device=dev)
        self.block_slot = torch.full((R, max_blocks), -1, dtype=i32, device=dev)
        self.fetch_block = torch.full((R, k), -1, dtype=i32, device=dev)
        self.fetch_slot = torch.full((R, k), -1, dtype=i32, device=dev)
        self.n_fetch = torch.zeros(R, dtype=i32, device=dev)
        self.counters = torch.zeros(R, 2, dtype=torch.int64, device=dev)
        self.ws_bytes = L.nosa_decode_workspace_size(self.shape)
        self.chunks_all = L.nosa_decode_chunks(self.shape, self.k, 1)
        self.ws = torch.empty(self.ws_bytes // 4 + 4, dtype=f32, device=dev)
        self.out = torch.empty(batch, n_q_heads, head_dim, dtype=torch_dtype(dtype), device=dev)
        if offload:
            self.cache = torch.empty(R, k, self.block_elems, dtype=torch_dtype(dtype), device=dev)
            self.cur = torch.empty(R, 1, self.block_elems, dtype=torch_dtype(dtype), device=dev)
            # one-entry fetch list that loads the newest block into `cur`
            self.cur_fb = torch.zeros(R, k, dtype=i32, device=dev)
            self.cur_fs = torch.zeros(R, k, dtype=i32, device=dev)
            self.cur_nf = torch.ones(R, dtype=i32, device=dev)
        self.fuse_select_swap = fuse_select_swap
        # scoring and selection through nosa_score_select (one launch with a
        # workgroup per row, or a split scoring grid and the selection when
        # the rows are too few to fill the chip); the default for bf16
        if fuse_score is None:
            fuse_score = dtype == L.NOSA_BF16
        self.fuse_score = fuse_score and fuse_select_swap
        self.scores_certified = self.scores_certified and self.fuse_score
        # Overlap (KV in HBM): on a step that completes no block, attention over
        # the eviction set (unchanged since the previous step) and the newest
        # block runs on a side stream while the scores and the selection run on
        # the caller's stream; the query-aware part follows the selection and a
        # combine merges both.
        self.overlap = overlap and not offload
        # Overlap (offloaded KV): the rows go in two halves of the batch; the
        # second half's fetch runs on a side stream while the first half's
        # attention (over its cache and newest block) and merge run on the
        # caller's stream, then the second half's attention follows its fetch.
        self.overlap_fetch = overlap and offload
        if self.overlap_fetch:
            if batch % 2:
                raise ValueError("the offload overlap splits the batch in two halves")
            self.half_shape = L.make_shape(batch // 2, n_q_heads, n_kv_heads, head_dim, k_e, k_q,
                                           max_blocks, dtype, decode_kernel=decode_kernel,
                                           scale=scale, pooled_dtype=pooled_dtype)
            self.ws_half_bytes = L.nosa_decode_workspace_size(self.half_shape)
            self.ws_half = [torch.empty(self.ws_half_bytes // 4 + 4, dtype=f32, device=dev)
                            for _ in range(2)]
            self.chunks_half = L.nosa_decode_chunks(self.half_shape, self.k, 1)
            self.side = torch.cuda.Stream(device=dev)
            self.fetch_a_done = torch.cuda.Event()
            self.fetch_b_done = torch.cuda.Event()
        if self.overlap:
            ke, kq = max(k_e, 1), max(k_q, 1)
            self.side = torch.cuda.Stream(device=dev)
            self.ge_list = [torch.full((R, ke), -1, dtype=i32, device=dev) for _ in range(2)]
            self.n_ge = [torch.zeros(R, dtype=i32, device=dev) for _ in range(2)]
            self.gq_list = torch.full((R, kq), -1, dtype=i32, device=dev)
            self.n_gq = torch.zeros(R, dtype=i32, device=dev)
            self.chunks_e = L.nosa_decode_chunks(self.shape, k_e, 1)
            self.chunks_q = L.nosa_decode_chunks(self.shape, k_q, 0)
            self.step_done = torch.cuda.Event()
            self.side_done = torch.cuda.Event()
            self.parity = 0
        # device_append: each step's token arrives as k_new / v_new [rows][D]
        # on the GPU and is written into the newest block (the newest-block
        # buffer when offloaded); with offloaded KV a completed block is then
        # written back to host memory, so the host KV needs only the prefill
        # evict_head = (w [n_kv_heads, hidden] KV dtype, b float32 [n_kv_heads]
        # or None): steps take the token's fused projection output and hidden
        # state instead (qkv, x), and one launch splits q / k / v, writes k and
        # v into the newest block, runs the eviction head into e_tok and pools
        # a block its token completes
        self.evict_head = evict_head
        if evict_head is not None:
            if overlap:
                raise ValueError("evict_head is not combined with overlap")
            device_append = True
            self.q_buf = torch.empty(batch, n_q_heads, head_dim, dtype=torch_dtype(dtype),
                                     device=dev)
        self.device_append = device_append
        if device_append and offload:
            # a one-entry fetch list per row ([rows][k] like every fetch list;
            # column 0 used): source block 0 of the buffer, destination block
            self.wb_fb = torch.zeros(R, k, dtype=i32, device=dev)
            self.wb_fs = torch.zeros(R, k, dtype=i32, device=dev)
            self.wb_nf = torch.ones(R, dtype=i32, device=dev)
        self.n_cand_prev = -1
        self.n_tokens = 0
        # optional callable(stage_name, fn, *args): runs fn(*args); a caller
        # may wrap the launch (for example with timing events)
        self.stage_hook = None

    # -- helpers -------------------------------------------------------------
    def _run(self, name, fn, *args):
        """Issue one ABI call; its last argument is the stream it runs on."""
        if self.stage_hook is None:
            fn(*args)
        else:
            self.stage_hook(name, fn, *args)

    def _kv_ptr(self, block: int) -> int:
        base = self.kv if isinstance(self.kv, int) else self.kv.data_ptr()
        return base + block * self.block_elems * self.elem_bytes

    @staticmethod
    def _fill(t: torch.Tensor, value: int, stream=None):
        """t.fill_(value), ordered on `stream` (a torch stream or None)."""
        if isinstance(stream, torch.cuda.Stream):
            with torch.cuda.stream(stream):
                t.fill_(value)
        else:
            t.fill_(value)

    def _load_cur(self, block: int, stream=None):
        self._fill(self.cur_fb[:, 0], block, stream)
        self._run("fetch_newest", L.nosa_fetch_blocks, self.shape, self.kv, self.kv_row_blocks,
                  self.cur_fb, self.cur_fs, self.cur_nf, 1, self.cur, 1, stream)

    # -- call sequence -------------------------------------------------------
    def start(self, n_tokens: int, stream=None):
        """Prefill stand-in: pool the complete blocks of the first n_tokens - 1
        tokens (the candidates of the step that brings n_tokens) and, with
        offloaded KV, load the newest block."""
        c0 = (n_tokens - 1) // BLOCK
        if c0 > 0:
            L.nosa_pool_blocks(self.shape, self.kv, self.kv_row_blocks, 0, self.e_tok,
                               self.e_stride, 0, c0, self.kbar, self.e_blk, stream)
        if self.offload:
            self._load_cur(c0, stream)
        self.n_cand_prev = -1
        self.pooled = c0

    def prefill(self, q_all: torch.Tensor, n_tokens: int, stream=None):
        """Causal prefill of the first n_tokens tokens of the resident KV with
        the selection per query block: q_all [batch, n_tokens, Hq, D] (bf16).
        Returns (out [batch, n_tokens, Hq, D], sel [n_qb, rows, k], n_sel
        [n_qb, rows]). Leaves K̄ and e_blk pooled for the complete blocks
        before the last query block; a decode run starts with start()."""
        if self.offload:
            raise ValueError("prefill reads a resident KV")
        nqb = -(-n_tokens // BLOCK)
        dev = self.kbar.device
        if nqb > 1:
            L.nosa_pool_blocks(self.shape, self.kv, self.kv_row_blocks, 0, self.e_tok,
                               self.e_stride, 0, nqb - 1, self.kbar, self.e_blk, stream)
        qbar = torch.empty(nqb, *q_all.shape[:1], *q_all.shape[2:],
                           dtype=torch_dtype(self.pooled_dtype), device=dev)
        self._run("pool_queries", L.nosa_prefill_pool_queries, self.shape, q_all, n_tokens, qbar,
                  stream)
        sel = torch.empty(nqb, self.rows, self.k, dtype=torch.int32, device=dev)
        n_sel = torch.empty(nqb, self.rows, dtype=torch.int32, device=dev)
        self._run("prefill_select", L.nosa_prefill_select, self.shape, qbar, self.kbar,
                  self.e_blk, n_tokens, sel, n_sel, stream)
        out = torch.empty_like(q_all)
        self._run("prefill_attention", L.nosa_prefill_attention, self.shape, q_all, n_tokens,
                  self.kv, self.kv_row_blocks, self.e_tok, self.e_stride, sel, n_sel, out, stream)
        self.n_cand_prev = -1
        return out, sel, n_sel

    def _write_back(self, block: int, stream=None):
        """Newest-block buffer -> host KV block `block` (offloaded KV)."""
        self._fill(self.wb_fs[:, 0], block, stream)
        self._run("write_back", L.nosa_fetch_blocks, self.shape, self.cur, 1, self.wb_fb,
                  self.wb_fs, self.wb_nf, 1, self.kv, self.kv_row_blocks, stream)

    def _ingest(self, qkv, x, n_tokens: int, stream=None):
        tok = n_tokens - 1
        c = tok // BLOCK
        w, b = self.evict_head
        dst, rb, blk = (self.cur, 1, 0) if self.offload else (self.kv, self.kv_row_blocks, c)
        self._run("ingest", L.nosa_ingest_tokens, self.shape, qkv, x, w, b, w.shape[1], n_tokens,
                  self.q_buf, dst, rb, blk, self.e_tok, self.e_stride, self.kbar, self.e_blk,
                  stream)
        if tok % BLOCK == BLOCK - 1:
            # the launch pooled block c; it is a candidate from the next step on
            self.pooled = c + 1
            if self.offload:
                self._write_back(c, stream)

    def step(self, q: torch.Tensor, n_tokens: int, stream=None, swap: bool = True,
             k_new=None, v_new=None, qkv=None, x=None) -> torch.Tensor:
        """One decode step at n_tokens tokens (the newest appended by this step;
        with device_append, k_new / v_new [rows][D] carry it; with an eviction
        head, qkv [batch][(Hq + 2 Hkv) D] and x [batch][hidden] do, and q is
        taken from qkv)."""
        c = (n_tokens - 1) // BLOCK
        if self.evict_head is not None:
            if qkv is None or x is None:
                raise ValueError("a layer with an eviction head needs the step's qkv and x")
            self._ingest(qkv, x, n_tokens, stream)
            q = self.q_buf
        elif self.device_append and (k_new is None or v_new is None):
            raise ValueError("device_append needs the step's k_new and v_new")
        if c > self.pooled:
            if self.offload:
                assert c == self.pooled + 1, "offloaded KV grows by one block per step"
                # the completed block is the newest-block buffer's content
                self._run("pool", L.nosa_pool_blocks, self.shape, self.cur, 1, 0, self.e_tok,
                          self.e_stride, self.pooled, c, self.kbar, self.e_blk, stream)
                if self.device_append:
                    # write it back to host block c - 1; the buffer starts block c
                    self._write_back(c - 1, stream)
                else:
                    self._load_cur(c, stream)
            else:
                self._run("pool", L.nosa_pool_blocks, self.shape, self.kv, self.kv_row_blocks,
                          self.pooled, self.e_tok, self.e_stride, self.pooled, c, self.kbar,
                          self.e_blk, stream)
            self.pooled = c
        if self.device_append and self.evict_head is None:
            pos = (n_tokens - 1) % BLOCK
            if self.offload:
                self._run("append", L.nosa_append_tokens, self.shape, k_new, v_new, pos, self.cur,
                          1, 0, stream)
            else:
                self._run("append", L.nosa_append_tokens, self.shape, k_new, v_new, pos, self.kv,
                          self.kv_row_blocks, c, stream)
        st = L.make_step(n_tokens, self.n_cand_prev)
        if self.overlap:
            self._step_overlap(q, n_tokens, c, st, stream, swap)
            self.n_cand_prev = c
            self.n_tokens = n_tokens
            return self.out
        if self.fuse_score:
            cache = (self.slot_block, self.block_slot, self.fetch_block, self.fetch_slot,
                     self.n_fetch, self.counters) if (swap or self.offload) else (None,) * 6
            self._run("score_select", L.nosa_score_select, self.shape, q, self.kbar, self.e_blk,
                      st, self.s_q, self.ge_bits, self.ev_bits, self.sel, self.n_sel,
                      self.sel_bits, *cache, stream)
        else:
            self._run("score", L.nosa_score_blocks, self.shape, q, self.kbar, st, self.s_q, stream)
            if (swap or self.offload) and self.fuse_select_swap:
                self._run("select", L.nosa_select_swap, self.shape, self.s_q, self.e_blk, st,
                          self.ge_bits, self.ev_bits, self.sel, self.n_sel, self.sel_bits,
                          self.slot_block, self.block_slot, self.fetch_block, self.fetch_slot,
                          self.n_fetch, self.counters, stream)
            else:
                self._run("select", L.nosa_select, self.shape, self.s_q, self.e_blk, st,
                          self.ge_bits, self.ev_bits, self.sel, self.n_sel, self.sel_bits, stream)
                if swap or self.offload:
                    self._run("swap", L.nosa_swap_diff, self.shape, self.sel, self.n_sel,
                              self.sel_bits, self.slot_block, self.block_slot, self.fetch_block,
                              self.fetch_slot, self.n_fetch, self.counters, stream)
        if self.overlap_fetch:
            self._offload_halves(q, st, stream)
            self.n_cand_prev = c
            self.n_tokens = n_tokens
            return self.out
        if self.offload:
            self._run("fetch", L.nosa_fetch_blocks, self.shape, self.kv, self.kv_row_blocks,
                      self.fetch_block, self.fetch_slot, self.n_fetch, self.k, self.cache, self.k,
                      stream)
            self._run("decode", L.nosa_decode_attend, self.shape, q, self.cache, self.k,
                      L.NOSA_KV_CACHE, self.slot_block, None, self.k, self.k, 1, self.cur, 1, st,
                      self.e_tok, self.e_stride, self.ws, self.ws_bytes, self.out, None, None,
                      stream)
        else:
            self._run("decode", L.nosa_decode_attend, self.shape, q, self.kv, self.kv_row_blocks,
                      L.NOSA_KV_FULL, self.sel, self.n_sel, self.k, self.k, 1, self._kv_ptr(c),
                      self.kv_row_blocks, st, self.e_tok, self.e_stride, self.ws, self.ws_bytes,
                      self.out, None, None, stream)
        self.n_cand_prev = c
        self.n_tokens = n_tokens
        return self.out

    def _offload_halves(self, q, st, stream):
        """Fetch, attention and merge of an offloaded step in two batch halves,
        the second half's fetch overlapping the first half's attention."""
        main = stream if stream is not None else torch.cuda.current_stream()
        Rh, Bh, k, sh = self.rows // 2, q.shape[0] // 2, self.k, self.half_shape
        base = self.kv if isinstance(self.kv, int) else self.kv.data_ptr()
        kv_b = base + Rh * self.kv_row_blocks * self.block_elems * self.elem_bytes
        halves = ((slice(0, Rh), slice(0, Bh), base), (slice(Rh, 2 * Rh), slice(Bh, 2 * Bh), kv_b))

        def fetch(h, on):
            rs, _, src = halves[h]
            self._run("fetch", L.nosa_fetch_blocks, sh, src, self.kv_row_blocks,
                      self.fetch_block[rs], self.fetch_slot[rs], self.n_fetch[rs], k,
                      self.cache[rs], k, on)

        def attend(h):
            rs, bs, _ = halves[h]
            self._run("decode", L.nosa_decode_partial, sh, q[bs], self.cache[rs], k,
                      L.NOSA_KV_CACHE, self.slot_block[rs], None, k, k, 1, self.cur[rs], 1, st,
                      self.e_tok[rs], self.e_stride, self.ws_half[h], self.ws_half_bytes, 0, main)
            self._run("combine", L.nosa_decode_combine, sh, self.chunks_half, self.out[bs],
                      self.ws_half[h], self.ws_half_bytes, main)

        fetch(0, main)
        self.fetch_a_done.record(main)
        self.side.wait_event(self.fetch_a_done)
        fetch(1, self.side)
        self.fetch_b_done.record(self.side)
        attend(0)
        main.wait_event(self.fetch_b_done)
        attend(1)

    # -- checkpoint / resume ---------------------------------------------------
    # The decode state a step leaves behind, all of it caller-owned device
    # memory plus three host counters: pooled keys and eviction scores, the
    # eviction / selection bitmaps (strict eviction is a property of this
    # state), the last selection, the cache's slot tables and, offloaded, the
    # cache and the newest-block buffer themselves.
    STATE = ("kbar_buf", "e_blk", "ge_bits", "ev_bits", "sel_bits", "sel", "n_sel", "slot_block",
             "block_slot", "fetch_block", "fetch_slot", "n_fetch", "counters")

    def state_dict(self) -> dict:
        """A copy of the layer's decode state (device tensors cloned in stream
        order on the current stream; host counters as ints). A layer built
        with the same arguments continues from it with load_state_dict."""
        d = {n: getattr(self, n).clone() for n in self.STATE}
        if self.offload:
            d["cache"] = self.cache.clone()
            d["cur"] = self.cur.clone()
        d["host"] = {"n_cand_prev": self.n_cand_prev, "pooled": getattr(self, "pooled", 0),
                     "n_tokens": self.n_tokens}
        return d

    def load_state_dict(self, d: dict):
        """Continue from a state_dict() of a layer with the same shape."""
        names = self.STATE + (("cache", "cur") if self.offload else ())
        for n in names:
            dst = getattr(self, n)
            if tuple(d[n].shape) != tuple(dst.shape) or d[n].dtype != dst.dtype:
                raise ValueError(f"state {n}: shape or dtype differs from this layer's")
            dst.copy_(d[n])
        h = d["host"]
        self.n_cand_prev, self.pooled, self.n_tokens = h["n_cand_prev"], h["pooled"], h["n_tokens"]

    def reset(self):
        """Forget the decode state (selections, eviction state, cache tables
        and counters); start() then begins a new decode."""
        for t in (self.ge_bits, self.ev_bits, self.sel_bits, self.n_sel, self.n_fetch,
                  self.counters):
            t.zero_()
        for t in (self.sel, self.slot_block, self.block_slot, self.fetch_block, self.fetch_slot):
            t.fill_(-1)
        self.n_cand_prev = -1
        self.n_tokens = 0

    # -- steps replayed from a captured graph ----------------------------------
    def graph_capture(self, n_tokens: int, q_buf: torch.Tensor, k_new_buf=None, v_new_buf=None,
                      swap: bool = True):
        """Capture one decode step of the resident KV into a hipGraph (through
        torch.cuda.CUDAGraph). Its calls read the step record from device
        memory (self.step_dev: n_tokens, n_cand_prev), and the step's last
        call moves the record on, so each replay is the next step. The step
        reads q from q_buf [batch][Hq][D] and, with device_append, the newest
        token from k_new_buf / v_new_buf [rows][D]: fill them before each
        replay. n_tokens is the first replayed step's token count; the layer
        continues from its current state (start() or earlier steps)."""
        if self.offload or self.overlap or self.evict_head is not None:
            raise ValueError("graph-replayed steps cover the resident KV path")
        if self.device_append and (k_new_buf is None or v_new_buf is None):
            raise ValueError("device_append needs the step's k_new_buf and v_new_buf")
        dev = self.kbar.device
        self.step_dev = torch.tensor([n_tokens, self.n_cand_prev], dtype=torch.int32, device=dev)
        # load every kernel of the step once outside the capture (on a scratch
        # record the advance kernel may move)
        scratch = torch.tensor([n_tokens, self.n_cand_prev], dtype=torch.int32, device=dev)
        L.nosa_step_advance(self.shape, scratch, None)
        torch.cuda.synchronize()
        cache = (self.slot_block, self.block_slot, self.fetch_block, self.fetch_slot,
                 self.n_fetch, self.counters) if swap else (None,) * 6
        rb = self.kv_row_blocks
        side = torch.cuda.Stream(device=dev)
        side.wait_stream(torch.cuda.current_stream())
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=side):
            if self.device_append:
                L.nosa_append_step(self.shape, k_new_buf, v_new_buf, self.kv, rb, self.step_dev)
            L.nosa_pool_step(self.shape, self.kv, rb, self.e_tok, self.e_stride, self.step_dev,
                             self.kbar, self.e_blk)
            L.nosa_score_select_step(self.shape, q_buf, self.kbar, self.e_blk, self.step_dev,
                                     self.s_q, self.ge_bits, self.ev_bits, self.sel, self.n_sel,
                                     self.sel_bits, *cache)
            L.nosa_decode_partial_step(self.shape, q_buf, self.kv, rb, L.NOSA_KV_FULL, self.sel,
                                       self.n_sel, self.k, self.k, 1, self.kv, rb, self.step_dev,
                                       self.e_tok, self.e_stride, self.ws, self.ws_bytes, 0)
            # the merge also moves the step record on (one kernel fewer per replay)
            L.nosa_decode_combine_step(self.shape, self.chunks_all, self.out, self.ws,
                                       self.ws_bytes, self.step_dev)
        torch.cuda.current_stream().wait_stream(side)
        return graph

    def graph_done(self, n_tokens_last: int):
        """Bring the host-side step state up to date after replays whose last
        step had n_tokens_last tokens (before eager steps follow)."""
        c = (n_tokens_last - 1) // BLOCK
        self.pooled = max(self.pooled, c)
        self.n_cand_prev = c
        self.n_tokens = n_tokens_last

    def _step_overlap(self, q, n_tokens, c, st, stream, swap):
        main = stream if stream is not None else torch.cuda.current_stream()
        cur, prev = self.parity, self.parity ^ 1
        k_e, k_q, rb = self.shape.k_e, self.shape.k_q, self.kv_row_blocks
        # Gamma_e changes only when candidates arrive (or at the first step)
        side = self.n_cand_prev >= 0 and c == self.n_cand_prev

        def part_e(lst, n_lst, on):
            self._run("decode_e", L.nosa_decode_partial, self.shape, q, self.kv, rb,
                      L.NOSA_KV_FULL, lst, n_lst, max(k_e, 1), k_e, 1, self._kv_ptr(c), rb, st,
                      self.e_tok, self.e_stride, self.ws, self.ws_bytes, 0, on)

        if side:
            # the previous step is complete: its lists are final, the workspace is free
            self.side.wait_event(self.step_done)
            part_e(self.ge_list[prev], self.n_ge[prev], self.side)
            self.side_done.record(self.side)
        self._run("score", L.nosa_score_blocks, self.shape, q, self.kbar, st, self.s_q, main)
        cache = (self.slot_block, self.block_slot, self.fetch_block, self.fetch_slot,
                 self.n_fetch, self.counters) if swap else (None,) * 6
        self._run("select", L.nosa_select_parts, self.shape, self.s_q, self.e_blk, st,
                  self.ge_bits, self.ev_bits, self.sel, self.n_sel, self.sel_bits,
                  self.ge_list[cur], self.n_ge[cur], self.gq_list, self.n_gq, *cache, main)
        if not side:
            part_e(self.ge_list[cur], self.n_ge[cur], main)
        if self.chunks_q:
            self._run("decode_q", L.nosa_decode_partial, self.shape, q, self.kv, rb,
                      L.NOSA_KV_FULL, self.gq_list, self.n_gq, max(k_q, 1), k_q, 0,
                      self._kv_ptr(c), rb, st, self.e_tok, self.e_stride, self.ws, self.ws_bytes,
                      self.chunks_e, main)
        if side:
            main.wait_event(self.side_done)
        self._run("combine", L.nosa_decode_combine, self.shape, self.chunks_e + self.chunks_q,
                  self.out, self.ws, self.ws_bytes, main)
        self.step_done.record(main)
        self.parity ^= 1


def default_scale(head_dim: int) -> float:
    return 1.0 / math.sqrt(head_dim)
