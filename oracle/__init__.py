"""NOSA decode-step oracle: plain CPU reference of what the hot path computes.

TEST INFRASTRUCTURE ONLY: the tests, ``__graft_entry__.smoke()`` and the
benchmark's CPU-baseline leg are the only users. The GPU path never imports
this package, and this package never imports the GPU path.

The arithmetic lives in ``nosa_oracle.c`` (plain single-threaded fp64 loops);
this module loads it with ctypes and adds the one stateful piece, the swap
list between consecutive steps, written with Python sets.

Pages followed: "NOSA: Native and Offloadable Sparse Attention" technical
summary, section Methodology: "1. Algorithm: NOSA" (dual selection, strict
eviction, locality guarantee, two-stage pooling, ED-DMA) and "2. System: NOSI"
(block-unit KV cache, set-difference for block swapping).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading
from dataclasses import dataclass, field

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "nosa_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
# a test that plants a mistake in a copy of the oracle's source points this
# at the copy's build, in a process of its own
_VARIANT = os.environ.get("NOSA_ORACLE_LIB")
_lock = threading.Lock()
_lib = None

_f = ctypes.POINTER(ctypes.c_float)
_d = ctypes.POINTER(ctypes.c_double)
_i = ctypes.POINTER(ctypes.c_int)
_u8 = ctypes.POINTER(ctypes.c_ubyte)


def compile_source(src: str, out: str) -> str:
    """gcc -O2, no fast-math, no FMA contraction, no threads."""
    tmp = out + ".tmp%d" % os.getpid()
    subprocess.check_call(["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-fno-fast-math",
                           "-ffp-contract=off", "-o", tmp, src, "-lm"])
    os.replace(tmp, out)
    return out


def build(force: bool = False) -> str:
    """Compile the oracle (see compile_source) unless it is up to date."""
    if _VARIANT:
        return _VARIANT
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        compile_source(_SRC, _LIB)
    return _LIB


def lib():
    global _lib
    with _lock:
        if _lib is None:
            L = ctypes.CDLL(build())
            L.oracle_round_bf16.argtypes = [ctypes.c_double]
            L.oracle_round_bf16.restype = ctypes.c_double
            L.oracle_pool_keys.argtypes = [_f, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                           ctypes.c_int, _d]
            L.oracle_pool_keys.restype = None
            L.oracle_evict_logit.argtypes = [_f, _f, ctypes.c_int, ctypes.c_double]
            L.oracle_evict_logit.restype = ctypes.c_double
            L.oracle_block_evict.argtypes = [_f, ctypes.c_int, ctypes.c_int, ctypes.c_int]
            L.oracle_block_evict.restype = ctypes.c_double
            L.oracle_block_score.argtypes = [_d, ctypes.c_int, ctypes.c_int, _f, ctypes.c_int,
                                             ctypes.c_int, ctypes.c_int, ctypes.c_double,
                                             ctypes.c_int]
            L.oracle_block_score.restype = ctypes.c_double
            L.oracle_topk.argtypes = [_d, _u8, ctypes.c_int, ctypes.c_int, _i]
            L.oracle_topk.restype = ctypes.c_int
            L.oracle_attend_tokens.argtypes = [_f, ctypes.c_int, ctypes.c_int, _f, _f, _f, _i,
                                               ctypes.c_int, ctypes.c_double, _d]
            L.oracle_attend_tokens.restype = None
            L.oracle_pool_queries.argtypes = [_f, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                              ctypes.c_int, _d]
            L.oracle_pool_queries.restype = None
            L.oracle_prefill_row.argtypes = [ctypes.c_int] * 7 + [ctypes.c_double, ctypes.c_int,
                                                                 _f, _f, _f, _f, _d, _i]
            L.oracle_prefill_row.restype = ctypes.c_int
            L.oracle_prefill_qblock.argtypes = [ctypes.c_int] * 7 + [ctypes.c_double, ctypes.c_int,
                                                                      _f, _f, _f, _f, ctypes.c_int,
                                                                      _d, _i]
            L.oracle_prefill_qblock.restype = None
            L.oracle_step_row.argtypes = [ctypes.c_int] * 7 + [ctypes.c_double, ctypes.c_int,
                                                              _f, _f, _f, _f,
                                                              _i, _i, _i, _i, _d, _d, _d]
            L.oracle_step_row.restype = ctypes.c_int
            _lib = L
    return _lib


def _pf(a: np.ndarray):
    assert a.dtype == np.float32 and a.flags.c_contiguous
    return a.ctypes.data_as(_f)


def _pd(a: np.ndarray):
    assert a.dtype == np.float64 and a.flags.c_contiguous
    return a.ctypes.data_as(_d)


def _pi(a: np.ndarray):
    assert a.dtype == np.int32 and a.flags.c_contiguous
    return a.ctypes.data_as(_i)


def _f32(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float32)


# ---------------------------------------------------------------------------
# single operations (for pins and for margin checks)
# ---------------------------------------------------------------------------

def round_bf16(x: float) -> float:
    """x rounded to the nearest bfloat16 value, ties to even."""
    return lib().oracle_round_bf16(float(x))


def pool_keys(K: np.ndarray, block: int, sub: int, j: int, pooled_bf16: bool = False) -> np.ndarray:
    """Sub-block means of block j's keys: [block // sub, D] fp64, exact
    (rounded to the nearest bfloat16 when pooled_bf16)."""
    K = _f32(K)
    D = K.shape[1]
    out = np.zeros((block // sub, D), dtype=np.float64)
    lib().oracle_pool_keys(_pf(K), D, block, sub, j, int(pooled_bf16), _pd(out))
    return out


def evict_logit(x: np.ndarray, w: np.ndarray, bias: float = 0.0) -> float:
    """Eviction-head logit of one token for one KV head: x . w + bias (double)."""
    x, w = _f32(x), _f32(w)
    assert x.shape == w.shape and x.ndim == 1
    return lib().oracle_evict_logit(_pf(x), _pf(w), x.shape[0], float(bias))


def qkv_split(qkv: np.ndarray, n_q_heads: int, n_kv_heads: int, head_dim: int):
    """Split one token's fused projection output [(Hq + 2 Hkv) * D] into
    q [Hq, D], k [Hkv, D], v [Hkv, D]: the query heads first, then the keys,
    then the values (reading of the pages' QKV split)."""
    D = head_dim
    a = np.asarray(qkv)
    assert a.shape == ((n_q_heads + 2 * n_kv_heads) * D,)
    q = a[:n_q_heads * D].reshape(n_q_heads, D)
    k = a[n_q_heads * D:(n_q_heads + n_kv_heads) * D].reshape(n_kv_heads, D)
    v = a[(n_q_heads + n_kv_heads) * D:].reshape(n_kv_heads, D)
    return q, k, v


def block_evict(e: np.ndarray, block: int, sub: int, j: int) -> float:
    """Pooled pre-exponential eviction score of block j."""
    e = _f32(e)
    return lib().oracle_block_evict(_pf(e), block, sub, j)


def block_score(q: np.ndarray, K: np.ndarray, block: int, sub: int, j: int, scale: float,
                pooled_bf16: bool = False) -> float:
    """Query-aware pooled score of block j for the query heads q [G, D]
    (taken as fp64: float32 queries exactly, pooled queries as they are)."""
    q, K = np.ascontiguousarray(q, dtype=np.float64), _f32(K)
    G, D = q.shape
    return lib().oracle_block_score(_pd(q), G, D, _pf(K), block, sub, j, scale, int(pooled_bf16))


def topk(x, k: int, allowed=None) -> list[int]:
    """Ascending indices of the k greatest entries of x (ties: lower index first)."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    n = x.shape[0]
    out = np.zeros(max(k, 1), dtype=np.int32)
    al = None
    if allowed is not None:
        al_arr = np.ascontiguousarray(allowed, dtype=np.uint8)
        al = al_arr.ctypes.data_as(_u8)
    cnt = lib().oracle_topk(_pd(x), al, n, k, _pi(out))
    return [int(v) for v in out[:cnt]]


def attend_tokens(q, K, V, e, tokens, scale: float) -> np.ndarray:
    """Softmax attention of q [G, D] over an explicit token list: [G, D] fp64."""
    q, K, V = _f32(q), _f32(K), _f32(V)
    G, D = q.shape
    tok = np.ascontiguousarray(tokens, dtype=np.int32)
    out = np.zeros((G, D), dtype=np.float64)
    ep = None
    if e is not None:
        e = _f32(e)
        ep = _pf(e)
    lib().oracle_attend_tokens(_pf(q), G, D, _pf(K), _pf(V), ep, _pi(tok), tok.shape[0],
                               scale, _pd(out))
    return out


# ---------------------------------------------------------------------------
# one decode step of one row
# ---------------------------------------------------------------------------

@dataclass
class RowStep:
    n_cand: int
    gamma_e: list
    gamma_q: list
    out: np.ndarray      # [G, D] fp64
    E: np.ndarray        # [n_cand] pooled eviction scores
    S: np.ndarray        # [n_cand] pooled query-aware scores

    @property
    def selected(self) -> list:
        return sorted(set(self.gamma_e) | set(self.gamma_q))


def step_row(n_tokens: int, q, K, V, e, block: int, sub: int, k_e: int, k_q: int,
             scale: float, pooled_bf16: bool = False) -> RowStep:
    """Selection and attention output of one row at one decode step.

    q [G, D]; K, V [>= n_tokens, D]; e [>= n_tokens]. All fp64 inside, the
    pooled keys exact; pooled_bf16 rounds them to the nearest bfloat16 (the
    variant that stores pooled keys in the model's dtype).
    """
    q, K, V, e = _f32(q), _f32(K), _f32(V), _f32(e)
    G, D = q.shape
    c = (n_tokens - 1) // block
    ge = np.zeros(max(k_e, 1), dtype=np.int32)
    gq = np.zeros(max(k_q, 1), dtype=np.int32)
    nge = np.zeros(1, dtype=np.int32)
    ngq = np.zeros(1, dtype=np.int32)
    out = np.zeros((G, D), dtype=np.float64)
    E = np.zeros(max(c, 1), dtype=np.float64)
    S = np.zeros(max(c, 1), dtype=np.float64)
    lib().oracle_step_row(n_tokens, G, D, block, sub, k_e, k_q, scale, int(pooled_bf16),
                          _pf(q), _pf(K), _pf(V),
                          _pf(e), _pi(ge), _pi(nge), _pi(gq), _pi(ngq), _pd(out), _pd(E), _pd(S))
    return RowStep(c, [int(v) for v in ge[: nge[0]]], [int(v) for v in gq[: ngq[0]]], out,
                   E[:c].copy(), S[:c].copy())


# ---------------------------------------------------------------------------
# swap list between consecutive steps (set difference, NOSI block swapping)
# ---------------------------------------------------------------------------

@dataclass
class SwapResult:
    fetch_block: list
    fetch_slot: list
    slot_block: list     # after the swap, -1 = empty slot
    gamma: float         # |Gamma(t) & Gamma(t-1)| / k


@dataclass
class SlotCache:
    """An HBM cache of k block slots for one row.

    After each step the cache holds exactly that step's selection. Blocks
    selected now but not cached are fetched, in ascending block order, into
    the free slots (empty, or holding a block no longer selected), taken in
    ascending slot order.
    """
    k: int
    slot_block: list = field(default_factory=list)
    prev: set = field(default_factory=set)

    def __post_init__(self):
        if not self.slot_block:
            self.slot_block = [-1] * self.k

    def step(self, selected) -> SwapResult:
        sel = set(int(b) for b in selected)
        assert len(sel) <= self.k
        cached = {b for b in self.slot_block if b >= 0}
        fetch = sorted(sel - cached)
        free = sorted(s for s, b in enumerate(self.slot_block) if b < 0 or b not in sel)
        assert len(free) >= len(fetch)
        slots = free[: len(fetch)]
        for b, s in zip(fetch, slots):
            self.slot_block[s] = b
        for s, b in enumerate(self.slot_block):
            if b >= 0 and b not in sel:
                self.slot_block[s] = -1
        gamma = len(sel & self.prev) / self.k
        self.prev = sel
        return SwapResult(fetch, slots, list(self.slot_block), gamma)


# ---------------------------------------------------------------------------
# prefill (training-time forward) with the selection per query block
# ---------------------------------------------------------------------------

def pool_queries(q: np.ndarray, pooled_bf16: bool = False) -> np.ndarray:
    """Pooled query of a query block, q [n, G, D] -> [G, D] fp64: the exact
    mean (rounded to the nearest bfloat16 with pooled_bf16)."""
    q = _f32(q)
    n, G, D = q.shape
    out = np.zeros((G, D), np.float64)
    lib().oracle_pool_queries(_pf(q), n, G, D, int(pooled_bf16), _pd(out))
    return out


@dataclass
class Prefill:
    out: np.ndarray      # [N, G, D] fp64
    sel: np.ndarray      # [n_query_blocks, k] int32, ascending, -1 padded


def prefill_row(q, K, V, e, block: int, sub: int, k_e: int, k_q: int, scale: float,
                pooled_bf16: bool = False) -> Prefill:
    """Causal prefill of one row with NOSA's selection per query block.
    q [N, G, D]; K, V [N, D]; e [N]."""
    q, K, V, e = _f32(q), _f32(K), _f32(V), _f32(e)
    N, G, D = q.shape
    nqb = -(-N // block)
    out = np.zeros((N, G, D), np.float64)
    sel = np.full((nqb, max(k_e + k_q, 1)), -1, np.int32)
    lib().oracle_prefill_row(N, G, D, block, sub, k_e, k_q, scale, int(pooled_bf16), _pf(q),
                             _pf(K), _pf(V), _pf(e), _pd(out), _pi(sel))
    return Prefill(out, sel[:, :k_e + k_q])


def prefill_qblock(q, K, V, e, i: int, block: int, sub: int, k_e: int, k_q: int, scale: float,
                   pooled_bf16: bool = False) -> Prefill:
    """Query block i alone of a row's prefill (what prefill_row computes for
    it): out [tokens of block i, G, D], sel [1, k]. q [N, G, D]; K, V [N, D];
    e [N]."""
    q, K, V, e = _f32(q), _f32(K), _f32(V), _f32(e)
    N, G, D = q.shape
    if not 0 <= i < -(-N // block):
        raise ValueError("query block out of range")
    n = min(block, N - i * block)
    out = np.zeros((n, G, D), np.float64)
    sel = np.full((1, max(k_e + k_q, 1)), -1, np.int32)
    lib().oracle_prefill_qblock(N, G, D, block, sub, k_e, k_q, scale, int(pooled_bf16), _pf(q),
                                _pf(K), _pf(V), _pf(e), i, _pd(out), _pi(sel))
    return Prefill(out, sel[:, :k_e + k_q])
