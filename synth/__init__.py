"""Seeded synthetic inputs for the NOSA decode path.

This module is shared by the GPU path's tests, the oracle's tests and the
benchmark. It holds *none* of the method's arithmetic: only the workload
shapes, a counter-based random source and rounding to the input dtype.

Random source: numpy's Philox4x32-10 bit generator (Salmon et al., "Parallel
random numbers: as easy as 1, 2, 3", SC'11), keyed per tensor slice, so any
slice (one row's keys, one step's queries, one block's eviction logits)
regenerates on its own without generating anything else.

Workloads stand in for the decode workloads that the NOSA pages evaluate on
(1B/3B/8B models, long-context and long-generation tasks; NOSA Technical
Summary, Experimental Results). Those models and datasets are not used: every
tensor here is synthetic, with the shapes of those workloads.
"""
from __future__ import annotations

import hashlib
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, replace

import numpy as np

__all__ = [
    "Workload", "WORKLOADS", "rne_bf16", "bf16_bits", "stream",
    "keys_row", "values_row", "evict_row", "queries_step", "Overrides",
    "hidden_size", "hidden_step", "evict_head_weights", "prefill_queries",
]


@dataclass(frozen=True)
class Workload:
    """Shape of one synthetic decode workload.

    ``context`` tokens are prefilled; decode step t (0-based) appends token
    ``context + t`` and then queries with that step's q.
    """
    name: str
    seed: int
    batch: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    context: int
    steps: int
    k_e: int
    k_q: int
    dtype: str                 # "f32" or "bf16": dtype of q, K, V and the output
    offload: bool = False      # full KV in pinned host memory, HBM holds k blocks per row
    n_layers: int = 1
    block: int = 64
    sub_block: int = 16
    key_offset_std: float = 0.0  # std of the per-block mean offset added to K
    host_kv_slabs: int = 0     # >0: layers share this many host KV slabs (layer l uses l % slabs)
    # dtype of the pooled keys (and of a prefill's pooled queries): "f32", the
    # exact means rounded once to float32 (the oracle keeps them exact), or
    # "bf16", the variant that stores them in the model's dtype
    pooled: str = "f32"
    key_common: float = 0.0    # a constant added to every key element (near-tied scores)

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    @property
    def rows(self) -> int:
        return self.batch * self.n_kv_heads

    @property
    def k(self) -> int:
        return self.k_e + self.k_q

    @property
    def n_max(self) -> int:
        return self.context + self.steps

    @property
    def nb_max(self) -> int:
        return -(-self.n_max // self.block)

    @property
    def kv_slabs(self) -> int:
        return self.host_kv_slabs if self.host_kv_slabs > 0 else self.n_layers

    def n_tokens(self, t: int) -> int:
        return self.context + t + 1

    def n_cand(self, t: int) -> int:
        return (self.n_tokens(t) - 1) // self.block

    def scaled(self, **kw) -> "Workload":
        return replace(self, **kw)


# The five decode workloads, with the shapes of the pages' 1B/3B/8B decode
# settings, plus reduced ones that the fp64 oracle finishes in seconds.
WORKLOADS: dict[str, Workload] = {
    # batch 1, 4 query / 1 KV head, d 64, 2048-token context, k = 4 + 4, fp32
    "tiny_f32": Workload("tiny_f32", 1000, 1, 4, 1, 64, 2048, 16, 4, 4, "f32"),
    # batch 8, 32 / 8 heads, d 128, 32k context, k = 48 + 16, bf16, KV in HBM
    "bf16_1layer_32k": Workload("bf16_1layer_32k", 1001, 8, 32, 8, 128, 32768, 128,
                                48, 16, "bf16", key_offset_std=0.5),
    # batch 32, 24 / 8 heads, d 128, 64k context, k = 96 + 32, bf16, KV in HBM
    "bf16_3b_64k": Workload("bf16_3b_64k", 1002, 32, 24, 8, 128, 65536, 256,
                            96, 32, "bf16", key_offset_std=0.5),
    # batch 16, 32 / 8 heads, d 128, 128k context, k = 48 + 16, KV in pinned host memory
    "offload_1layer_128k": Workload("offload_1layer_128k", 1003, 16, 32, 8, 128, 131072, 256,
                                    48, 16, "bf16", offload=True, key_offset_std=0.5),
    # 32 layers, batch 64, 32 / 8 heads, d 128, 32k context, k = 48 + 16, host KV.
    # The full host KV of 32 layers would be 279 GB of pinned memory; layers
    # share 2 host slabs (layer l reads slab l % 2), which leaves every shape
    # and the bytes moved per step unchanged.
    "offload_8b_32layer_32k": Workload("offload_8b_32layer_32k", 1004, 64, 32, 8, 128, 32768, 512,
                                       48, 16, "bf16", offload=True, n_layers=32,
                                       key_offset_std=0.5, host_kv_slabs=2),
    # ---- reduced workloads: several tiles, ragged tails, block boundaries ----
    # fp32, 3 rows, 2 block boundaries crossed, ragged context
    "small_f32": Workload("small_f32", 2000, 1, 6, 2, 64, 1000, 140, 5, 3, "f32"),
    # bf16, GQA 4, 4 rows, a boundary crossed at t = 7
    "small_bf16": Workload("small_bf16", 2001, 2, 8, 2, 128, 3000, 80, 12, 6, "bf16",
                           key_offset_std=0.5),
    # bf16 offload, GQA 3
    "small_offload": Workload("small_offload", 2002, 2, 6, 2, 128, 4000, 72, 10, 6, "bf16",
                              offload=True, key_offset_std=0.5),
}


# ---------------------------------------------------------------------------
# rounding to the input dtype
# ---------------------------------------------------------------------------

def rne_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16, ties to even.

    Returns float32 values that are exactly representable in bfloat16.
    Inputs are finite (normal draws), so no NaN handling is needed.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) & np.uint32(0xFFFF0000)
    return r.view(np.float32)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Upper 16 bits of float32 values that are already bfloat16-exact."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    if np.any(u & np.uint32(0xFFFF)):
        raise ValueError("values are not bfloat16-exact")
    return (u >> np.uint32(16)).astype(np.uint16)


def _to_dtype(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "bf16":
        return rne_bf16(x)
    raise ValueError(dtype)


# ---------------------------------------------------------------------------
# keyed counter-based streams
# ---------------------------------------------------------------------------

def stream(*key) -> np.random.Generator:
    """Philox generator keyed by a tuple (workload seed, tensor tag, indices...)."""
    h = hashlib.blake2b(repr(key).encode(), digest_size=16).digest()
    k = np.frombuffer(h, dtype=np.uint64).copy()
    return np.random.Generator(np.random.Philox(key=k))


@dataclass
class Overrides:
    """Resampling attempts chosen by a caller that enforces selection margins.

    ``evict[(layer, b, g, block)] = a`` regenerates that block's 64 eviction
    logits from attempt ``a``; ``query[(layer, t, b, g)] = a`` regenerates the
    group's G query vectors for step t from attempt ``a``. Attempt 0 is the
    bulk draw.
    """
    evict: dict = None
    query: dict = None

    def __post_init__(self):
        self.evict = dict(self.evict or {})
        self.query = dict(self.query or {})


def keys_row(w: Workload, slab: int, b: int, g: int) -> np.ndarray:
    """Keys of row (b, g) in host-KV slab ``slab``: [n_max, D] in the input dtype.

    K = z + mu_block + key_common with z ~ N(0, 1) per element and, per
    block, a D-vector mu ~ N(0, key_offset_std^2) added to every key of that
    block.
    """
    z = stream(w.seed, "K", slab, b, g).standard_normal((w.n_max, w.head_dim), dtype=np.float32)
    if w.key_offset_std > 0:
        mu = stream(w.seed, "Kmu", slab, b, g).standard_normal(
            (w.nb_max, w.head_dim), dtype=np.float32) * np.float32(w.key_offset_std)
        z = z + np.repeat(mu, w.block, axis=0)[: w.n_max]
    if w.key_common:
        z = z + np.float32(w.key_common)
    return _to_dtype(z, w.dtype)


def values_row(w: Workload, slab: int, b: int, g: int) -> np.ndarray:
    """Values of row (b, g): [n_max, D] ~ N(0, 1) in the input dtype."""
    z = stream(w.seed, "V", slab, b, g).standard_normal((w.n_max, w.head_dim), dtype=np.float32)
    return _to_dtype(z, w.dtype)


def evict_row(w: Workload, layer: int, b: int, g: int, ov: Overrides | None = None) -> np.ndarray:
    """Per-token eviction logits of row (b, g): [n_max] float32 ~ N(0, 1)."""
    e = stream(w.seed, "E", layer, b, g).standard_normal(w.n_max, dtype=np.float32)
    if ov is not None:
        # a snapshot: other threads may add overrides for their own rows
        for (l, bb, gg, j), a in list(ov.evict.items()):
            if (l, bb, gg) == (layer, b, g) and a > 0:
                lo, hi = j * w.block, min((j + 1) * w.block, w.n_max)
                e[lo:hi] = stream(w.seed, "E", layer, b, g, j, a).standard_normal(
                    hi - lo, dtype=np.float32)
    return e


def queries_step(w: Workload, layer: int, t: int, ov: Overrides | None = None) -> np.ndarray:
    """Queries of decode step t: [batch, n_q_heads, D] in the input dtype.

    Query heads g*G .. g*G+G-1 belong to KV head g.
    """
    z = stream(w.seed, "Q", layer, t).standard_normal(
        (w.batch, w.n_q_heads, w.head_dim), dtype=np.float32)
    if ov is not None:
        G = w.group
        for (l, tt, b, g), a in list(ov.query.items()):
            if (l, tt) == (layer, t) and a > 0:
                z[b, g * G:(g + 1) * G] = stream(w.seed, "Q", layer, t, b, g, a).standard_normal(
                    (G, w.head_dim), dtype=np.float32)
    return _to_dtype(z, w.dtype)


def prefill_queries(w: Workload, layer: int, n_tokens: int, ov: Overrides | None = None,
                    batch: int | None = None, workers: int = 8) -> np.ndarray:
    """Queries of every token of a prefilled sequence: [batch, n_tokens, n_q_heads, D]
    ~ N(0, 1) in the input dtype, one stream per batch entry (``batch=b``:
    entry b alone, [n_tokens, n_q_heads, D]). ``ov.query[("prefill", layer, b,
    g, i)] = a`` regenerates query block i (its 64 tokens) of KV head g's query
    heads from attempt a."""
    if batch is None:
        return np.stack(parallel_map(lambda b: prefill_queries(w, layer, n_tokens, ov, b),
                                     range(w.batch), workers))
    b0 = batch
    z = stream(w.seed, "QP", layer, n_tokens, b0).standard_normal(
        (n_tokens, w.n_q_heads, w.head_dim), dtype=np.float32)
    if ov is not None:
        G = w.group
        for key, a in list(ov.query.items()):
            if len(key) == 5 and key[0] == "prefill" and key[1] == layer and key[2] == b0 and a > 0:
                _, _, b, g, i = key
                lo, hi = 64 * i, min(64 * i + 64, n_tokens)
                z[lo:hi, g * G:(g + 1) * G] = stream(w.seed, "QP", layer, b, g, i, a).standard_normal(
                    (hi - lo, G, w.head_dim), dtype=np.float32)
    return _to_dtype(z, w.dtype)


def hidden_size(w: Workload) -> int:
    """Model width of the synthetic eviction head's input: n_q_heads * head_dim."""
    return w.n_q_heads * w.head_dim


def hidden_step(w: Workload, layer: int, t: int) -> np.ndarray:
    """Hidden states of decode step t's token: [batch, hidden] ~ N(0, 1), input dtype."""
    z = stream(w.seed, "X", layer, t).standard_normal((w.batch, hidden_size(w)), dtype=np.float32)
    return _to_dtype(z, w.dtype)


def evict_head_weights(w: Workload, layer: int) -> np.ndarray:
    """Synthetic eviction-head weights [n_kv_heads, hidden] ~ N(0, 1/hidden), input dtype."""
    H = hidden_size(w)
    z = stream(w.seed, "WE", layer).standard_normal((w.n_kv_heads, H), dtype=np.float32)
    return _to_dtype(z * np.float32(1.0 / np.sqrt(H)), w.dtype)


def parallel_map(fn, items, workers: int = 8):
    """Map over independent slices with a thread pool (numpy releases the GIL)."""
    with ThreadPoolExecutor(max_workers=workers) as ex:
        return list(ex.map(fn, items))
