#!/usr/bin/env python3
"""Benchmark of the NOSA per-decode-step path on one MI355X.

A step is one pass of the whole path over one batch: pooling of a block that
just became complete (every 64 steps), block scoring, dual selection (Gamma_e
and Gamma_q), set difference against the cached blocks, block fetch from
pinned host memory (offloaded workloads only) and sparse decode attention.

Headline workload (the largest one-GPU configuration): the 8B-shaped decode
step, 32 layers, batch 64, 32 query / 8 KV heads, head_dim 128, 32k-token
context, blocks of 64 with sub-blocks of 16, budget k = 48 + 16, bf16, the
full KV in pinned host memory and an HBM cache of k blocks per row and layer.
`value` is its 32-layer decode steps/s over exactly --steps timed steps after
--warmup untimed ones (the first of which fills the empty caches). Legs, each
timed on its own: the 64k 3B-shaped and the 32k single-layer workloads with
the KV in HBM (attention against the HBM roofline), the 128k offloaded
single layer, prefill, the fused ingest launch and graph replay. Inputs are
synthetic (seeded Philox streams), resident in HBM (or pinned host memory for
the offloaded KV) when the timed region starts.

Prints one JSON line on stdout; progress goes to stderr.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "sparse decode steps/s + attn HBM GB/s (% peak); swap GB/s (% PCIe)"
HBM_PEAK_GBS = 8000.0
# the MI355X host link, PCIe 5.0 x16: 32 GT/s per lane, 64 GB/s per direction
PCIE_PEAK_GBS = 64.0


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="offload_8b_32layer_32k",
                    help="headline workload: offload_8b_32layer_32k (default) or a single-layer "
                         "workload with the KV in HBM")
    ap.add_argument("--legs", default="all", choices=["all", "none", "prefill"],
                    help="none: the headline workload alone (for profiler runs); prefill: the "
                         "headline workload, then the prefill leg alone")
    ap.add_argument("--resident-steps", type=int, default=200,
                    help="timed steps of each resident leg (64k 3B-shaped, 32k single layer); "
                         "their attention launches are timed in 25 or more of them")
    ap.add_argument("--decode-kernel", default="auto", choices=["auto", "valu", "mfma"])
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="wall-clock budget of the oracle sample (0 = skip)")
    ap.add_argument("--no-stage-breakdown", action="store_true")
    ap.add_argument("--overlap", action="store_true",
                    help="with KV in HBM, run attention over the unchanged eviction set on a "
                         "second stream, concurrently with scoring and selection (measured "
                         "slower on MI355X: both halves are HBM-bound and the query-set part "
                         "becomes a latency-bound launch of its own)")
    ap.add_argument("--offload-steps", type=int, default=60,
                    help="steps of the offloaded 128k-context leg (0 = skip)")
    ap.add_argument("--no-ablation", action="store_true",
                    help="skip the locality ablation of the offload leg (budget splits "
                         "k_e + k_q = k with k_e = 32 and 0, and per-block / per-token "
                         "hipMemcpyAsync copies against the fetch kernel)")
    ap.add_argument("--no-ingest", action="store_true",
                    help="skip the leg that runs the workload with the fused ingest launch "
                         "(QKV split, eviction head, KV append, pooling) in every step")
    ap.add_argument("--no-prefill", action="store_true",
                    help="skip the leg that prefills the workload's context with the selection "
                         "per query block (block-sparse causal attention on the matrix cores)")
    ap.add_argument("--no-graph", action="store_true",
                    help="skip the run with the step captured into a hipGraph and replayed")
    ap.add_argument("--no-cold", action="store_true",
                    help="skip the resident runs with the Infinity Cache flushed before each "
                         "step (a 1 GiB scratch read, then a 512 MiB scratch write)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run 4 device-to-device copies of 512 MiB (a reference kernel "
                         "of known traffic for hardware byte counters)")
    return ap.parse_args()


def recorded_traffic(workload: str, key: str = "traffic_bytes_per_launch"):
    """HBM bytes per launch recorded from rocprofv3 byte counters for this
    workload (key: traffic_bytes_per_launch, the attention kernel;
    fetch_hbm_bytes_per_launch, the fetch kernel's writes into the HBM cache),
    if the kernel sources are unchanged since; else None."""
    import hashlib
    prof = os.path.join(ROOT, "profiles", f"decode_step_{workload}.md")
    csrc = os.path.join(ROOT, "trainable_block_sparse_nosa_amd", "csrc")
    if not os.path.exists(prof):
        return None
    h = hashlib.sha256()
    for f in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(fh.read())
    fields = {}
    with open(prof) as fh:
        for line in fh:
            if ":" in line and line.split(":")[0] in (key, "source_sha256_16"):
                k, v = line.split(":", 1)
                fields[k.strip()] = v.strip()
    if fields.get("source_sha256_16") != h.hexdigest()[:16] or key not in fields:
        return None
    return float(fields[key])


def cpu_baseline(w, seconds: float):
    """Time the fp64 oracle as it stands (one thread) on a bounded sample of
    row-steps of the same workload (layer 0's rows in order at step 0, then
    step 1, ...) and scale the mean time per row-step to whole steps: all rows
    of every layer. The oracle is stateless per step, so each row-step pools
    and scores every candidate again."""
    import oracle
    import synth
    sc = 1.0 / math.sqrt(w.head_dim)
    done, t_used = 0, 0.0
    rows = {}
    t = 0
    while t_used < seconds and t < w.steps:
        q_t = synth.queries_step(w, 0, t)
        for r in range(w.rows):
            b, g = divmod(r, w.n_kv_heads)
            if r not in rows:
                rows[r] = (synth.keys_row(w, 0, b, g), synth.values_row(w, 0, b, g),
                           synth.evict_row(w, 0, b, g))
            K, V, e = rows[r]
            q = q_t[b, g * w.group:(g + 1) * w.group]
            t0 = time.perf_counter()
            oracle.step_row(w.n_tokens(t), q, K, V, e, 64, 16, w.k_e, w.k_q, sc,
                            pooled_bf16=w.pooled == "bf16")
            t_used += time.perf_counter() - t0
            done += 1
            if t_used >= seconds:
                break
        t += 1
    per_row_step = t_used / done
    per_step = w.rows * w.n_layers
    out = {
        "value": 1.0 / (per_row_step * per_step), "unit": "steps/s", "cores": 1, "kind": "oracle",
        "sample": f"{done} row-steps of {w.name} (layer 0, rows in order from step 0), "
                  f"{t_used:.1f} s of single-threaded fp64 oracle time, scaled to "
                  f"{w.rows} rows x {w.n_layers} layer(s) per step",
        "s_per_row_step": per_row_step,
    }
    out.update(cpu_info())
    return out


def setup(w, args, dev, device_append=False):
    """Generate the workload's inputs (untimed) and build its layer. Returns
    (layer, q, kv, new): with device_append, new = (k_new, v_new), each step's
    token of every row [T][rows][D] on the GPU (appended by the step; a
    completed block is written back to the host KV); else None."""
    import numpy as np
    import torch

    import synth
    from trainable_block_sparse_nosa_amd import _lib as L
    from trainable_block_sparse_nosa_amd.hostmem import PinnedBuffer
    from trainable_block_sparse_nosa_amd.pipeline import DecodeLayer, pack_blocks

    T = args.warmup + args.steps
    nb = w.nb_max
    BE = 2 * 64 * w.head_dim
    elem = 4 if w.dtype == "f32" else 2

    def conv(x):
        return np.ascontiguousarray(x, np.float32) if w.dtype == "f32" else synth.bf16_bits(x)

    def row_blocks(r):
        b, g = divmod(r, w.n_kv_heads)
        return pack_blocks(conv(synth.keys_row(w, 0, b, g)), conv(synth.values_row(w, 0, b, g)), nb)

    def to_dev(a):
        if w.dtype == "f32":
            return torch.from_numpy(a).to(dev)
        return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)

    t0 = time.time()
    if w.offload:
        host = PinnedBuffer(w.rows * nb * BE * elem)
        view = host.array(np.float32 if w.dtype == "f32" else np.uint16, (w.rows, nb, BE))

        def fill(r):
            view[r] = row_blocks(r)
        synth.parallel_map(fill, range(w.rows), 16)
        kv, kv_ptr = host, host.dev
    else:
        kv = torch.empty(w.rows, nb, BE, dtype=torch.float32 if w.dtype == "f32" else torch.bfloat16,
                         device=dev)
        for r0 in range(0, w.rows, 16):
            rr = list(range(r0, min(w.rows, r0 + 16)))
            for r, p in zip(rr, synth.parallel_map(row_blocks, rr, 16)):
                kv[r].copy_(to_dev(p))
        kv_ptr = kv
    e = np.zeros((w.rows, nb * 64), np.float32)   # rows padded to whole blocks
    e[:, :w.n_max] = np.stack(synth.parallel_map(
        lambda r: synth.evict_row(w, 0, *divmod(r, w.n_kv_heads)), range(w.rows), 16))
    e_tok = torch.from_numpy(e).to(dev)
    q = to_dev(np.stack(synth.parallel_map(lambda t: conv(synth.queries_step(w, 0, t)), range(T), 16)))
    torch.cuda.synchronize()
    log(f"{w.name}: inputs ready in {time.time() - t0:.1f} s")
    kind = {"auto": L.NOSA_DECODE_AUTO, "valu": L.NOSA_DECODE_VALU,
            "mfma": L.NOSA_DECODE_MFMA}[args.decode_kernel]
    new = None
    if device_append:
        def tokens(r):
            b, g = divmod(r, w.n_kv_heads)
            return (conv(synth.keys_row(w, 0, b, g)[w.context:w.context + T]),
                    conv(synth.values_row(w, 0, b, g)[w.context:w.context + T]))
        kvn = synth.parallel_map(tokens, range(w.rows), 16)
        new = (to_dev(np.ascontiguousarray(np.stack([k for k, _ in kvn], 1))),
               to_dev(np.ascontiguousarray(np.stack([v for _, v in kvn], 1))))
    layer = DecodeLayer(batch=w.batch, n_q_heads=w.n_q_heads, n_kv_heads=w.n_kv_heads,
                        head_dim=w.head_dim, k_e=w.k_e, k_q=w.k_q, max_blocks=nb,
                        dtype=L.NOSA_F32 if w.dtype == "f32" else L.NOSA_BF16, kv=kv_ptr,
                        kv_row_blocks=nb, e_tok=e_tok, offload=w.offload, decode_kernel=kind,
                        overlap=getattr(args, "overlap", False), device_append=device_append)
    return layer, q, kv, new


def run_step(layer, q, new, t, n_tokens, stream):
    """Step t of a layer built by setup (new: None, (k_new, v_new), or
    ("ingest", qkv, x) for a layer with an eviction head)."""
    if new is None:
        layer.step(q[t], n_tokens, stream)
    elif new[0] == "ingest":
        layer.step(None, n_tokens, stream, qkv=new[1][t], x=new[2][t])
    else:
        layer.step(q[t], n_tokens, stream, k_new=new[0][t], v_new=new[1][t])


MFMA_BF16_PEAK_TFLOPS = 2500.0


def prefill_flops(w, n_tokens: int, n_sel) -> float:
    """Algorithmic matrix flops of the prefill attention: per query token and
    head, 2 D for q.k and 2 D for p.v per attended token (the selected blocks'
    64 tokens each, plus its own block up to itself)."""
    G, D = w.group, w.head_dim
    total = 0.0
    nqb = -(-n_tokens // 64)
    for i in range(nqb):
        lo, hi = 64 * i, min(64 * i + 64, n_tokens)
        own = sum(range(1, hi - lo + 1))                # causal tokens of the block's queries
        sel_tokens = float(n_sel[i].sum()) * 64 * (hi - lo)  # summed over rows
        total += (sel_tokens + own * w.rows) * G * 4 * D
    return total


def prefill_leg(w, args, dev, stream):
    """The same workload's context prefilled with the selection per query
    block (pool the blocks, pool the queries, select per query block, causal
    block-sparse attention on the matrix cores), synthetic queries."""
    import torch
    from trainable_block_sparse_nosa_amd import _lib as L
    N = w.context
    sub = argparse.Namespace(**vars(args))
    sub.steps, sub.warmup = 1, 0
    layer, q, kv, _ = setup(w, sub, dev)
    del q
    g = torch.Generator(device="cpu").manual_seed(w.seed + 7)
    q_all = torch.empty(w.batch, N, w.n_q_heads, w.head_dim, dtype=torch.bfloat16, device=dev)
    for b in range(w.batch):
        q_all[b].copy_(torch.randn(N, w.n_q_heads, w.head_dim, generator=g).to(torch.bfloat16))
    times = {}

    def hook(name, fn, *a):
        on = a[-1] if a[-1] is not None else torch.cuda.current_stream()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(on)
        fn(*a)
        e1.record(on)
        times.setdefault(name, []).append((e0, e1))

    out, sel, n_sel = layer.prefill(q_all, N, stream)    # warm-up
    torch.cuda.synchronize()
    layer.stage_hook = hook
    t0 = time.perf_counter()
    out, sel, n_sel = layer.prefill(q_all, N, stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    layer.stage_hook = None
    ms = {k: sum(a.elapsed_time(b) for a, b in v) for k, v in times.items()}
    flops = prefill_flops(w, N, n_sel.cpu().numpy())
    att_s = ms["prefill_attention"] / 1e3
    res = {
        "workload": w.name, "n_tokens": N, "tokens_per_s": w.batch * N / wall,
        "ms_total": wall * 1e3, "ms_pool_queries": ms.get("pool_queries"),
        "ms_select": ms.get("prefill_select"), "ms_attention": ms["prefill_attention"],
        "roofline": {"kernel": "prefill_mfma_kernel", "bound": "mfma",
                     "achieved": flops / att_s / 1e12, "peak": MFMA_BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": flops / att_s / 1e12 / MFMA_BF16_PEAK_TFLOPS,
                     "algorithmic_flops": flops},
    }
    del layer, kv, q_all, out
    torch.cuda.empty_cache()
    return res


def ingest_leg(w, args, dev, stream, main_steps_per_s):
    """The same workload with the step before the path fused in (one launch per
    step: QKV split, eviction head, KV append, pooling of a completed block):
    its launch time and the whole step's rate. Hidden states, the fused
    projection output and the eviction head are synthetic (hidden = Hq * D)."""
    import numpy as np
    import torch
    import synth
    from trainable_block_sparse_nosa_amd import _lib as L
    from trainable_block_sparse_nosa_amd.pipeline import DecodeLayer
    T = args.warmup + args.steps
    layer, q, kv, new = setup(w, args, dev, device_append=True)
    H = synth.hidden_size(w)
    g = torch.Generator(device="cpu").manual_seed(w.seed)
    x = torch.randn(T, w.batch, H, generator=g).to(torch.bfloat16).to(dev)
    qkv = torch.cat([q.view(T, w.batch, -1), new[0].view(T, w.batch, -1),
                     new[1].view(T, w.batch, -1)], dim=2).contiguous()
    wt = torch.from_numpy(synth.bf16_bits(synth.evict_head_weights(w, 0)).view(np.int16)).to(dev)
    wt = wt.view(torch.bfloat16)
    lay = DecodeLayer(batch=w.batch, n_q_heads=w.n_q_heads, n_kv_heads=w.n_kv_heads,
                      head_dim=w.head_dim, k_e=w.k_e, k_q=w.k_q, max_blocks=w.nb_max,
                      dtype=L.NOSA_BF16, kv=kv, kv_row_blocks=w.nb_max, e_tok=layer.e_tok,
                      offload=False, evict_head=(wt, None))
    del layer
    elapsed, ev, _ = timed_run(lay, w, q, args, stream, event_stages=("ingest",),
                               new=("ingest", qkv, x))
    ms = [m for n, _, m in ev if n == "ingest"]
    # the same work unfused, for comparison: torch copies for the split, the
    # append launch, a torch matmul for the head and its scatter into e_tok,
    # the pool launch when a block completes
    Hq, Hkv, D = w.n_q_heads, w.n_kv_heads, w.head_dim
    wf = wt.float()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for _ in range(3):   # library handles and kernels loaded outside the timing
        torch.matmul(x[0].float(), wf.t())
    torch.cuda.synchronize()
    e0.record(stream)
    for t in range(args.steps):
        n = w.n_tokens(args.warmup + t)
        tok = n - 1
        row = qkv[args.warmup + t]
        lay.q_buf.copy_(row[:, :Hq * D].view(w.batch, Hq, D))
        kn = row[:, Hq * D:(Hq + Hkv) * D].contiguous()
        vn = row[:, (Hq + Hkv) * D:].contiguous()
        L.nosa_append_tokens(lay.shape, kn, vn, tok % 64, kv, w.nb_max, tok // 64, stream)
        lay.e_tok[:, tok] = torch.matmul(x[args.warmup + t].float(), wf.t()).reshape(-1)
        if tok % 64 == 63:
            L.nosa_pool_blocks(lay.shape, kv, w.nb_max, tok // 64, lay.e_tok, lay.e_stride,
                               tok // 64, tok // 64 + 1, lay.kbar, lay.e_blk, stream)
    e1.record(stream)
    torch.cuda.synchronize()
    out = {"steps_per_s": args.steps / elapsed, "ingest_us_avg": sum(ms) / len(ms) * 1e3,
           "ingest_us_max": max(ms) * 1e3, "hidden": H,
           "unfused_us_per_step": e0.elapsed_time(e1) * 1e3 / args.steps,
           "vs_main_steps_per_s": args.steps / elapsed / main_steps_per_s}
    del lay, kv, q, new, qkv, x
    torch.cuda.empty_cache()
    return out


ATTN_STAGES = ("decode", "decode_e", "decode_q")


def bracket(ev, i0: int, h: int, fn, a):
    """Run fn(*a) between events i0 and i0 + 1 of ev on stream handle h. The
    attention calls pass the two events to the library, which records them at
    the attention kernel's own start and end (so they agree with a kernel
    trace); any other call sits between two event records."""
    from trainable_block_sparse_nosa_amd import _lib as L
    if fn is L.nosa_decode_partial:
        L.nosa_decode_partial_timed(*a[:-1], ev.handle(i0), ev.handle(i0 + 1), a[-1])
    elif fn is L.nosa_decode_attend:
        L.nosa_decode_attend(*a[:-3], ev.handle(i0), ev.handle(i0 + 1), a[-1])
    else:
        ev.record(i0, h)
        fn(*a)
        ev.record(i0 + 1, h)


class HipTimingEvents:
    """A pool of HIP timing events created with hipEventDisableSystemFence:
    recording one does not write back and invalidate the caches, so bracketing
    every timed launch costs the step little. Uses the HIP runtime that torch
    has already loaded (the one libnosa.so resolves to as well)."""
    DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self, n: int):
        import ctypes
        import torch
        torch.cuda.init()
        path = None
        with open("/proc/self/maps") as fh:
            for line in fh:
                if "libamdhip64.so" in line:
                    path = line.split()[-1]
                    break
        if path is None:
            raise RuntimeError("the HIP runtime is not loaded")
        self._c = ctypes
        self.hip = ctypes.CDLL(path)
        P = ctypes.c_void_p
        self.hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(P), ctypes.c_uint]
        self.hip.hipEventRecord.argtypes = [P, P]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), P, P]
        self.hip.hipEventDestroy.argtypes = [P]
        self.events = []
        for _ in range(n):
            e = P()
            self._chk(self.hip.hipEventCreateWithFlags(ctypes.byref(e), self.DISABLE_SYSTEM_FENCE))
            self.events.append(e)

    @staticmethod
    def _chk(rc):
        if rc != 0:
            raise RuntimeError(f"HIP event call failed with error {rc}")

    def record(self, i: int, stream_handle: int):
        self._chk(self.hip.hipEventRecord(self.events[i], stream_handle))

    def handle(self, i: int) -> int:
        """The hipEvent_t of event i, as an integer."""
        return self.events[i].value

    def elapsed_ms(self, i: int, j: int) -> float:
        ms = self._c.c_float()
        self._chk(self.hip.hipEventElapsedTime(self._c.byref(ms), self.events[i], self.events[j]))
        return ms.value

    def close(self):
        for e in self.events:
            self.hip.hipEventDestroy(e)
        self.events = []


def timed_run(layer, w, q, args, stream, event_stages=ATTN_STAGES, new=None, sample_every=8,
              hist=None):
    """Warm up, then time exactly args.steps steps. HIP events bracket the
    listed stages in every sample_every-th timed step (see bracket(): the
    attention kernel's events mark its own start and end; timing
    every step would understate the throughput by ~8 % on the 32k workload).
    hist [warmup + steps][rows][k] (optional): each step's selection is copied
    there after the step (for the locality statistics; one small device copy
    per step, inside the timed region). Returns (elapsed s, [(stage, step,
    ms)], blocks fetched in the timed steps)."""
    import torch
    layer.start(w.n_tokens(0), stream)
    for t in range(args.warmup):
        run_step(layer, q, new, t, w.n_tokens(t), stream)
        if hist is not None:
            hist[t].copy_(layer.sel)
    torch.cuda.synchronize()
    fetched0 = int(layer.counters[:, 0].sum().item())
    pending = []
    cur = {"i": 0}
    ev = HipTimingEvents(2 * (3 * args.steps + 8))

    def hook(name, fn, *a):
        if name in event_stages and cur["i"] % sample_every == 0:
            on = a[-1] if a[-1] is not None else torch.cuda.current_stream()
            h = on.cuda_stream if hasattr(on, "cuda_stream") else int(on)
            i0 = 2 * len(pending)
            bracket(ev, i0, h, fn, a)
            pending.append((name, cur["i"], i0, i0 + 1))
        else:
            fn(*a)

    layer.stage_hook = hook
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for i in range(args.steps):
        cur["i"] = i
        run_step(layer, q, new, args.warmup + i, w.n_tokens(args.warmup + i), stream)
        if hist is not None:
            hist[args.warmup + i].copy_(layer.sel)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t_start
    layer.stage_hook = None
    fetched = int(layer.counters[:, 0].sum().item()) - fetched0
    times = [(n, i, ev.elapsed_ms(a, b)) for n, i, a, b in pending]
    ev.close()
    return elapsed, times, fetched


def attn_bytes(w, stage: str, n_tokens: int, n_blocks: int) -> int:
    """Algorithmic HBM bytes of one partial-attention launch over all rows:
    K and V of n_blocks blocks per row (plus the newest block's tokens when
    the launch covers it), one float32 eviction score per token, and q."""
    elem = 4 if w.dtype == "f32" else 2
    c = (n_tokens - 1) // 64
    cur = n_tokens - 64 * c if stage in ("decode", "decode_e") else 0
    toks = n_blocks * 64 + cur
    per_row = toks * (2 * w.head_dim * elem + 4)
    return w.rows * per_row + w.batch * w.n_q_heads * w.head_dim * elem


def h2d_peak_gbs(dev, nbytes=1 << 30, reps=5):
    """hipMemcpyAsync from pinned host memory to HBM (torch pinned tensor)."""
    import torch
    src = torch.empty(nbytes, dtype=torch.uint8, pin_memory=True)
    dst = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    dst.copy_(src, non_blocking=True)
    torch.cuda.synchronize()
    best = 0.0
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        dst.copy_(src, non_blocking=True)
        e1.record()
        torch.cuda.synchronize()
        best = max(best, nbytes / (e0.elapsed_time(e1) * 1e-3) / 1e9)
    del src, dst
    return best


def graph_leg(w, args, dev):
    """The resident workload's decode step captured once into a hipGraph and
    replayed step after step: the step's calls read the step record from
    device memory and its last call advances it. Before each replay the
    step's query is copied into the captured query buffer (inside the timed
    region, as a serving loop would do)."""
    import torch
    layer, q, kv, _ = setup(w, args, dev)
    layer.start(w.n_tokens(0))
    for t in range(args.warmup):
        run_step(layer, q, None, t, w.n_tokens(t), None)
    torch.cuda.synchronize()
    q_buf = torch.empty_like(q[0])
    graph = layer.graph_capture(w.n_tokens(args.warmup), q_buf)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        q_buf.copy_(q[args.warmup + i])
        graph.replay()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    del graph, layer, q, kv
    torch.cuda.empty_cache()
    return {"steps": args.steps, "steps_per_s": args.steps / elapsed,
            "ms_per_step": elapsed / args.steps * 1e3}


def read_probe_gbs(dev, nbytes=2 << 30, reps=10):
    """Achievable streaming HBM read bandwidth: the library's read probe over a
    buffer 8x the 256 MB Infinity Cache, best of `reps` launches (HIP events
    on the launch stream)."""
    import torch
    from trainable_block_sparse_nosa_amd import _lib as L
    src = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    src.fill_(1)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    st = torch.cuda.current_stream()
    L.nosa_read_probe(src, nbytes, sink, 2048, st)
    best = 0.0
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(st)
        L.nosa_read_probe(src, nbytes, sink, 2048, st)
        e1.record(st)
        torch.cuda.synchronize()
        best = max(best, nbytes / (e0.elapsed_time(e1) * 1e-3) / 1e9)
    del src, sink
    torch.cuda.empty_cache()
    return best


def cold_cache_run(layer, w, q, args, stream, n_steps: int, scratch_mib: int = 1024,
                   mode: str = "read"):
    """The resident workload with the Infinity Cache (256 MB) flushed before
    every step by touching scratch_mib MiB of scratch memory: mode "read"
    streams it through the read probe (clean lines: nothing to write back),
    mode "write" fills it (the dirty lines it leaves are written back while the
    next kernel runs, and that cost lands on the step's first kernels). HIP
    events around the attention partial launch of each step."""
    import torch
    from trainable_block_sparse_nosa_amd import _lib as L
    scratch = torch.zeros(scratch_mib << 20, dtype=torch.uint8, device=torch.device("cuda"))
    sink = torch.zeros(1, dtype=torch.int32, device=scratch.device)
    n = min(n_steps, args.warmup + args.steps)
    if n < 2:
        return None   # the first step (eviction top-k start) is not counted
    ev = HipTimingEvents(2 * n + 2)
    done = []

    def hook(name, fn, *a):
        if name == "decode":
            on = a[-1] if a[-1] is not None else torch.cuda.current_stream()
            h = on.cuda_stream if hasattr(on, "cuda_stream") else int(on)
            i0 = 2 * len(done)
            bracket(ev, i0, h, fn, a)
            done.append((t, i0))
        else:
            fn(*a)

    layer.start(w.n_tokens(0), stream)
    on = stream if stream is not None else torch.cuda.current_stream()
    layer.stage_hook = hook
    for t in range(n):
        if mode == "read":
            L.nosa_read_probe(scratch, scratch.numel(), sink, 2048, on)
        else:
            with torch.cuda.stream(on):
                scratch.fill_(t & 0xFF)
        run_step(layer, q, None, t, w.n_tokens(t), stream)
    torch.cuda.synchronize()
    layer.stage_hook = None
    c0 = w.n_cand(0)
    n_blk = min(w.k_e, c0) + min(w.k_q, c0 - min(w.k_e, c0))
    # the first step's launch includes the eviction top-k start; skip it
    res = [(ev.elapsed_ms(i0, i0 + 1), attn_bytes(w, "decode", w.n_tokens(t), n_blk))
           for t, i0 in done[1:]]
    ev.close()
    del scratch, sink
    ms = sum(a for a, _ in res) / len(res)
    gbs = sum(b for _, b in res) / (sum(a for a, _ in res) / 1e3) / 1e9
    return {"flush": mode, "scratch_mib": scratch_mib, "steps": len(res),
            "avg_launch_us": ms * 1e3, "achieved_gbs": gbs, "frac": gbs / HBM_PEAK_GBS}


def offload_leg(args, dev, stream):
    """The 128k-context offloaded workload: steps/s and swap GB/s of the fetch
    kernel against the measured pinned-host-to-HBM copy bandwidth. Each step's
    token is appended on the GPU and a completed block is written back to the
    host KV, so the loop is the whole offload cycle."""
    import synth
    base = synth.WORKLOADS["offload_1layer_128k"]
    w = base.scaled(steps=max(base.steps, args.warmup + args.offload_steps))
    sub = argparse.Namespace(**vars(args))
    sub.steps = args.offload_steps
    layer, q, kv, new = setup(w, sub, dev, device_append=True)
    import torch
    T = sub.warmup + sub.steps
    hist = torch.empty(T, w.rows, w.k, dtype=torch.int32, device=dev)
    # every step bracketed: the swap rate needs the fetch time of every step
    # (a step here takes ~1.3 ms, so the records cost it little)
    elapsed, ev, fetched = timed_run(layer, w, q, sub, stream, event_stages=("fetch", "decode"),
                                     new=new, sample_every=1, hist=hist)
    fetch_s = sum(ms for n, _, ms in ev if n == "fetch") / 1e3
    dec_ms = [ms for n, _, ms in ev if n == "decode"]
    block_bytes = 2 * 64 * w.head_dim * 2
    swap_gbs = fetched * block_bytes / fetch_s / 1e9
    peak = h2d_peak_gbs(dev)
    zc = zero_copy_contiguous_gbs(layer, w, stream)
    hk = host_memory_kinds(layer, w, stream)
    log(f"fetch kernel from coherent pinned memory {hk['coherent_gbs']:.1f} GB/s, "
        f"non-coherent {hk['noncoherent_gbs']:.1f} GB/s")
    gam = gamma_stats(hist.cpu().numpy(), [w.n_cand(t) for t in range(T)], w.k, w.k_e)
    del hist
    out = {
        "workload": w.name, "steps": sub.steps, "steps_per_s": sub.steps / elapsed,
        "ms_per_step": elapsed / sub.steps * 1e3,
        "fetched_mib_per_step": fetched * block_bytes / sub.steps / 2**20,
        "fetch_us_per_step": fetch_s / sub.steps * 1e6,
        "swap_gbs": swap_gbs, "h2d_memcpy_gbs": peak, "frac_of_h2d": swap_gbs / peak,
        "zero_copy_contiguous_gbs": zc, "host_memory_kinds": hk,
        "attn_partial_us_per_step": sum(dec_ms) / len(dec_ms) * 1e3,
        "gamma_mean": gam["mean"], "gamma": gam,
        "device_append": True,
    }
    # the same loop in two batch halves, the second half's fetch overlapping
    # the first half's attention
    from trainable_block_sparse_nosa_amd.pipeline import DecodeLayer
    from trainable_block_sparse_nosa_amd import _lib as L
    lay = DecodeLayer(batch=w.batch, n_q_heads=w.n_q_heads, n_kv_heads=w.n_kv_heads,
                      head_dim=w.head_dim, k_e=w.k_e, k_q=w.k_q, max_blocks=w.nb_max,
                      dtype=L.NOSA_BF16, kv=kv.dev, kv_row_blocks=w.nb_max, e_tok=layer.e_tok,
                      offload=True, device_append=new is not None, overlap=True)
    el2, _, _ = timed_run(lay, w, q, sub, stream, event_stages=(), new=new)
    out["overlap_halves"] = {"steps_per_s": sub.steps / el2,
                             "vs_serial": sub.steps / el2 / out["steps_per_s"]}
    log(f"offload in two batch halves, fetch overlapping attention: "
        f"{out['overlap_halves']['steps_per_s']:.1f} steps/s "
        f"({out['overlap_halves']['vs_serial']:.3f}x)")
    del lay
    if not args.no_ablation:
        out["ablation"] = locality_ablation(w, layer, q, kv, sub, dev, stream, out, block_bytes,
                                            new)
    kv.free()
    del layer, q
    return out


def gamma_stats(hist, n_cand, k: int, k_e: int) -> dict:
    """Locality from recorded selections: hist [T][..., k] int32 ascending
    block ids (-1 padded) of consecutive steps, n_cand[T] their candidate
    counts. gamma(t) = |Gamma(t) & Gamma(t-1)| / k per row (Methodology,
    Locality Guarantee), for t >= 1 of the record; the bound k_e / k is
    checked on the steps that complete no new block."""
    import numpy as np
    h = np.asarray(hist).reshape(len(hist), -1, k)
    T, R = h.shape[0], h.shape[1]
    nb = int(max(h.max(), 0)) + 2
    prev = None
    gam, gam_nn = [], []
    rows = np.arange(R)[:, None]
    for t in range(T):
        cur = np.zeros((R, nb), bool)
        cur[rows, np.where(h[t] >= 0, h[t], nb - 1)] = True
        cur[:, nb - 1] = False
        if prev is not None:
            g = (cur & prev).sum(axis=1) / k
            gam.append(g)
            if n_cand[t] == n_cand[t - 1]:
                gam_nn.append(g)
        prev = cur
    g_all = np.concatenate(gam) if gam else np.zeros(0)
    g_nn = np.concatenate(gam_nn) if gam_nn else np.zeros(0)
    bound = k_e / k
    return {"steps": T - 1, "rows": R, "mean": float(g_all.mean()) if g_all.size else None,
            "min": float(g_all.min()) if g_all.size else None,
            "min_no_new_block": float(g_nn.min()) if g_nn.size else None,
            "bound": bound, "bound_holds": bool(g_nn.size == 0 or g_nn.min() >= bound - 1e-12)}


def model_leg(args, dev, stream, h2d_gbs=None):
    """The 32-layer 8B-shaped decode step (batch 64, 32 / 8 heads, 32k context,
    k = 48 + 16, KV in pinned host memory): all five stages in every layer of
    every step, layer after layer on one stream. The host KV of 32 layers
    would take 279 GB of pinned memory; layers share two host slabs (layer l
    reads slab l % 2), which leaves every shape and the bytes moved per step
    unchanged. max(--warmup, 1) untimed steps come first (step 0 fills the
    empty HBM caches: every selected block is fetched, reported apart), then
    exactly --steps steps are timed, with HIP events at the start and end of
    every layer's fetch and attention kernels, and each layer's selection
    copied aside after its step (one small device copy per layer) for the
    locality statistics."""
    import numpy as np
    import torch

    import synth
    from trainable_block_sparse_nosa_amd import _lib as L
    from trainable_block_sparse_nosa_amd.hostmem import PinnedBuffer
    from trainable_block_sparse_nosa_amd.pipeline import DecodeLayer, pack_blocks

    base = synth.WORKLOADS["offload_8b_32layer_32k"]
    n, warm = args.steps, max(args.warmup, 1)
    T = warm + n
    w = base.scaled(steps=max(base.steps, T))
    nb, BE = w.nb_max, 2 * 64 * w.head_dim
    t0 = time.time()
    slabs = []
    for sl in range(w.kv_slabs):
        buf = PinnedBuffer(w.rows * nb * BE * 2)
        view = buf.array(np.uint16, (w.rows, nb, BE))

        def fill(r, sl=sl, view=view):
            b, g = divmod(r, w.n_kv_heads)
            view[r] = pack_blocks(synth.bf16_bits(synth.keys_row(w, sl, b, g)),
                                  synth.bf16_bits(synth.values_row(w, sl, b, g)), nb)
        synth.parallel_map(fill, range(w.rows), 16)
        slabs.append(buf)
    layers, qs = [], []
    for li in range(w.n_layers):
        e = np.zeros((w.rows, nb * 64), np.float32)
        e[:, :w.n_max] = np.stack(synth.parallel_map(
            lambda r: synth.evict_row(w, li, *divmod(r, w.n_kv_heads)), range(w.rows), 16))
        e_tok = torch.from_numpy(e).to(dev)
        qh = np.stack(synth.parallel_map(lambda t: synth.bf16_bits(synth.queries_step(w, li, t)),
                                         range(T), 16))
        qs.append(torch.from_numpy(qh.view(np.int16)).to(dev).view(torch.bfloat16))
        layers.append(DecodeLayer(batch=w.batch, n_q_heads=w.n_q_heads, n_kv_heads=w.n_kv_heads,
                                  head_dim=w.head_dim, k_e=w.k_e, k_q=w.k_q, max_blocks=nb,
                                  dtype=L.NOSA_BF16, kv=slabs[li % w.kv_slabs].dev,
                                  kv_row_blocks=nb, e_tok=e_tok, offload=True))
    torch.cuda.synchronize()
    log(f"{w.name}: {w.n_layers} layers ready in {time.time() - t0:.1f} s "
        f"({w.kv_slabs} pinned host slabs of {slabs[0].nbytes / 2**30:.1f} GiB)")

    def fetched_blocks():
        return sum(int(layer.counters[:, 0].sum().item()) for layer in layers)

    for layer in layers:
        layer.start(w.n_tokens(0), stream)
    torch.cuda.synchronize()
    tc = time.perf_counter()
    for li, layer in enumerate(layers):
        layer.step(qs[li][0], w.n_tokens(0), stream)
    torch.cuda.synchronize()
    cold_s = time.perf_counter() - tc
    cold_blocks = fetched_blocks()
    for t in range(1, warm):
        for li, layer in enumerate(layers):
            layer.step(qs[li][t], w.n_tokens(t), stream)
    # selections of the last untimed step and of every timed step
    hist = torch.empty(n + 1, w.n_layers, w.rows, w.k, dtype=torch.int32, device=dev)
    for li, layer in enumerate(layers):
        hist[0, li].copy_(layer.sel)
    torch.cuda.synchronize()
    f0 = fetched_blocks()
    ev = HipTimingEvents(2 * 2 * w.n_layers * n + 8)
    pending = []

    def hook(name, fn, *a):
        if name in ("fetch", "decode"):
            on = a[-1] if a[-1] is not None else torch.cuda.current_stream()
            h = on.cuda_stream if hasattr(on, "cuda_stream") else int(on)
            i0 = 2 * len(pending)
            bracket(ev, i0, h, fn, a)
            pending.append((name, i0, i0 + 1))
        else:
            fn(*a)

    for layer in layers:
        layer.stage_hook = hook
    torch.cuda.synchronize()
    ts = time.perf_counter()
    for i, t in enumerate(range(warm, T)):
        for li, layer in enumerate(layers):
            layer.step(qs[li][t], w.n_tokens(t), stream)
            hist[i + 1, li].copy_(layer.sel)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - ts
    for layer in layers:
        layer.stage_hook = None
    fetched = fetched_blocks() - f0
    fetch_ms = [ev.elapsed_ms(a, b) for nm, a, b in pending if nm == "fetch"]
    dec = [ev.elapsed_ms(a, b) for nm, a, b in pending if nm == "decode"]
    ev.close()
    block_bytes = 2 * 64 * w.head_dim * 2
    fetch_bytes = fetched * block_bytes
    swap_gbs = fetch_bytes / (sum(fetch_ms) / 1e3) / 1e9
    # attention: every layer's selection holds the full budget (512 candidates)
    attn_b = attn_bytes(w, "decode", w.n_tokens(warm), w.k)
    dec_avg_s = sum(dec) / len(dec) / 1e3
    attn_gbs = attn_b / dec_avg_s / 1e9
    gam = gamma_stats(hist.cpu().numpy(), [w.n_cand(t) for t in range(warm - 1, T)], w.k, w.k_e)
    out = {
        "workload": w.name, "layers": w.n_layers, "host_kv_slabs": w.kv_slabs,
        "steps": n, "warmup": warm, "steps_per_s": n / elapsed, "ms_per_step": elapsed / n * 1e3,
        "fetched_gib_per_step": fetch_bytes / n / 2**30,
        "fetch_ms_per_step": sum(fetch_ms) / n, "swap_gbs": swap_gbs,
        "attn_us_per_layer": dec_avg_s * 1e6,
        "gamma": gam,
        "cold_step_s": cold_s, "cold_fetched_gib": cold_blocks * block_bytes / 2**30,
        "fetch_roofline": {
            "kernel": "fetch_kernel (blocks of the swap list, pinned host memory to the HBM "
                      "cache, over PCIe)",
            "bound": "pcie", "achieved": swap_gbs, "peak": PCIE_PEAK_GBS, "unit": "GB/s",
            "frac": swap_gbs / PCIE_PEAK_GBS,
            "traffic": recorded_traffic(w.name, "fetch_hbm_bytes_per_launch"),
            "measured_h2d_gbs": h2d_gbs, "frac_of_measured_h2d": swap_gbs / h2d_gbs if h2d_gbs else None,
            "avg_launch_us": sum(fetch_ms) / len(fetch_ms) * 1e3,
            "algorithmic_bytes_per_launch": fetch_bytes / len(fetch_ms),
            "launches_timed": len(fetch_ms),
        },
        "attn_roofline": {
            "kernel": "decode_mfma_kernel (one chunk per row: the launch writes the output)",
            "bound": "hbm", "achieved": attn_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": attn_gbs / HBM_PEAK_GBS, "traffic": recorded_traffic(w.name),
            "avg_launch_us": dec_avg_s * 1e6, "algorithmic_bytes_per_launch": attn_b,
            "launches_timed": len(dec),
        },
    }
    del layers, qs, hist
    for buf in slabs:
        buf.free()
    torch.cuda.empty_cache()
    return out


def zero_copy_contiguous_gbs(layer, w, stream, reps=3):
    """The fetch kernel over contiguous host blocks (blocks 0..k-1 of every row
    into slots 0..k-1): the zero-copy read rate without the scatter of a
    selection."""
    import torch
    from trainable_block_sparse_nosa_amd import _lib as L
    dev = layer.cache.device
    k = w.k
    fb = torch.arange(k, dtype=torch.int32, device=dev).repeat(w.rows, 1).contiguous()
    nf = torch.full((w.rows,), k, dtype=torch.int32, device=dev)
    on = stream if stream is not None else torch.cuda.current_stream()
    best = 0.0
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(on)
        L.nosa_fetch_blocks(layer.shape, layer.kv, layer.kv_row_blocks, fb, fb, nf, k,
                            layer.cache, k, on)
        e1.record(on)
        torch.cuda.synchronize()
        best = max(best, w.rows * k * 2 * 64 * w.head_dim * 2 / (e0.elapsed_time(e1) * 1e-3) / 1e9)
    return best


def host_memory_kinds(layer, w, stream, reps=3):
    """The fetch kernel reading k blocks per row (256 MiB on the 128k shape)
    from pinned host memory allocated coherent (fine-grained, the default
    here) and non-coherent (coarse-grained): GB/s of each, best of
    `reps`."""
    import numpy as np
    import torch
    from trainable_block_sparse_nosa_amd import _lib as L
    from trainable_block_sparse_nosa_amd.hostmem import PinnedBuffer
    dev = layer.cache.device
    k = w.k
    nbytes = w.rows * k * 2 * 64 * w.head_dim * 2
    fb = torch.arange(k, dtype=torch.int32, device=dev).repeat(w.rows, 1).contiguous()
    nf = torch.full((w.rows,), k, dtype=torch.int32, device=dev)
    on = stream if stream is not None else torch.cuda.current_stream()
    out = {}
    for name, coherent in (("coherent_gbs", True), ("noncoherent_gbs", False)):
        buf = PinnedBuffer(nbytes, coherent=coherent)
        buf.array(np.uint8, (nbytes,))[:] = 1
        best = 0.0
        for _ in range(reps + 1):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(on)
            L.nosa_fetch_blocks(layer.shape, buf.dev, k, fb, fb, nf, k, layer.cache, k, on)
            e1.record(on)
            torch.cuda.synchronize()
            best = max(best, nbytes / (e0.elapsed_time(e1) * 1e-3) / 1e9)
        buf.free()
        out[name] = best
    out["bytes"] = nbytes
    return out


def locality_ablation(w, layer, q, kv, sub, dev, stream, nosa_run, block_bytes, new):
    """Same inputs, same budget k, other splits k_e + k_q: k_e = 0 is unconstrained
    query-aware top-k (no locality bound); NOSA's k_e bounds gamma >= k_e / k and
    with it the blocks fetched per step. Also the fetch kernel against copies
    issued one block (32 KiB) or one token (K and V rows, 512 B) at a time."""
    import numpy as np
    import torch
    from trainable_block_sparse_nosa_amd import _lib as L
    from trainable_block_sparse_nosa_amd.pipeline import DecodeLayer
    k = w.k
    rows = [dict(k_e=w.k_e, k_q=w.k_q, gamma_bound=w.k_e / k, gamma_mean=nosa_run["gamma_mean"],
                 gamma_min_no_new_block=nosa_run["gamma"]["min_no_new_block"],
                 fetched_mib_per_step=nosa_run["fetched_mib_per_step"],
                 steps_per_s=nosa_run["steps_per_s"], ms_per_step=nosa_run["ms_per_step"])]
    T = sub.warmup + sub.steps
    hist = torch.empty(T, w.rows, k, dtype=torch.int32, device=dev)
    for ke in (k // 2, 0):
        if ke == w.k_e:
            continue
        lay = DecodeLayer(batch=w.batch, n_q_heads=w.n_q_heads, n_kv_heads=w.n_kv_heads,
                          head_dim=w.head_dim, k_e=ke, k_q=k - ke, max_blocks=w.nb_max,
                          dtype=L.NOSA_BF16, kv=kv.dev, kv_row_blocks=w.nb_max,
                          e_tok=layer.e_tok, offload=True, device_append=new is not None)
        elapsed, _, fetched = timed_run(lay, w, q, sub, stream, event_stages=(), new=new,
                                        hist=hist)
        gam = gamma_stats(hist.cpu().numpy(), [w.n_cand(t) for t in range(T)], k, ke)
        rows.append(dict(k_e=ke, k_q=k - ke, gamma_bound=ke / k, gamma_mean=gam["mean"],
                         gamma_min_no_new_block=gam["min_no_new_block"],
                         fetched_mib_per_step=fetched * block_bytes / sub.steps / 2**20,
                         steps_per_s=sub.steps / elapsed, ms_per_step=elapsed / sub.steps * 1e3))
        log(f"ablation k_e={ke} k_q={k - ke}: {rows[-1]['steps_per_s']:.1f} steps/s, "
            f"gamma {rows[-1]['gamma_mean']:.3f}, {rows[-1]['fetched_mib_per_step']:.1f} MiB/step")
        del lay
        torch.cuda.empty_cache()
    # transfer granularity: the blocks the fetch kernel moved in the last step,
    # copied by hipMemcpyAsync (torch copy_) one block, then one 512-B token, at a time
    fb = layer.fetch_block.cpu().numpy()
    nf = layer.n_fetch.cpu().numpy()
    pairs = [(r, int(b)) for r in range(w.rows) for b in fb[r, :nf[r]]]
    if not pairs:
        return {"splits": rows, "granularity": None}
    host = torch.from_numpy(kv.array(np.uint8, (w.rows, w.nb_max, block_bytes)))
    dst = torch.empty(len(pairs), block_bytes, dtype=torch.uint8, device=dev)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev0.record(stream)
    for i, (r, b) in enumerate(pairs):
        dst[i].copy_(host[r, b], non_blocking=True)
    ev1.record(stream)
    torch.cuda.synchronize()
    per_block_gbs = len(pairs) * block_bytes / (ev0.elapsed_time(ev1) * 1e-3) / 1e9
    tok = 512
    n_tok = min(len(pairs) * (block_bytes // tok), 4096)   # a bounded sample of token copies
    flat = host.view(-1)
    ev0.record(stream)
    for i in range(n_tok):
        r, b = pairs[(i // (block_bytes // tok)) % len(pairs)]
        o = ((r * w.nb_max + b) * block_bytes) + (i % (block_bytes // tok)) * tok
        dst.view(-1)[i * tok:(i + 1) * tok].copy_(flat[o:o + tok], non_blocking=True)
    ev1.record(stream)
    torch.cuda.synchronize()
    per_token_gbs = n_tok * tok / (ev0.elapsed_time(ev1) * 1e-3) / 1e9
    del dst
    return {"splits": rows,
            "granularity": {"fetch_kernel_gbs": nosa_run["swap_gbs"],
                            "memcpy_per_block_gbs": per_block_gbs,
                            "memcpy_per_token_gbs": per_token_gbs,
                            "blocks": len(pairs), "token_copies_sampled": n_tok}}


def resident_leg(name, args, dev, stream, probe, steps, sample_every, extras=True):
    """A single-layer workload with the KV in HBM: `steps` timed steps after
    args.warmup untimed ones, the attention call bracketed by HIP events at its
    kernel's own start and end in every sample_every-th timed step, then
    (untimed) the per-stage breakdown, the locality statistics of a fresh
    replay of the same steps and, with extras, the cold-cache runs."""
    import torch
    import synth
    sub = argparse.Namespace(**vars(args))
    sub.steps = steps
    base = synth.WORKLOADS[name]
    T = sub.warmup + steps
    w = base.scaled(steps=max(base.steps, T))
    log(f"leg {w.name}: rows={w.rows} G={w.group} D={w.head_dim} ctx={w.context} "
        f"k={w.k_e}+{w.k_q} steps={T}")
    layer, q, kv, _ = setup(w, sub, dev)
    elapsed, ev, _ = timed_run(layer, w, q, sub, stream, sample_every=sample_every)
    c0 = w.n_cand(sub.warmup)
    n_e = min(w.k_e, c0)
    n_q = min(w.k_q, c0 - n_e)
    blocks = {"decode": n_e + n_q, "decode_e": n_e, "decode_q": n_q}
    tot_bytes = sum(attn_bytes(w, n, w.n_tokens(sub.warmup + i), blocks[n]) for n, i, _ in ev)
    tot_ms = sum(ms for _, _, ms in ev)
    dec_avg_s = tot_ms / len(ev) / 1e3
    achieved = tot_bytes / (tot_ms / 1e3) / 1e9
    sampled = len({i for _, i, _ in ev})
    steps_per_s = steps / elapsed
    log(f"{w.name}: {steps} steps in {elapsed * 1e3:.1f} ms: {steps_per_s:.1f} steps/s, "
        f"attention {dec_avg_s * 1e6:.1f} us avg over {len(ev)} launches, {achieved:.0f} GB/s")
    out = {
        "workload": w.name, "steps": steps, "warmup": sub.warmup, "steps_per_s": steps_per_s,
        "ms_per_step": elapsed / steps * 1e3,
        "roofline": {
            "kernel": "split-K attention kernel (decode_mfma_kernel: partials for the merge "
                      "kernel, or with one chunk per row the output itself)",
            "bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBS, "traffic": recorded_traffic(w.name),
            "avg_launch_us": dec_avg_s * 1e6, "algorithmic_bytes_per_launch": tot_bytes / len(ev),
            "launches_per_step": len(ev) / sampled, "launches_timed": len(ev),
            "read_probe_gbs": probe, "frac_of_read_probe": achieved / probe,
        },
        "attn_us_per_step": tot_ms / sampled * 1e3,
    }
    if not args.no_stage_breakdown:
        out["stages_us"] = stage_breakdown(layer, w, q, sub.warmup, min(steps, 50), stream)
    # locality: a fresh decode of the same steps, each step's selection copied aside
    layer.reset()
    layer.start(w.n_tokens(0), stream)
    hist = torch.empty(T, w.rows, w.k, dtype=torch.int32, device=dev)
    for t in range(T):
        layer.step(q[t], w.n_tokens(t), stream)
        hist[t].copy_(layer.sel)
    out["gamma"] = gamma_stats(hist.cpu().numpy(), [w.n_cand(t) for t in range(T)], w.k, w.k_e)
    if extras and not args.no_cold:
        out["cold_cache"] = {m: cold_cache_run(layer, w, q, sub, stream, 26, mib, m)
                             for m, mib in (("read", 1024), ("write", 512))}
        for m, c in out["cold_cache"].items():
            log(f"cache flushed by a {c['scratch_mib']} MiB scratch {m} before each step: "
                f"attention {c['avg_launch_us']:.1f} us, {c['achieved_gbs']:.0f} GB/s")
    del layer, q, kv, hist
    torch.cuda.empty_cache()
    if extras and not args.no_graph:
        g = graph_leg(w, sub, dev)
        g["vs_eager"] = g["steps_per_s"] / steps_per_s
        out["graph"] = g
        log(f"graph-replayed steps: {g['steps_per_s']:.1f} steps/s ({g['vs_eager']:.3f}x eager)")
    return w, out


def cpu_info() -> dict:
    model = None
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"cpu_model": model, "nproc": os.cpu_count(),
            "affinity_cpus": len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else None}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: --gpus {args.gpus} is not supported "
              "(rows shard across GPUs with no exchange; only the one-GPU share is measured)",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import synth

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()

    if args.copy_calibration:
        src = torch.empty(512 << 20, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(4):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        log("copy calibration: 4 x 512 MiB device-to-device")

    probe = read_probe_gbs(dev)
    log(f"streaming-read probe: {probe:.0f} GB/s")
    h2d = h2d_peak_gbs(dev)
    log(f"pinned hipMemcpy H2D: {h2d:.1f} GB/s")

    legs = {}
    hw = synth.WORKLOADS[args.workload]
    if hw.offload and hw.n_layers > 1:
        head = model_leg(args, dev, stream, h2d)
        log(f"{head['workload']}: {head['steps_per_s']:.2f} steps/s ({head['ms_per_step']:.1f} ms "
            f"per 32-layer step), {head['fetched_gib_per_step']:.2f} GiB fetched per step at "
            f"{head['swap_gbs']:.1f} GB/s, attention {head['attn_us_per_layer']:.1f} us per layer; "
            f"gamma mean {head['gamma']['mean']:.4f}, min on no-new-block steps "
            f"{head['gamma']['min_no_new_block']}")
        value, w_head = head["steps_per_s"], hw
        roofline, attn_roofline = head.pop("fetch_roofline"), head.pop("attn_roofline")
        ms_per_step = head["ms_per_step"]
        legs[hw.name] = head
    elif not hw.offload:
        w_head, head = resident_leg(args.workload, argparse.Namespace(**{**vars(args)}), dev,
                                    stream, probe, args.steps, max(1, args.steps // 25))
        value, ms_per_step = head["steps_per_s"], head["ms_per_step"]
        roofline, attn_roofline = head.pop("roofline"), None
        legs[hw.name] = head
    else:
        print("the headline workload is the 32-layer offload step or a resident one",
              file=sys.stderr)
        sys.exit(2)

    # resident legs: the 64k 3B-shaped workload (1.6 GB of HBM reads per step,
    # the bandwidth of record) and the 32k one (its working set fits the 256 MB
    # Infinity Cache); 25 or more attention launches timed in each
    if args.legs in ("none", "prefill"):
        args.no_ingest = True
        args.no_prefill = args.legs == "none"
        args.offload_steps = 0
    for name, extras in (("bf16_3b_64k", False), ("bf16_1layer_32k", True)):
        if args.legs in ("none", "prefill"):
            break
        if name in legs:
            continue
        rs = args.resident_steps
        _, legs[name] = resident_leg(name, args, dev, stream, probe, rs, max(1, rs // 25), extras)

    w32 = synth.WORKLOADS["bf16_1layer_32k"]
    if not args.no_ingest and "bf16_1layer_32k" in legs:
        sub = argparse.Namespace(**vars(args))
        sub.steps = args.resident_steps
        log(f"ingest leg: {w32.name} with the fused ingest launch")
        legs["ingest"] = ingest_leg(w32.scaled(steps=max(w32.steps, sub.warmup + sub.steps)), sub,
                                    dev, stream, legs["bf16_1layer_32k"]["steps_per_s"])
        log(f"ingest: {legs['ingest']['steps_per_s']:.1f} steps/s, launch "
            f"{legs['ingest']['ingest_us_avg']:.1f} us")
    if not args.no_prefill:
        log(f"prefill leg: {w32.name}, {w32.context} tokens")
        legs["prefill"] = prefill_leg(w32, args, dev, stream)
        p = legs["prefill"]
        log(f"prefill: {p['tokens_per_s']:.0f} tokens/s, attention {p['ms_attention']:.1f} ms = "
            f"{p['roofline']['achieved']:.0f} TFLOP/s, selection {p['ms_select']:.1f} ms")
    if args.offload_steps > 0:
        log("offload leg: offload_1layer_128k")
        legs["offload_1layer_128k"] = offload_leg(args, dev, stream)
        o = legs["offload_1layer_128k"]
        log(f"offload: {o['steps_per_s']:.1f} steps/s, swap {o['swap_gbs']:.1f} GB/s = "
            f"{100 * o['frac_of_h2d']:.1f} % of hipMemcpy H2D {o['h2d_memcpy_gbs']:.1f} GB/s")

    cpu = None
    if args.cpu_seconds > 0:
        log("timing the oracle samples on the host")
        cpu = cpu_baseline(w_head, args.cpu_seconds)
        cpu["by_workload"] = {n: cpu_baseline(synth.WORKLOADS[n], args.cpu_seconds / 4)
                              for n in ("bf16_1layer_32k", "bf16_3b_64k")}
        for n, c in cpu["by_workload"].items():
            c.pop("by_workload", None)

    result = {
        "metric": METRIC,
        "value": value,
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": legs[w_head.name].get("warmup", args.warmup),
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w_head.dtype,
        "data": "synthetic",
        "config": {
            "workload": w_head.name, "layers": w_head.n_layers, "batch": w_head.batch,
            "n_q_heads": w_head.n_q_heads, "n_kv_heads": w_head.n_kv_heads,
            "head_dim": w_head.head_dim, "context": w_head.context, "block": 64,
            "sub_block": 16, "k_e": w_head.k_e, "k_q": w_head.k_q,
            "kv": "pinned host" if w_head.offload else "hbm", "pooled_keys": "f32",
            "decode_kernel": args.decode_kernel,
        },
        "roofline": roofline,
        "attn_roofline": attn_roofline,
        "read_probe_gbs": probe,
        "h2d_memcpy_gbs": h2d,
        "legs": legs,
        "cpu_baseline": cpu,
    }
    print(json.dumps(result), flush=True)


def stage_breakdown(layer, w, q, t0: int, n: int, stream):
    """Per-stage GPU time (us per call) from events placed around each stage's
    launch, on a replay of the timed steps from a fresh start. The "decode"
    stage is the whole attention call: with several chunks per row it holds
    the partial kernel and the merge kernel, with one chunk per row a single
    launch."""
    import torch
    pending = []

    def hook(name, fn, *a):
        on = a[-1] if a[-1] is not None else torch.cuda.current_stream()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(on)
        fn(*a)
        e1.record(on)
        pending.append((name, e0, e1))

    layer.start(w.n_tokens(0), stream)
    for t in range(t0):
        layer.step(q[t], w.n_tokens(t), stream)
    layer.stage_hook = hook
    try:
        for t in range(t0, t0 + n):
            layer.step(q[t], w.n_tokens(t), stream)
        torch.cuda.synchronize()
    finally:
        layer.stage_hook = None
    acc, cnt = {}, {}
    for name, e0, e1 in pending:
        acc[name] = acc.get(name, 0.0) + e0.elapsed_time(e1) * 1e3
        cnt[name] = cnt.get(name, 0) + 1
    return {k: acc[k] / cnt[k] for k in acc}


if __name__ == "__main__":
    main()
