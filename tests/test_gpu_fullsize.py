"""Parity at the full workload shapes, in the launch configuration bench.py
times: every row runs on the GPU for every step; sampled rows are checked
against the oracle at every step (the oracle replays those rows from step 0,
so slot tables compare bit for bit too).
"""
import numpy as np
import pytest

import synth
from harness import oracle_trace
from test_gpu_parity import _compare_step, _gpu

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def _fullsize(name, rows, steps, w=None, all_rows_at=()):
    """Sampled rows at every step (selections, swap lists, slot tables,
    outputs); with all_rows_at, every row at those steps too (selections and
    outputs: the oracle's selection and attention need no history)."""
    gh = _gpu()
    w = w or synth.WORKLOADS[name]
    print(f"[fullsize] {name}: oracle on rows {rows}, steps 0..{steps - 1}", flush=True)
    tr = oracle_trace(w, rows=rows, steps=list(range(steps)))
    tr_all = None
    if all_rows_at:
        print(f"[fullsize] {name}: oracle on all {w.rows} rows at steps {list(all_rows_at)}",
              flush=True)
        tr_all = oracle_trace(w, steps=list(all_rows_at), ov=tr.ov, swaps=False)
    print(f"[fullsize] {name}: uploading inputs", flush=True)
    inp = gh.upload(w, ov=tr.ov, steps=steps)
    print(f"[fullsize] {name}: running the GPU path", flush=True)
    layer, res = gh.run(w, inp, list(range(steps)))
    for t in range(steps):
        for r in rows:
            _compare_step(w, tr, t, r, res[t])
    for t in all_rows_at:
        for r in range(w.rows):
            _compare_step(w, tr_all, t, r, res[t], check_swap=False)
    # every row's selection is a valid one: sizes, ascending, candidates only
    last = res[steps - 1]
    c = w.n_cand(steps - 1)
    for r in range(w.rows):
        n = int(last["n_sel"][r])
        sel = last["sel"][r, :n]
        assert n == min(w.k, c)
        assert (np.diff(sel) > 0).all() and sel[0] >= 0 and sel[-1] < c
    # locality: gamma >= k_e / k on average over rows and steps
    cnt = last["counters"]
    assert cnt[:, 1].sum() >= (w.k_e / w.k) * w.k * w.rows * (steps - 1) - 1e-9
    return layer


def test_fullsize_bf16_1layer_32k():
    _fullsize("bf16_1layer_32k", rows=[0, 21, 63], steps=128, all_rows_at=(0, 63, 64, 127))


def test_fullsize_bf16_3b_64k():
    _fullsize("bf16_3b_64k", rows=[0, 131, 255], steps=256, all_rows_at=(0, 255))


def test_fullsize_offload_1layer_128k():
    _fullsize("offload_1layer_128k", rows=[0, 77, 127], steps=256, all_rows_at=(0, 200))


@pytest.mark.parametrize("k_e", [32, 0])
def test_fullsize_offload_128k_budget_splits(k_e):
    """The locality ablation's other splits of the same budget k = 64 on the
    128k offload shape: k_e = 32, and k_e = 0 (query-aware top-k only, no
    locality bound). Steps 0..65 cross a block boundary (step 63)."""
    base = synth.WORKLOADS["offload_1layer_128k"]
    w = base.scaled(k_e=k_e, k_q=base.k - k_e, name=f"offload_1layer_128k_ke{k_e}")
    _fullsize(w.name, rows=[0, 77, 127], steps=66, w=w)


def test_fullsize_offload_128k_device_append():
    """The 128k offload shape with the host KV holding the context only: each
    step's token is appended on the GPU and the block completed at step 63 is
    written back to host memory; sampled rows match the oracle at every step
    and the written-back block matches the tokens."""
    from harness import row_kv
    gh = _gpu()
    w = synth.WORKLOADS["offload_1layer_128k"]
    steps, rows = 66, [0, 77, 127]
    tr = oracle_trace(w, rows=rows, steps=list(range(steps)))
    inp = gh.upload(w, ov=tr.ov, steps=steps, prefix_only=True)
    layer, res = gh.run(w, inp, list(range(steps)))
    for t in range(steps):
        for r in rows:
            _compare_step(w, tr, t, r, res[t])
    D, j = w.head_dim, w.n_cand(0)
    assert w.n_cand(steps - 1) == j + 1
    host = inp.kv.array(np.uint16, (w.rows, inp.nb, 2 * 64 * D))
    for r in range(w.rows):
        b, g = divmod(r, w.n_kv_heads)
        K, V = row_kv(w, 0, b, g)
        k_blk, v_blk = gh.unpack_blocks(host[r, j:j + 1], D)
        np.testing.assert_array_equal(k_blk, synth.bf16_bits(K[64 * j:64 * j + 64]),
                                      err_msg=f"row {r} K")
        np.testing.assert_array_equal(v_blk, synth.bf16_bits(V[64 * j:64 * j + 64]),
                                      err_msg=f"row {r} V")
    inp.kv.free()


# Steps of the 512-step 32-layer run checked against the oracle: the start,
# the first boundaries (a new candidate block at steps 64 and 128), the
# middle, the boundary at step 448 and the end of the run.
C4_STEPS = (0, 1, 2, 62, 63, 64, 65, 66, 126, 127, 128, 129, 130, 255, 256, 447, 448, 449,
            510, 511)


def test_fullsize_offload_8b_32layer_32k():
    """32 layers x batch 64 x 8 KV heads, all five stages per layer per step,
    the whole run of 512 steps (a new candidate block at steps 64, 128, ...,
    448).
    Layers 0, 17 and 31 are checked at the steps above on sampled rows, with
    the oracle replaying those rows from step 0 so that swap lists and slot
    tables compare bit for bit, and every row of layer 17 at step 64 and of
    layer 31 at step 511."""
    gh = _gpu()
    w = synth.WORKLOADS["offload_8b_32layer_32k"]
    steps = w.steps
    assert steps == 512 and max(C4_STEPS) == steps - 1
    layers_checked = {0: [0, 300, 511], 17: [5, 257], 31: [0, 511]}
    print(f"[fullsize] 8b: oracle layers {sorted(layers_checked)}, steps 0..{steps - 1}",
          flush=True)
    # the layers' traces side by side (the oracle's C calls release the GIL)
    traces = dict(zip(layers_checked, synth.parallel_map(
        lambda l: oracle_trace(w, layer=l, rows=layers_checked[l], steps=list(range(steps))),
        list(layers_checked), len(layers_checked))))
    all_at = {17: 64, 31: steps - 1}     # every row of a layer at one step
    tr_all = {}
    for l, t in all_at.items():
        print(f"[fullsize] 8b: oracle layer {l}, all {w.rows} rows, step {t}", flush=True)
        tr_all[l] = oracle_trace(w, layer=l, steps=[t], ov=traces[l].ov, swaps=False, workers=16)
    print("[fullsize] 8b: pinned host KV slabs", flush=True)
    slabs = gh.upload_slabs(w)
    layers, inputs = [], []
    for l in range(w.n_layers):
        ov = traces[l].ov if l in traces else None
        inp = gh.upload_layer(w, l, slabs[l % w.kv_slabs], ov, steps)
        inputs.append(inp)
        layers.append(gh.make_layer(w, inp))
    print("[fullsize] 8b: running 32 layers", flush=True)
    for layer in layers:
        layer.start(w.n_tokens(0))
    checked = 0
    for t in range(steps):
        for l, layer in enumerate(layers):
            layer.step(inputs[l].q[t], w.n_tokens(t))
            if l in traces and t in C4_STEPS:
                got = gh.snapshot(layer, w)
                for r in layers_checked[l]:
                    _compare_step(w, traces[l], t, r, got)
                    checked += 1
                if all_at.get(l) == t:
                    for r in range(w.rows):
                        _compare_step(w, tr_all[l], t, r, got, check_swap=False)
                    # every row's selection is a valid one at any size
                    c = w.n_cand(t)
                    for r in range(w.rows):
                        n = int(got["n_sel"][r])
                        sel = got["sel"][r, :n]
                        assert n == min(w.k, c)
                        assert (np.diff(sel) > 0).all() and sel[0] >= 0 and sel[-1] < c
        if t % 64 == 0:
            print(f"[fullsize] 8b: step {t} done", flush=True)
    assert checked == len(C4_STEPS) * sum(len(r) for r in layers_checked.values())
    for buf, _ in slabs:
        buf.free()
