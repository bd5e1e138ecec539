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


def _fullsize(name, rows, steps):
    gh = _gpu()
    w = synth.WORKLOADS[name]
    print(f"[fullsize] {name}: oracle on rows {rows}, steps 0..{steps - 1}", flush=True)
    tr = oracle_trace(w, rows=rows, steps=list(range(steps)))
    print(f"[fullsize] {name}: uploading inputs", flush=True)
    inp = gh.upload(w, ov=tr.ov, steps=steps)
    print(f"[fullsize] {name}: running the GPU path", flush=True)
    layer, res = gh.run(w, inp, list(range(steps)))
    for t in range(steps):
        for r in rows:
            _compare_step(w, tr, t, r, res[t])
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
    _fullsize("bf16_1layer_32k", rows=[0, 21, 63], steps=128)


def test_fullsize_bf16_3b_64k():
    _fullsize("bf16_3b_64k", rows=[0, 131, 255], steps=256)


def test_fullsize_offload_1layer_128k():
    _fullsize("offload_1layer_128k", rows=[0, 77, 127], steps=256)
