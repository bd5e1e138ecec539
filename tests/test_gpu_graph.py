"""Decode steps replayed from a captured graph: the step record lives in
device memory, every call of the step reads it in its kernels and the step's
last call moves it on. Each replayed step is compared with the fp64 oracle
like an eagerly launched one: selections, swap lists and slot tables
bit-exact, outputs within the dtype's tolerance."""
import pytest

import synth
from harness import oracle_trace

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gpu_harness
    return gpu_harness


@pytest.mark.parametrize("name,append", [("small_bf16", False), ("small_bf16", True),
                                         ("small_f32", False), ("small_f32", True)])
def test_graph_replayed_steps(name, append):
    gh = _gpu()
    from test_gpu_parity import _compare_step
    w = synth.WORKLOADS[name]
    tr = oracle_trace(w)
    inp = gh.upload(w, ov=tr.ov, prefix_only=append)
    layer = gh.make_layer(w, inp, fuse_score=True, device_append=append)
    layer.start(w.n_tokens(0))
    q_buf = torch.empty_like(inp.q[0])
    kb = torch.empty_like(inp.k_new[0]) if append else None
    vb = torch.empty_like(inp.v_new[0]) if append else None
    graph = layer.graph_capture(w.n_tokens(0), q_buf, kb, vb)
    for t in range(w.steps):
        q_buf.copy_(inp.q[t])
        if append:
            kb.copy_(inp.k_new[t])
            vb.copy_(inp.v_new[t])
        graph.replay()
        got = gh.snapshot(layer, w)
        for r in range(w.rows):
            _compare_step(w, tr, t, r, got)
    last = w.steps - 1
    assert layer.step_dev.cpu().tolist() == [w.n_tokens(last) + 1, w.n_cand(last)]


def test_eager_steps_continue_after_replays():
    """Half the steps replayed, the rest launched eagerly on the same layer."""
    gh = _gpu()
    from test_gpu_parity import _compare_step
    w = synth.WORKLOADS["small_bf16"]
    tr = oracle_trace(w)
    inp = gh.upload(w, ov=tr.ov)
    layer = gh.make_layer(w, inp, fuse_score=True)
    layer.start(w.n_tokens(0))
    q_buf = torch.empty_like(inp.q[0])
    graph = layer.graph_capture(w.n_tokens(0), q_buf)
    half = w.steps // 2
    for t in range(w.steps):
        if t < half:
            q_buf.copy_(inp.q[t])
            graph.replay()
            if t == half - 1:
                torch.cuda.synchronize()
                layer.graph_done(w.n_tokens(t))
        else:
            layer.step(inp.q[t], w.n_tokens(t))
        got = gh.snapshot(layer, w)
        for r in range(w.rows):
            _compare_step(w, tr, t, r, got)


def test_graph_replayed_steps_fullsize_32k():
    """The 8 x 32/8-head, 32k-context workload (the benchmark's) replayed from
    one captured graph for 70 steps, across the block boundary at step 63;
    sampled rows compared with the oracle at every step, the record at the
    end. With 64 rows, the step's scoring runs on the split grid and the
    selection as its own launch, both reading the step record."""
    gh = _gpu()
    from test_gpu_parity import _compare_step
    w = synth.WORKLOADS["bf16_1layer_32k"]
    steps, rows = 70, [0, 21, 63]
    tr = oracle_trace(w, rows=rows, steps=list(range(steps)))
    inp = gh.upload(w, ov=tr.ov, steps=steps)
    layer = gh.make_layer(w, inp)
    layer.start(w.n_tokens(0))
    q_buf = torch.empty_like(inp.q[0])
    graph = layer.graph_capture(w.n_tokens(0), q_buf)
    for t in range(steps):
        q_buf.copy_(inp.q[t])
        graph.replay()
        got = gh.snapshot(layer, w)
        for r in rows:
            _compare_step(w, tr, t, r, got)
    assert w.n_cand(steps - 1) > w.n_cand(0), "a block completes during the replays"
    assert layer.step_dev.cpu().tolist() == [w.n_tokens(steps - 1) + 1, w.n_cand(steps - 1)]


@pytest.mark.parametrize("case", ["split", "fused"])
def test_graph_replayed_certified_near_ties(case):
    """Certified scoring with the step record in device memory: the near-tie
    workloads of the parity tests (every candidate inside the bf16 copy's
    window, the rescoring in two passes) replayed from a captured graph."""
    gh = _gpu()
    from test_gpu_parity import NEAR_TIES, _compare_step
    base = synth.WORKLOADS["small_bf16"]
    w = base.scaled(name="graph_ties_" + case, seed=3500 + ["split", "fused"].index(case),
                    **NEAR_TIES[case])
    tr = oracle_trace(w)
    inp = gh.upload(w, ov=tr.ov)
    layer = gh.make_layer(w, inp, fuse_score=True)
    assert layer.scores_certified
    layer.start(w.n_tokens(0))
    q_buf = torch.empty_like(inp.q[0])
    graph = layer.graph_capture(w.n_tokens(0), q_buf)
    for t in range(w.steps):
        q_buf.copy_(inp.q[t])
        graph.replay()
        got = gh.snapshot(layer, w)
        for r in range(w.rows):
            _compare_step(w, tr, t, r, got)
