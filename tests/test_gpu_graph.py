"""The entry points captured in a HIP graph (torch.cuda.CUDAGraph) and
replayed step after step give, bit for bit, what the same calls give when
launched one by one.

"r9700-stack v0.2.4" (section "A defect found and fixed before the tag")
describes a conv-window update whose result depended on how a step was
launched: right inside full graphs, wrong in eagerly built steps, because a
host-side width stood in for what the record holds.  Here every value that
changes from step to step (inputs, acceptance counts, parity, lengths, page
indices) reaches the kernels through device memory, and the counters the
kernels use (arrival words, the decode work counter, the verify flag word)
return to their resting values inside the kernels, so one capture serves
every later step of the same host-side shape.  Each replay is preceded by
ordinary eager work (copying that step's inputs into the captured buffers)
and followed by a synchronisation and a comparison with the eager run."""
import numpy as np
import pytest
import torch

import gdn_workloads as wk
from gpu_util import DEV, dev, dims_of, gdn, make_batch, params_of, seq_pools

pytestmark = pytest.mark.gpu

REPLAYS = 4


def _seq_case(wl, chunk):
    """Pools for an eager run and a graph run of the same steps, the static
    input buffers of each, and the per-step inputs."""
    g = gdn()
    base = wk.make_sequence_inputs(wl)
    n = len(wl.seqlens)
    pages = list(range(n))
    runs = []
    for _ in range(2):
        dims, conv, state = seq_pools(wl, base, pages, n)
        runs.append(dict(conv=conv, state=state))
    params = params_of(base, wl)
    steps = []
    for s in range(REPLAYS):
        f = wk.make_sequence_inputs(wl.replace(seed=wl.seed + 200 + s))
        steps.append(tuple(dev(f[k], dims.act_torch) for k in ("x", "a", "b")))
    n_rows = steps[0][0].shape[0]
    batch = make_batch(base["cu_seqlens"], pages, n_rows)
    for r in runs:
        r["x"], r["a"], r["b"] = (torch.empty_like(t) for t in steps[0])
        r["o"] = torch.full((n_rows, wl.h_v, wl.d_v), float("nan"), device=DEV)
        r["ws"] = None
        if chunk:
            need = g.gdn_chunked_workspace_bytes(dims, batch.n_seqs, batch.n_rows, chunk)
            r["ws"] = torch.empty(max(need, 1), dtype=torch.uint8, device=DEV)
    return g, dims, params, batch, runs, steps


def _seq_call(g, dims, params, batch, r, chunk):
    if chunk:
        g.gdn_chunked_prefill(dims, params, r["x"], r["a"], r["b"], batch, r["conv"], r["state"], chunk=chunk,
                              o=r["o"], workspace=r["ws"])
    else:
        g.gdn_recurrent_seq(dims, params, r["x"], r["a"], r["b"], batch, r["conv"], r["state"], o=r["o"])


def _warm(fn):
    """Run fn once on a side stream (the library's first call on a device
    queries the resident grid size), as torch's capture recipe asks."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()


@pytest.mark.parametrize("case", ["decode", "short_prefill", "chunked"])
def test_sequence_steps_replayed_from_a_graph_equal_eager_launches(case):
    """Decode (the streaming kernel with its work counter), a ragged
    token-by-token batch and a chunked prefill, each captured once and
    replayed for four steps that continue the same sequences."""
    if case == "decode":
        wl, chunk = wk.DECODE, 0
    elif case == "short_prefill":
        wl, chunk = wk.DECODE.replace(seqlens=(45, 83, 7, 1, 130), seed=41), 0
    else:
        wl, chunk = wk.DECODE.replace(seqlens=(200, 64, 1, 131), seed=42), 64
    g, dims, params, batch, (eager, graph), steps = _seq_case(wl, chunk)

    # a throw-away call on copies of the pools warms the library up
    spare = dict(graph, conv=type(graph["conv"])(graph["conv"].buf.clone(), graph["conv"].sync.clone()),
                 state=type(graph["state"])(graph["state"].buf.clone()))
    for t, src in zip(("x", "a", "b"), steps[0]):
        spare[t] = src.clone()
    spare["o"] = torch.empty_like(graph["o"])
    _warm(lambda: _seq_call(g, dims, params, batch, spare, chunk))

    cg = torch.cuda.CUDAGraph()
    with torch.cuda.graph(cg):
        _seq_call(g, dims, params, batch, graph, chunk)

    for s, (x, a, b) in enumerate(steps):
        for r in (eager, graph):
            r["x"].copy_(x)
            r["a"].copy_(a)
            r["b"].copy_(b)
            r["o"].fill_(float("nan"))
        _seq_call(g, dims, params, batch, eager, chunk)
        cg.replay()
        torch.cuda.synchronize()
        assert not torch.isnan(eager["o"]).any(), s
        assert torch.equal(graph["o"], eager["o"]), s
        assert torch.equal(graph["state"].buf, eager["state"].buf), s
        assert torch.equal(graph["conv"].buf, eager["conv"].buf), s
        assert int(graph["conv"].sync.abs().sum()) == 0, s
    # the steps moved the state: the replays were not idle
    assert not torch.equal(graph["state"].buf, spare["state"].buf)


@pytest.mark.parametrize("layout", [0, 1])
def test_verify_steps_replayed_from_a_graph_equal_eager_launches(layout):
    """Speculative verify captured once (one-page and slots) and replayed
    for every step of the workload, with that step's candidates, the
    previous step's acceptance counts and the step parity written into the
    captured buffers before each replay; the flag word alternates inside the
    kernel, so the replays walk the record's two slots."""
    g = gdn()
    wl = wk.SPEC_VERIFY.replace(n_req=8, n_steps=6, seed=43)
    inp = wk.make_verify_inputs(wl)
    dims = dims_of(wl, n_spec=wl.n_cand - 1)
    R, K, C = wl.n_req, wl.n_cand, wl.c_conv
    params = params_of(inp, wl)
    rp = torch.arange(R, dtype=torch.int32, device=DEV)

    def make():
        pages = g.SpecPages.alloc(dims, layout, R, DEV)
        conv = g.ConvPool.alloc(dims, R, 3 + dims.n_spec, DEV)
        st = pages.states()
        for r in range(R):
            st[r, 0] = dev(inp["S0"][r], dims.state_torch)
            conv.buf[r, :3] = dev(inp["window0"][r], dims.act_torch)
        return dict(pages=pages, conv=conv,
                    x=torch.empty((R * K, C), dtype=dims.act_torch, device=DEV),
                    a=torch.empty((R * K, wl.h_v), dtype=dims.act_torch, device=DEV),
                    b=torch.empty((R * K, wl.h_v), dtype=dims.act_torch, device=DEV),
                    acc=torch.zeros(R, dtype=torch.int32, device=DEV),
                    par=torch.zeros(R, dtype=torch.uint8, device=DEV),
                    o=torch.full((R * K, wl.h_v, wl.d_v), float("nan"), device=DEV),
                    err=torch.zeros(1, dtype=torch.int32, device=DEV))

    def call(r):
        g.gdn_spec_verify(dims, params, r["pages"], r["x"], r["a"], r["b"], R, K, rp, r["acc"], r["par"],
                          r["conv"], o=r["o"], err=r["err"])

    def load_step(r, s):
        r["x"].copy_(dev(inp["x"][s].reshape(R * K, C), dims.act_torch))
        r["a"].copy_(dev(inp["a"][s].reshape(R * K, wl.h_v), dims.act_torch))
        r["b"].copy_(dev(inp["b"][s].reshape(R * K, wl.h_v), dims.act_torch))
        prev = inp["accepted"][s - 1] if s > 0 else np.zeros(R, np.int32)
        r["acc"].copy_(torch.as_tensor(np.asarray(prev, np.int32)))
        r["par"].fill_((s + 1) & 1)
        r["o"].fill_(float("nan"))

    eager, graph, spare = make(), make(), make()
    load_step(spare, 0)
    _warm(lambda: call(spare))

    cg = torch.cuda.CUDAGraph()
    load_step(graph, 0)
    with torch.cuda.graph(cg):
        call(graph)

    for s in range(wl.n_steps):
        load_step(eager, s)
        load_step(graph, s)
        call(eager)
        cg.replay()
        torch.cuda.synchronize()
        assert not torch.isnan(eager["o"]).any(), s
        assert torch.equal(graph["o"], eager["o"]), s
        assert torch.equal(graph["pages"].buf, eager["pages"].buf), s
        assert torch.equal(graph["conv"].buf, eager["conv"].buf), s
        assert int(graph["err"].item()) == 0 and int(eager["err"].item()) == 0, s
        assert int(graph["conv"].sync.abs().sum()) == 0, s
