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


def test_mixed_steps_replayed_from_a_graph_equal_eager_launches():
    """One launch mixing four decode sequences (a token each) with six
    one-page verify requests in a shared conv pool, captured once and
    replayed for three steps with new tokens, candidates, acceptance counts
    and parity written in between."""
    g = gdn()
    base = dict(h_k=4, h_v=8, d_k=128, d_v=128, conv_w=4, act_dtype=wk.BF16, state_dtype=wk.F32, seed=44)
    ws = wk.Workload("graph_mixed_seq", seqlens=(1, 1, 1, 1), **base)
    wv = wk.Workload("graph_mixed_verify", n_req=6, n_cand=8, n_steps=3, **base)
    si, vi = wk.make_sequence_inputs(ws), wk.make_verify_inputs(wv)
    dims = dims_of(ws, n_spec=wv.n_cand - 1)
    NS, R, K, C = len(ws.seqlens), wv.n_req, wv.n_cand, ws.c_conv
    params = params_of(si, ws)
    batch = make_batch(si["cu_seqlens"], list(range(NS)), NS)
    req_page = torch.arange(NS, NS + R, dtype=torch.int32, device=DEV)
    tokens = [wk.make_sequence_inputs(ws.replace(seed=ws.seed + 300 + s)) for s in range(wv.n_steps)]
    act = dims.act_torch

    def make():
        conv = g.ConvPool.alloc(dims, NS + R, 3 + dims.n_spec, DEV)
        state = g.StatePool.alloc(dims, NS, DEV)
        pages = g.SpecPages.alloc(dims, 0, NS + R, DEV)
        for s in range(NS):
            conv.buf[s, :3] = dev(si["window0"][s], act)
            state.buf[s] = dev(si["S0"][s], dims.state_torch)
        st = pages.states()
        for r in range(R):
            st[NS + r, 0] = dev(vi["S0"][r], dims.state_torch)
            conv.buf[NS + r, :3] = dev(vi["window0"][r], act)
        seq = dict(x=torch.empty((NS, C), dtype=act, device=DEV), a=torch.empty((NS, ws.h_v), dtype=act, device=DEV),
                   b=torch.empty((NS, ws.h_v), dtype=act, device=DEV), batch=batch, conv=conv, state=state,
                   o=torch.empty((NS, ws.h_v, ws.d_v), device=DEV))
        ver = dict(pages=pages, x=torch.empty((R * K, C), dtype=act, device=DEV),
                   a=torch.empty((R * K, ws.h_v), dtype=act, device=DEV),
                   b=torch.empty((R * K, ws.h_v), dtype=act, device=DEV), n_req=R, n_cand=K, req_page=req_page,
                   num_accepted=torch.zeros(R, dtype=torch.int32, device=DEV),
                   step_parity=torch.zeros(R, dtype=torch.uint8, device=DEV), conv=conv,
                   o=torch.empty((R * K, ws.h_v, ws.d_v), device=DEV))
        return dict(seq=seq, ver=ver, err=torch.zeros(1, dtype=torch.int32, device=DEV))

    def call(w):
        g.gdn_mixed_step(dims, params, seq=w["seq"], verify=w["ver"], err=w["err"])

    def load(w, s):
        sq, vr, f = w["seq"], w["ver"], tokens[s]
        for k in ("x", "a", "b"):
            sq[k].copy_(dev(f[k], act))
        vr["x"].copy_(dev(vi["x"][s].reshape(R * K, C), act))
        vr["a"].copy_(dev(vi["a"][s].reshape(R * K, ws.h_v), act))
        vr["b"].copy_(dev(vi["b"][s].reshape(R * K, ws.h_v), act))
        prev = vi["accepted"][s - 1] if s > 0 else np.zeros(R, np.int32)
        vr["num_accepted"].copy_(torch.as_tensor(np.asarray(prev, np.int32)))
        vr["step_parity"].fill_((s + 1) & 1)
        sq["o"].fill_(float("nan"))
        vr["o"].fill_(float("nan"))

    eager, graph, spare = make(), make(), make()
    load(spare, 0)
    _warm(lambda: call(spare))
    load(graph, 0)
    cg = torch.cuda.CUDAGraph()
    with torch.cuda.graph(cg):
        call(graph)

    for s in range(wv.n_steps):
        load(eager, s)
        load(graph, s)
        call(eager)
        cg.replay()
        torch.cuda.synchronize()
        for part in ("seq", "ver"):
            assert not torch.isnan(eager[part]["o"]).any(), (s, part)
            assert torch.equal(graph[part]["o"], eager[part]["o"]), (s, part)
        assert torch.equal(graph["seq"]["state"].buf, eager["seq"]["state"].buf), s
        assert torch.equal(graph["ver"]["pages"].buf, eager["ver"]["pages"].buf), s
        assert torch.equal(graph["seq"]["conv"].buf, eager["seq"]["conv"].buf), s
        assert int(graph["err"].item()) == 0 and int(eager["err"].item()) == 0, s
        assert int(graph["seq"]["conv"].sync.abs().sum()) == 0, s
