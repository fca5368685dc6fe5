"""GPU tests of gdn_mixed_step: one launch for a step that mixes
token-by-token sequences with speculative verify requests gives the results
of the two separate launches (gdn_recurrent_seq, then gdn_spec_verify) bit
for bit -- outputs, states, conv windows and buffers, page headers and
records -- with both parts in one conv pool, over several steps, and with
either part absent."""
import numpy as np
import pytest
import torch

import gdn_workloads as wk
from gpu_util import DEV, dev, dims_of, gdn, host, make_batch, max_slice_rel_o, params_of

pytestmark = pytest.mark.gpu

N_SEQ_PAGES = 4      # pages 0..3: token-by-token sequences
N_REQ = 6            # pages 4..9: verify requests


def _workloads(state_dtype, seed, d_k=128, d_v=128):
    base = dict(h_k=4, h_v=8, d_k=d_k, d_v=d_v, conv_w=4, act_dtype=wk.BF16, state_dtype=state_dtype, seed=seed)
    ws = wk.Workload("mixed_seq", seqlens=(45, 83, 17, 1), **base)
    wv = wk.Workload("mixed_verify", n_req=N_REQ, n_cand=8, n_steps=3, **base)
    return ws, wv


class World:
    """Pools for one run: a shared conv pool (rows for verify), the sequence
    state pool, and one-page verify pages."""

    def __init__(self, ws, wv, si, vi, layout):
        g = gdn()
        self.g = g
        self.dims = dims_of(ws, n_spec=wv.n_cand - 1)
        n_pages = N_SEQ_PAGES + N_REQ
        self.conv = g.ConvPool.alloc(self.dims, n_pages, 3 + self.dims.n_spec, DEV)
        self.state = g.StatePool.alloc(self.dims, N_SEQ_PAGES, DEV)
        self.pages = g.SpecPages.alloc(self.dims, layout, n_pages, DEV)
        for s in range(N_SEQ_PAGES):
            self.conv.buf[s, :3] = dev(si["window0"][s], self.dims.act_torch)
            self.state.buf[s] = dev(si["S0"][s], self.dims.state_torch)
        st = self.pages.states()
        for r in range(N_REQ):
            p = N_SEQ_PAGES + r
            st[p, 0] = dev(wk.round_to(vi["S0"][r], ws.state_dtype), self.dims.state_torch)
            self.conv.buf[p, :3] = dev(vi["window0"][r], self.dims.act_torch)
        self.params = params_of(si, ws)
        self.err = torch.zeros(1, dtype=torch.int32, device=DEV)

    def snapshot(self):
        return [self.conv.buf.clone(), self.conv.sync.clone(), self.state.buf.clone(), self.pages.buf.clone(),
                self.err.clone()]


def _step_args(w, ws, wv, si, vi, step, seq_rows, seq_cu, pages, vstep):
    d = w.dims
    seq = None
    if seq_rows is not None:
        r0, r1 = seq_rows
        x = dev(si["x"][r0:r1], d.act_torch)
        a = dev(si["a"][r0:r1], d.act_torch)
        b = dev(si["b"][r0:r1], d.act_torch)
        batch = make_batch(seq_cu, pages, r1 - r0)
        o = torch.full((r1 - r0, ws.h_v, ws.d_v), float("nan"), device=DEV)
        seq = dict(x=x, a=a, b=b, batch=batch, conv=w.conv, state=w.state, o=o)
    ver = None
    if vstep is not None:
        s, acc = vstep
        R, K, C = N_REQ, wv.n_cand, ws.c_conv
        ver = dict(pages=w.pages, x=dev(vi["x"][s].reshape(R * K, C), d.act_torch),
                   a=dev(vi["a"][s].reshape(R * K, ws.h_v), d.act_torch),
                   b=dev(vi["b"][s].reshape(R * K, ws.h_v), d.act_torch), n_req=R, n_cand=K,
                   req_page=torch.arange(N_SEQ_PAGES, N_SEQ_PAGES + R, dtype=torch.int32, device=DEV),
                   num_accepted=torch.tensor(np.asarray(acc, np.int32), device=DEV),
                   step_parity=torch.full((R,), (step + 1) & 1, dtype=torch.uint8, device=DEV), conv=w.conv,
                   o=torch.full((R * K, ws.h_v, ws.d_v), float("nan"), device=DEV))
    return seq, ver


def _run(layout, state_dtype, fused, d_k=128, d_v=128, launches=0):
    ws, wv = _workloads(state_dtype, seed=71, d_k=d_k, d_v=d_v)
    si = wk.make_sequence_inputs(ws)
    vi = wk.make_verify_inputs(wv)
    w = World(ws, wv, si, vi, layout)
    g = w.g
    cu = si["cu_seqlens"]
    zero = np.zeros(N_REQ, np.int32)
    # decode rows for step 2: one more token per sequence, drawn from a second seeded batch
    ws2 = ws.replace(seqlens=(1, 1, 1, 1), seed=72)
    si2 = wk.make_sequence_inputs(ws2)
    plan = [  # (sequence rows and cu, inputs, verify step)
        ((0, int(cu[-1])), cu, si, (0, zero)),
        ((0, 4), si2["cu_seqlens"], si2, (1, vi["accepted"][0])),
        (None, None, None, (2, vi["accepted"][1])),
        ((0, 4), si2["cu_seqlens"], si2, None),
    ]
    outs = []
    for step, (rows, scu, sinp, vstep) in enumerate(plan):
        seq, ver = _step_args(w, ws, wv, sinp if sinp is not None else si, vi, step if vstep is None else vstep[0],
                              rows, scu, list(range(N_SEQ_PAGES)), vstep)
        if fused:
            g.gdn_mixed_step(w.dims, w.params, seq=seq, verify=ver, err=w.err, launches=launches)
        else:
            if seq is not None:
                g.gdn_recurrent_seq(w.dims, w.params, seq["x"], seq["a"], seq["b"], seq["batch"], w.conv, w.state,
                                    o=seq["o"], err=w.err)
            if ver is not None:
                g.gdn_spec_verify(w.dims, w.params, w.pages, ver["x"], ver["a"], ver["b"], ver["n_req"],
                                  ver["n_cand"], ver["req_page"], ver["num_accepted"], ver["step_parity"], w.conv,
                                  o=ver["o"], err=w.err)
        torch.cuda.synchronize()
        outs.append((None if seq is None else seq["o"].clone(), None if ver is None else ver["o"].clone(),
                     w.snapshot()))
    return outs


@pytest.mark.parametrize("launches", [0, 1, 2])
@pytest.mark.parametrize("state_dtype", [wk.F32, wk.BF16])
def test_mixed_step_equals_separate_launches(state_dtype, launches):
    """Every launch choice (the library's, one grid, two launches) gives the
    separate launches' results bit for bit; the step with decode rows is the
    one the library runs as two launches."""
    fused = _run(0, state_dtype, fused=True, launches=launches)
    sep = _run(0, state_dtype, fused=False)
    for step, ((so_f, vo_f, snap_f), (so_s, vo_s, snap_s)) in enumerate(zip(fused, sep)):
        for got, ref in ((so_f, so_s), (vo_f, vo_s)):
            assert (got is None) == (ref is None)
            if got is not None:
                assert not torch.isnan(got).any(), step
                assert torch.equal(got, ref), step
        for got, ref in zip(snap_f, snap_s):
            assert torch.equal(got, ref), step
        assert int(snap_f[4].item()) == 0          # no device error
        assert int(snap_f[1].abs().sum()) == 0     # sync words back to zero


def test_mixed_step_slots_layout():
    fused = _run(1, wk.F32, fused=True)
    sep = _run(1, wk.F32, fused=False)
    for (so_f, vo_f, snap_f), (so_s, vo_s, snap_s) in zip(fused, sep):
        for got, ref in ((so_f, so_s), (vo_f, vo_s)):
            if got is not None:
                assert torch.equal(got, ref)
        for got, ref in zip(snap_f, snap_s):
            assert torch.equal(got, ref)


def _prefill_then_verify(state_dtype, via_spec_pages, launches=0):
    """Prefill four sequences, then run verify steps on their pages.  Either
    the prefill writes straight into the speculative pages (state pool
    aliased onto the checkpoints, spec_pages set, headers left fresh), or it
    runs on a separate state pool whose states are copied into the pages and
    whose headers are zeroed by hand."""
    g = gdn()
    ws, wv = _workloads(state_dtype, seed=73)
    wv = wv.replace(n_req=4)
    si = wk.make_sequence_inputs(ws)
    vi = wk.make_verify_inputs(wv)
    dims = dims_of(ws, n_spec=wv.n_cand - 1)
    n = len(ws.seqlens)
    conv = g.ConvPool.alloc(dims, n, 3 + dims.n_spec, DEV)
    pages = g.SpecPages.alloc(dims, 0, n, DEV)
    pages.header()[:, :4] = torch.tensor([0x301, 5, 7, 3], dtype=torch.int32, device=DEV)  # a stale record
    for s in range(n):
        conv.buf[s, :3] = dev(si["window0"][s], dims.act_torch)
    params = params_of(si, ws)
    x, a, b = dev(si["x"], dims.act_torch), dev(si["a"], dims.act_torch), dev(si["b"], dims.act_torch)
    batch = make_batch(si["cu_seqlens"], list(range(n)), x.shape[0])
    o_pref = torch.full((x.shape[0], ws.h_v, ws.d_v), float("nan"), device=DEV)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    if via_spec_pages:
        state = pages.checkpoint_pool()
        state.buf.copy_(dev(si["S0"], dims.state_torch))
        g.gdn_mixed_step(dims, params, seq=dict(x=x, a=a, b=b, batch=batch, conv=conv, state=state, o=o_pref,
                                                spec_pages=pages), err=err, launches=launches)
    else:
        state = g.StatePool(dev(si["S0"], dims.state_torch))
        g.gdn_recurrent_seq(dims, params, x, a, b, batch, conv, state, o=o_pref, err=err)
        pages.states()[:, 0] = state.buf
        pages.header().zero_()
    outs = [o_pref.clone()]
    rp = torch.arange(n, dtype=torch.int32, device=DEV)
    R, K, C = n, wv.n_cand, ws.c_conv
    for step in range(wv.n_steps):
        acc = torch.tensor(np.asarray(vi["accepted"][step - 1] if step else np.zeros(R), np.int32), device=DEV)
        o = torch.full((R * K, ws.h_v, ws.d_v), float("nan"), device=DEV)
        g.gdn_spec_verify(dims, params, pages, dev(vi["x"][step].reshape(R * K, C), dims.act_torch),
                          dev(vi["a"][step].reshape(R * K, ws.h_v), dims.act_torch),
                          dev(vi["b"][step].reshape(R * K, ws.h_v), dims.act_torch), R, K, rp, acc,
                          torch.full((R,), (step + 1) & 1, dtype=torch.uint8, device=DEV), conv, o=o, err=err)
        outs.append(o.view(R, K, ws.h_v, ws.d_v).clone())
    g.gdn_spec_verify(dims, params, pages, None, None, None, R, 0, rp,
                      torch.tensor(np.asarray(vi["accepted"][wv.n_steps - 1], np.int32), device=DEV),
                      torch.full((R,), (wv.n_steps + 1) & 1, dtype=torch.uint8, device=DEV), conv, err=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    return outs, pages, conv, (ws, wv, si, vi)


@pytest.mark.parametrize("launches", [0, 2])
@pytest.mark.parametrize("state_dtype", [wk.F32, wk.BF16])
def test_prefill_into_spec_pages_equals_copy_and_zero(state_dtype, launches):
    """Also with two launches forced: the sequences then take the 32-column
    kernel, which leaves the page headers fresh as the one grid does."""
    got, pages_a, conv_a, _ = _prefill_then_verify(state_dtype, True, launches=launches)
    ref, pages_b, conv_b, _ = _prefill_then_verify(state_dtype, False)
    for g_, r_ in zip(got, ref):
        assert not torch.isnan(g_).any()
        assert torch.equal(g_, r_)
    assert torch.equal(pages_a.buf, pages_b.buf)
    assert torch.equal(conv_a.buf, conv_b.buf)


def test_prefill_into_spec_pages_oracle_parity(ora):
    """Prefill through the mixed step into the pages, then verify steps:
    against the oracle's layer on the prefill followed by its verify
    semantics from the prefill's final state and window (1e-4)."""
    outs, pages, conv, (ws, wv, si, vi) = _prefill_then_verify(wk.F32, True)
    dm = ora.dims_of(ws)
    o_ref, win, S = ora.layer(dm, si["conv_w"], si["a_log"], si["dt_bias"], si["x"], si["a"], si["b"],
                              si["cu_seqlens"], si["window0"], si["S0"])
    vo_ref, win2, S2 = ora.verify(dm, vi["conv_w"], vi["a_log"], vi["dt_bias"], vi["x"], vi["a"], vi["b"],
                                  vi["accepted"], win, S)
    from gpu_util import host, max_slice_rel_o
    assert max_slice_rel_o(host(outs[0]), o_ref, si["cu_seqlens"]) <= 1e-4
    got = np.stack([host(t) for t in outs[1:]])       # [steps][req][cand][h_v][d_v]
    worst = 0.0
    for r in range(wv.n_req):
        for h in range(ws.h_v):
            ref = vo_ref[:, r, :, h]
            worst = max(worst, np.abs(got[:, r, :, h] - ref).max() / np.abs(ref).max())
    assert worst <= 1e-4, worst
    St = host(pages.states()[:, 0])
    for r in range(wv.n_req):
        for h in range(ws.h_v):
            assert np.abs(St[r, h] - S2[r, h]).max() / np.abs(S2[r, h]).max() <= 1e-4
    np.testing.assert_array_equal(host(conv.buf[:, :3]), win2)


def test_spec_pages_empty_sequence_keeps_its_header():
    """A sequence of length 0 is a no-op: its page keeps its header (and its
    record) while the other sequences' pages are left fresh."""
    g = gdn()
    ws, _ = _workloads(wk.F32, seed=74)
    ws = ws.replace(seqlens=(20, 0, 5))
    si = wk.make_sequence_inputs(ws)
    dims = dims_of(ws, n_spec=7)
    n = 3
    conv = g.ConvPool.alloc(dims, n, 3 + dims.n_spec, DEV)
    pages = g.SpecPages.alloc(dims, 0, n, DEV)
    stale = torch.tensor([0x301, 5, 7, 3], dtype=torch.int32, device=DEV)
    pages.header()[:, :4] = stale
    state = pages.checkpoint_pool()
    state.buf.copy_(dev(si["S0"], dims.state_torch))
    before = pages.buf[1].clone()
    x, a, b = dev(si["x"], dims.act_torch), dev(si["a"], dims.act_torch), dev(si["b"], dims.act_torch)
    batch = make_batch(si["cu_seqlens"], list(range(n)), x.shape[0])
    o = torch.full((x.shape[0], ws.h_v, ws.d_v), float("nan"), device=DEV)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    g.gdn_mixed_step(dims, params_of(si, ws), seq=dict(x=x, a=a, b=b, batch=batch, conv=conv, state=state, o=o,
                                                       spec_pages=pages), err=err)
    torch.cuda.synchronize()
    h = pages.header()
    assert int(h[0, :4].abs().sum()) == 0 and int(h[2, :4].abs().sum()) == 0
    assert torch.equal(pages.buf[1], before)
    assert int(err.item()) == 0 and not torch.isnan(o).any()


@pytest.mark.parametrize("d_k,d_v", [(64, 96), (32, 32)])
def test_mixed_step_small_head_dims(d_k, d_v):
    """The mixed kernel's instantiations with 32-column verify blocks
    (d_v not a multiple of 128), including d_k = 32."""
    fused = _run(0, wk.F32, True, d_k, d_v)
    sep = _run(0, wk.F32, False, d_k, d_v)
    for (so_f, vo_f, snap_f), (so_s, vo_s, snap_s) in zip(fused, sep):
        for got, ref in ((so_f, so_s), (vo_f, vo_s)):
            if got is not None:
                assert not torch.isnan(got).any()
                assert torch.equal(got, ref)
        for got, ref in zip(snap_f, snap_s):
            assert torch.equal(got, ref)


def test_mixed_step_at_the_benchmark_shape(ora):
    """The benchmark's mix: the full short-prefill batch (8 sequences, 2,159
    rows) with 32 one-page verify requests of 8 candidates, H_k = 16,
    H_v = 32, d = 128, in one launch, equals the two separate launches bit
    for bit: outputs, states, pages and the shared conv pool.  Two such
    steps (the sequences continue with the same rows, the verify requests
    replay their first step's accepted rows) match the oracle: its layer
    twice over the batch, and its verify semantics for the requests
    (1e-4)."""
    g = gdn()
    ws = wk.SHORT_PREFILL
    wv = wk.SPEC_VERIFY
    si, vi = wk.make_sequence_inputs(ws), wk.make_verify_inputs(wv)
    dims = dims_of(ws, n_spec=wv.n_cand - 1)
    NS, R, K, C = len(ws.seqlens), wv.n_req, wv.n_cand, ws.c_conv
    params = params_of(si, ws)
    x, a, b = dev(si["x"], dims.act_torch), dev(si["a"], dims.act_torch), dev(si["b"], dims.act_torch)
    batch = make_batch(si["cu_seqlens"], list(range(NS)), x.shape[0])
    rp = torch.arange(NS, NS + R, dtype=torch.int32, device=DEV)

    def vstep(step):
        """Step `step` of the verify workload: candidates, the previous
        step's acceptance counts (the second step replays), parity."""
        prev = vi["accepted"][step - 1] if step > 0 else np.zeros(R, np.int32)
        return (dev(vi["x"][step].reshape(R * K, C), dims.act_torch),
                dev(vi["a"][step].reshape(R * K, ws.h_v), dims.act_torch),
                dev(vi["b"][step].reshape(R * K, ws.h_v), dims.act_torch),
                torch.tensor(np.asarray(prev, np.int32), device=DEV),
                torch.full((R,), (step + 1) & 1, dtype=torch.uint8, device=DEV))

    def world():
        conv = g.ConvPool.alloc(dims, NS + R, 3 + dims.n_spec, DEV)
        state = g.StatePool(dev(si["S0"], dims.state_torch))
        pages = g.SpecPages.alloc(dims, 0, NS + R, DEV)
        conv.buf[:NS, :3] = dev(si["window0"], dims.act_torch)
        conv.buf[NS:, :3] = dev(vi["window0"], dims.act_torch)
        pages.states()[NS:, 0] = dev(vi["S0"], dims.state_torch)
        o_s = torch.full((x.shape[0], ws.h_v, ws.d_v), float("nan"), device=DEV)
        o_v = torch.full((R * K, ws.h_v, ws.d_v), float("nan"), device=DEV)
        err = torch.zeros(1, dtype=torch.int32, device=DEV)
        return conv, state, pages, o_s, o_v, err

    fused, sep = world(), world()
    outs = []
    for step in (0, 1):
        vx, va, vb, acc, par = vstep(step)
        conv, state, pages, o_s, o_v, err = fused
        g.gdn_mixed_step(dims, params, seq=dict(x=x, a=a, b=b, batch=batch, conv=conv, state=state, o=o_s),
                         verify=dict(pages=pages, x=vx, a=va, b=vb, n_req=R, n_cand=K, req_page=rp,
                                     num_accepted=acc, step_parity=par, conv=conv, o=o_v), err=err)
        conv, state, pages, o_s, o_v, err = sep
        g.gdn_recurrent_seq(dims, params, x, a, b, batch, conv, state, o=o_s, err=err)
        g.gdn_spec_verify(dims, params, pages, vx, va, vb, R, K, rp, acc, par, conv, o=o_v, err=err)
        torch.cuda.synchronize()
        for got, ref in zip(fused, sep):
            t_got = got.buf if hasattr(got, "buf") else got
            t_ref = ref.buf if hasattr(ref, "buf") else ref
            assert torch.equal(t_got, t_ref), step
        assert not torch.isnan(fused[3]).any() and not torch.isnan(fused[4]).any(), step
        assert int(fused[5].item()) == 0, step
        assert int(fused[0].sync.abs().sum()) == 0, step
        outs.append((host(fused[3]), host(fused[4]).reshape(R, K, ws.h_v, ws.d_v)))
    # the oracle: the layer twice over the batch, and two verify steps
    from gpu_util import max_slice_rel_S, oracle_seq
    dm = ora.dims_of(ws)
    cu = si["cu_seqlens"]
    o1, win1, S1 = oracle_seq(ora, ws, si)
    o2, win2, S2 = ora.layer(dm, si["conv_w"], si["a_log"], si["dt_bias"], si["x"], si["a"], si["b"], cu, win1, S1)
    for got, ref in ((outs[0][0], o1), (outs[1][0], o2)):
        assert max_slice_rel_o(got, ref, cu) <= 1e-4
    conv, state = fused[0], fused[1]
    assert max_slice_rel_S(host(state.buf), S2) <= 1e-4
    np.testing.assert_array_equal(host(conv.buf[:NS, :3]), win2)
    # one layer: both parts run with the sequence workload's conv weights and gates
    vo, _, _ = ora.verify(dm, si["conv_w"], si["a_log"], si["dt_bias"], vi["x"][:2], vi["a"][:2], vi["b"][:2],
                          vi["accepted"][:2], vi["window0"], vi["S0"])
    worst = 0.0
    for step in (0, 1):
        for r in range(R):
            for h in range(ws.h_v):
                ref = vo[step, r, :, h]
                worst = max(worst, np.abs(outs[step][1][r, :, h] - ref).max() / np.abs(ref).max())
    assert worst <= 1e-4, worst


def test_mixed_step_launch_choice_at_decode_and_prefill_shapes():
    """The library picks two launches for a step whose sequences have at
    most four rows each beside verify requests, one launch otherwise."""
    g = gdn()
    ws, wv = _workloads(wk.F32, seed=75)
    si = wk.make_sequence_inputs(ws.replace(seqlens=(1, 5, 2, 3)))
    vi = wk.make_verify_inputs(wv)
    w = World(ws, wv, wk.make_sequence_inputs(ws), vi, 0)
    for lens, want in (((1, 4, 2, 3), g.GDN_MIXED_TWO_LAUNCHES), ((1, 5, 2, 3), g.GDN_MIXED_ONE_LAUNCH)):
        cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
        seq, ver = _step_args(w, ws, wv, si, vi, 0, (0, int(cu[-1])), cu, list(range(N_SEQ_PAGES)),
                              (0, np.zeros(N_REQ, np.int32)))
        assert g.gdn_mixed_launches(w.dims, seq=seq, verify=ver) == want, lens
        assert g.gdn_mixed_launches(w.dims, seq=seq) == g.GDN_MIXED_ONE_LAUNCH
