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
from gpu_util import DEV, dev, dims_of, gdn, make_batch, params_of

pytestmark = pytest.mark.gpu

N_SEQ_PAGES = 4      # pages 0..3: token-by-token sequences
N_REQ = 6            # pages 4..9: verify requests


def _workloads(state_dtype, seed):
    base = dict(h_k=4, h_v=8, d_k=128, d_v=128, conv_w=4, act_dtype=wk.BF16, state_dtype=state_dtype, seed=seed)
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


def _run(layout, state_dtype, fused):
    ws, wv = _workloads(state_dtype, seed=71)
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
            g.gdn_mixed_step(w.dims, w.params, seq=seq, verify=ver, err=w.err)
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


@pytest.mark.parametrize("state_dtype", [wk.F32, wk.BF16])
def test_mixed_step_equals_separate_launches(state_dtype):
    fused = _run(0, state_dtype, fused=True)
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
