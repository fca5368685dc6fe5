"""GPU tests of speculative verify (gdn_spec_verify): the one-page record
design against the per-candidate-slot design (bit-exact, fp32 state first,
then bf16), both against the oracle's verify semantics, the flag-word and
record bookkeeping against the oracle's bookkeeping model after every step,
and the device error paths."""
import numpy as np
import pytest
import torch

import gdn_workloads as wk
from gpu_util import DEV, VerifyRun, dev, gdn, host, run_seq

pytestmark = pytest.mark.gpu

ONEPAGE, SLOTS = 0, 1


def _inputs(wl, state_dtype):
    inp = wk.make_verify_inputs(wl)
    inp["S0"] = wk.round_to(inp["S0"], state_dtype)
    return inp


def _small(**kw):
    base = dict(n_req=6, n_steps=5, seed=31)
    base.update(kw)
    return wk.SPEC_VERIFY.replace(**base)


@pytest.mark.parametrize("state_dtype", [wk.F32, wk.BF16])  # fp32 first: it exposes 1-ulp differences
def test_onepage_equals_slots_bit_exact(state_dtype):
    wl = wk.SPEC_VERIFY
    inp = _inputs(wl, state_dtype)
    one = VerifyRun(wl, inp, ONEPAGE, state_dtype)
    slots = VerifyRun(wl, inp, SLOTS, state_dtype)
    o1, o2 = one.run(), slots.run()
    assert not torch.isnan(o1).any()
    assert torch.equal(o1, o2)
    assert torch.equal(one.committed_state(), slots.committed_state())
    assert torch.equal(one.conv.buf, slots.conv.buf)
    assert int(one.err.item()) == 0 and int(slots.err.item()) == 0
    assert int(one.conv.sync.abs().sum()) == 0 and int(slots.conv.sync.abs().sum()) == 0


@pytest.mark.parametrize("state_dtype,tol", [(wk.F32, 1e-4), (wk.BF16, 3e-3)])
def test_verify_oracle_parity(ora, state_dtype, tol):
    wl = wk.SPEC_VERIFY
    inp = _inputs(wl, state_dtype)
    run = VerifyRun(wl, inp, ONEPAGE, state_dtype)
    o = host(run.run())
    dm = ora.dims_of(wl)
    o_ref, win_ref, S_ref = ora.verify(dm, inp["conv_w"], inp["a_log"], inp["dt_bias"], inp["x"], inp["a"],
                                       inp["b"], inp["accepted"], inp["window0"], inp["S0"],
                                       state_bf16=(state_dtype == wk.BF16))
    worst = 0.0
    for r in range(wl.n_req):
        for h in range(wl.h_v):
            y, ref = o[:, r, :, h], o_ref[:, r, :, h]
            worst = max(worst, float(np.abs(y - ref).max() / np.abs(ref).max()))
    assert worst <= tol, worst
    S = host(run.committed_state())
    worstS = max(float(np.abs(S[r, h] - S_ref[r, h]).max() / np.abs(S_ref[r, h]).max())
                 for r in range(wl.n_req) for h in range(wl.h_v))
    assert worstS <= tol, worstS
    np.testing.assert_array_equal(host(run.committed_window()), win_ref)


def test_header_bookkeeping(ora):
    """After every step the headers (flag word, n_rows, acceptance echo) and
    every page's whole conv buffer equal the oracle's bookkeeping model bit
    for bit (VerifyRun.step checks them), and the record slot the step wrote
    holds its candidates: a and b exactly, the post-conv q|k|v within fp32
    rounding of the oracle's conv + SiLU from the step's window."""
    wl = _small()
    inp = _inputs(wl, wk.F32)
    run = VerifyRun(wl, inp, ONEPAGE, wk.F32)
    lay = run.pages.lay
    row = lay["record_row_bytes"] // 4
    C, K = wl.c_conv, wl.n_cand
    for s in range(wl.n_steps):
        prev = inp["accepted"][s - 1] if s > 0 else np.zeros(wl.n_req, np.int32)
        cbuf_before, hdr_before = run.book.cbuf.copy(), run.book.hdr.copy()
        run.step(s, prev)
        for r, p in enumerate(run.req_page):
            held = int(hdr_before[p, 1 + (int(hdr_before[p, 0]) & 1)])
            a_rep = int(prev[r]) if held > 0 else 0
            y_ref, _ = ora.conv_seq(inp["x"][s][r], inp["conv_w"], cbuf_before[p, a_rep:a_rep + 3])
            slot = int(run.book.hdr[p, 0]) & 1
            assert int(run.book.hdr[p, 1 + slot]) == K
            rec = run.pages.buf[p, lay["record_off"]:].view(torch.float32)
            got = host(rec[slot * K * row:(slot + 1) * K * row].view(K, row))
            np.testing.assert_array_equal(got[:, C:C + wl.h_v], inp["a"][s][r])
            np.testing.assert_array_equal(got[:, C + wl.h_v:C + 2 * wl.h_v], inp["b"][s][r])
            rel_rows = np.abs(got[:, :C] - y_ref).max(axis=1) / np.abs(y_ref).max(axis=1)
            assert rel_rows.max() <= 1e-5, (s, r, rel_rows.max())


def test_all_accepted_chain_equals_sequence_kernel():
    """With every draft accepted, verify's outputs are the token-by-token
    kernel's outputs on the concatenated stream, bit for bit (fp32 state)."""
    wl = _small(n_req=4)
    inp = _inputs(wl, wk.F32)
    inp["accepted"][:] = wl.n_cand - 1
    run = VerifyRun(wl, inp, ONEPAGE, wk.F32)
    o_ver = run.run()
    T = wl.n_steps * wl.n_cand
    sw = wk.DECODE.replace(seqlens=(T,) * wl.n_req)
    sinp = {"conv_w": inp["conv_w"], "a_log": inp["a_log"], "dt_bias": inp["dt_bias"],
            "S0": inp["S0"], "window0": inp["window0"],
            "x": inp["x"].transpose(1, 0, 2, 3).reshape(-1, wl.c_conv),
            "a": inp["a"].transpose(1, 0, 2, 3).reshape(-1, wl.h_v),
            "b": inp["b"].transpose(1, 0, 2, 3).reshape(-1, wl.h_v),
            "cu_seqlens": np.arange(wl.n_req + 1, dtype=np.int32) * T}
    o_seq, conv_seq, st_seq = run_seq(sw, sinp)
    o_seq = o_seq.view(wl.n_req, wl.n_steps, wl.n_cand, wl.h_v, wl.d_v).transpose(0, 1)
    assert torch.equal(o_ver, o_seq)
    assert torch.equal(run.committed_state(), st_seq.buf)
    assert torch.equal(run.committed_window(), conv_seq.buf)


def test_lockstep_copies_equal_lone_request():
    wl = _small(n_req=3)
    inp = _inputs(wl, wk.BF16)
    for k in ("S0", "window0"):
        inp[k][1:] = inp[k][:1]
    for k in ("x", "a", "b"):
        inp[k][:, 1:] = inp[k][:, :1]
    inp["accepted"][:, 1:] = inp["accepted"][:, :1]
    o3 = VerifyRun(wl, inp, ONEPAGE, wk.BF16).run()
    lone = wl.replace(n_req=1)
    inp1 = {k: (v[:1] if k in ("S0", "window0") else v[:, :1] if k in ("x", "a", "b", "accepted") else v)
            for k, v in inp.items()}
    o1 = VerifyRun(lone, inp1, ONEPAGE, wk.BF16).run()
    for r in range(3):
        assert torch.equal(o3[:, r], o1[:, 0])


def test_relaunch_and_bad_acceptance_are_rejected():
    g = gdn()
    wl = _small(n_req=3)
    inp = _inputs(wl, wk.F32)
    run = VerifyRun(wl, inp, ONEPAGE, wk.F32)
    run.step(0, np.zeros(3, np.int32))
    snap = run.pages.buf.clone(), run.conv.buf.clone()
    # the same step again (same parity) is refused and changes nothing (the
    # bookkeeping model refuses it too: VerifyRun.step compares the two)
    run.step(1, np.zeros(3, np.int32), parity=1)
    assert int(run.err.item()) & g.GDN_DEVERR_PARITY
    assert torch.equal(run.pages.buf, snap[0]) and torch.equal(run.conv.buf, snap[1])
    run.clear_err()
    # an acceptance beyond the record's rows is refused
    run.step(1, np.array([0, wl.n_cand, 1], np.int32))
    assert int(run.err.item()) & g.GDN_DEVERR_ACCEPTED
    hdr = run.pages.header().cpu().numpy()
    assert hdr[1, 0] == snap[0][1, :4].view(torch.int32)[0].item()   # request 1 untouched
    assert hdr[0, 0] != snap[0][0, :4].view(torch.int32)[0].item()   # the others advanced


def test_padding_requests_are_skipped():
    wl = _small(n_req=4)
    inp = _inputs(wl, wk.F32)
    run = VerifyRun(wl, inp, ONEPAGE, wk.F32, pages_of=[2, -1, 0, 3], n_pages=5)
    before = run.pages.buf.clone()
    o = run.step(0, np.zeros(4, np.int32))
    assert torch.isnan(o[1]).all() and not torch.isnan(o[0]).any()
    assert torch.equal(run.pages.buf[1], before[1]) and torch.equal(run.pages.buf[4], before[4])


@pytest.mark.parametrize("state_dtype", [wk.F32, wk.BF16])
def test_prefix_snapshot_after_commit_continues_bit_identically(ora, state_dtype):
    """One page per request with a prefix cache ("r9700-stack v0.2.4" leaves
    prefix caching to the stock pages): after a commit-only step the
    checkpoint and conv rows 0..2 hold the committed prefix and the record is
    empty, so a cached copy of them, restored into fresh pages (all-zero
    header), continues exactly as the original request does."""
    wl = _small(n_steps=8)
    inp = _inputs(wl, state_dtype)
    zero = np.zeros(wl.n_req, np.int32)
    A = VerifyRun(wl, inp, ONEPAGE, state_dtype)
    for s in range(4):
        A.step(s, inp["accepted"][s - 1] if s else zero)
    A.step(0, inp["accepted"][3], n_cand=0)              # commit: the prefix cache point
    cached_S = A.committed_state().clone()
    cached_W = A.committed_window().clone()
    hdr = A.pages.header()[A.req_page]
    assert int(hdr[:, 1 + (int(hdr[0, 0]) & 1)].abs().sum()) == 0   # the live record holds no rows
    # the cached prefix is the oracle's committed state and window after four steps
    dm = ora.dims_of(wl)
    _, win_ref, S_ref = ora.verify(dm, inp["conv_w"], inp["a_log"], inp["dt_bias"], inp["x"][:4], inp["a"][:4],
                                   inp["b"][:4], inp["accepted"][:4], inp["window0"], inp["S0"],
                                   state_bf16=(state_dtype == wk.BF16))
    np.testing.assert_array_equal(host(cached_W), win_ref)
    Sc = host(cached_S)
    tol = 1e-4 if state_dtype == wk.F32 else 3e-3
    for r in range(wl.n_req):
        for h in range(wl.h_v):
            assert np.abs(Sc[r, h] - S_ref[r, h]).max() <= tol * np.abs(S_ref[r, h]).max(), (r, h)
    B = VerifyRun(wl, inp, ONEPAGE, state_dtype)
    B.pages.states()[B.req_page, 0] = cached_S
    B.conv.buf[B.req_page, :3] = cached_W
    B.book.cbuf[B.req_page, :3] = host(cached_W)
    for s in range(4, 8):
        prev = inp["accepted"][s - 1] if s > 4 else zero
        oa, ob = A.step(s, prev), B.step(s, prev)
        assert torch.equal(oa, ob), s
    A.step(0, inp["accepted"][7], n_cand=0)
    B.step(0, inp["accepted"][7], n_cand=0)
    assert torch.equal(A.committed_state(), B.committed_state())
    assert torch.equal(A.committed_window(), B.committed_window())
    assert int(A.err.item()) == 0 and int(B.err.item()) == 0


@pytest.mark.parametrize("n_cand", [12, 16])
def test_more_candidates_than_half_the_token_rows(ora, n_cand):
    """Steps whose candidates (or replayed rows) exceed half of the kernel's
    16 token rows run the replay and the candidates through the same rows
    one after the other, up to the page layout's maximum of 16 candidates:
    one-page equals slots bit for bit and the oracle within 1e-4."""
    wl = _small(n_req=4, n_steps=5, n_cand=n_cand, seed=37)
    inp = _inputs(wl, wk.F32)
    inp["accepted"][1] = n_cand - 1          # a full-length replay in step 2
    one = VerifyRun(wl, inp, ONEPAGE, wk.F32)
    o1 = one.run()
    slots = VerifyRun(wl, inp, SLOTS, wk.F32)
    o2 = slots.run()
    assert torch.equal(o1, o2)
    assert torch.equal(one.committed_state(), slots.committed_state())
    assert torch.equal(one.committed_window(), slots.committed_window())
    dm = ora.dims_of(wl)
    o_ref, win_ref, S_ref = ora.verify(dm, inp["conv_w"], inp["a_log"], inp["dt_bias"], inp["x"], inp["a"],
                                       inp["b"], inp["accepted"], inp["window0"], inp["S0"])
    o = host(o1)
    worst = max(float(np.abs(o[:, r, :, h] - o_ref[:, r, :, h]).max() / np.abs(o_ref[:, r, :, h]).max())
                for r in range(wl.n_req) for h in range(wl.h_v))
    assert worst <= 1e-4, worst
    S = host(one.committed_state())
    worstS = max(float(np.abs(S[r, h] - S_ref[r, h]).max() / np.abs(S_ref[r, h]).max())
                 for r in range(wl.n_req) for h in range(wl.h_v))
    assert worstS <= 1e-4, worstS
    np.testing.assert_array_equal(host(one.committed_window()), win_ref)
    assert int(one.err.item()) == 0 and int(slots.err.item()) == 0


@pytest.mark.parametrize("state_dtype", [wk.F32, wk.BF16])
@pytest.mark.parametrize("d_k,d_v", [(64, 96), (32, 32)])
def test_other_head_dims(ora, d_k, d_v, state_dtype):
    """Head dims other than 128: d_k = 64 and 32 with value blocks of 32
    columns (d_v not a multiple of 128), one-page equals slots bit for bit
    and the oracle within 1e-4 (3e-3 with bf16 checkpoints)."""
    wl = _small(n_req=3, n_steps=4, h_k=2, h_v=4, d_k=d_k, d_v=d_v, seed=39, state_dtype=state_dtype)
    inp = _inputs(wl, state_dtype)
    one = VerifyRun(wl, inp, ONEPAGE, state_dtype)
    o1 = one.run()
    slots = VerifyRun(wl, inp, SLOTS, state_dtype)
    assert torch.equal(o1, slots.run())
    assert torch.equal(one.committed_state(), slots.committed_state())
    dm = ora.dims_of(wl)
    o_ref, win_ref, S_ref = ora.verify(dm, inp["conv_w"], inp["a_log"], inp["dt_bias"], inp["x"], inp["a"],
                                       inp["b"], inp["accepted"], inp["window0"], inp["S0"],
                                       state_bf16=(state_dtype == wk.BF16))
    o = host(o1)
    worst = max(float(np.abs(o[:, r, :, h] - o_ref[:, r, :, h]).max() / np.abs(o_ref[:, r, :, h]).max())
                for r in range(wl.n_req) for h in range(wl.h_v))
    assert worst <= (1e-4 if state_dtype == wk.F32 else 3e-3), worst
    np.testing.assert_array_equal(host(one.committed_window()), win_ref)


def test_fp32_activations(ora):
    """fp32 activations (x, a, b, conv weights and buffer): one-page equals
    slots bit for bit and the oracle within 1e-4."""
    wl = _small(n_req=3, n_steps=4, h_k=2, h_v=4, act_dtype=wk.F32, seed=41)
    inp = _inputs(wl, wk.F32)
    one = VerifyRun(wl, inp, ONEPAGE, wk.F32)
    o1 = one.run()
    slots = VerifyRun(wl, inp, SLOTS, wk.F32)
    assert torch.equal(o1, slots.run())
    dm = ora.dims_of(wl)
    o_ref, win_ref, S_ref = ora.verify(dm, inp["conv_w"], inp["a_log"], inp["dt_bias"], inp["x"], inp["a"],
                                       inp["b"], inp["accepted"], inp["window0"], inp["S0"])
    o = host(o1)
    worst = max(float(np.abs(o[:, r, :, h] - o_ref[:, r, :, h]).max() / np.abs(o_ref[:, r, :, h]).max())
                for r in range(wl.n_req) for h in range(wl.h_v))
    assert worst <= 1e-4, worst
    np.testing.assert_array_equal(host(one.committed_window()), win_ref)


def test_candidate_count_varies_between_steps(ora):
    """Steps with 8, 3, 1, 8 and 5 candidates: the conv buffer rolls by the
    width the record holds, not by the current step's ("A defect found and
    fixed before the tag" of "r9700-stack v0.2.4").  Checked against the
    oracle run one step at a time from each step's committed state and
    window, and one-page against slots bit for bit."""
    Ks = (8, 3, 1, 8, 5)
    wl = _small(n_req=3, n_steps=len(Ks), seed=43)
    inp = _inputs(wl, wk.F32)
    rng = np.random.default_rng(43)
    acc = np.stack([rng.integers(0, K, size=wl.n_req) for K in Ks]).astype(np.int32)
    runs = {lay: VerifyRun(wl, inp, lay, wk.F32) for lay in (ONEPAGE, SLOTS)}
    outs = {lay: [] for lay in runs}
    zero = np.zeros(wl.n_req, np.int32)
    for s, K in enumerate(Ks):
        for lay, run in runs.items():
            outs[lay].append(host(run.step(s, acc[s - 1] if s else zero, n_cand=K)))
    for run in runs.values():
        run.step(0, acc[-1], n_cand=0)
    for a, b in zip(outs[ONEPAGE], outs[SLOTS]):
        assert np.array_equal(a, b)
    dm = ora.dims_of(wl)
    win, S = inp["window0"], inp["S0"]
    for s, K in enumerate(Ks):
        o_ref, win, S = ora.verify(dm, inp["conv_w"], inp["a_log"], inp["dt_bias"], inp["x"][s:s + 1, :, :K],
                                   inp["a"][s:s + 1, :, :K], inp["b"][s:s + 1, :, :K], acc[s:s + 1], win, S)
        got = outs[ONEPAGE][s]
        for r in range(wl.n_req):
            for h in range(wl.h_v):
                ref = o_ref[0, r, :, h]
                assert np.abs(got[r, :, h] - ref).max() <= 1e-4 * np.abs(ref).max(), (s, r, h)
    one = runs[ONEPAGE]
    np.testing.assert_array_equal(host(one.committed_window()), win)
    Sg = host(one.committed_state())
    for r in range(wl.n_req):
        for h in range(wl.h_v):
            assert np.abs(Sg[r, h] - S[r, h]).max() <= 1e-4 * np.abs(S[r, h]).max()
    assert int(one.err.item()) == 0


@pytest.mark.parametrize("h_k,h_v", [(4, 4), (2, 8)])
def test_gqa_ratios(ora, h_k, h_v):
    """One and four value heads per key head (the workloads use two): the
    key-head mapping, the q/k record rows written by one workgroup per key
    head and the window hand-off after r arrivals; one-page equals slots bit
    for bit and the oracle within 1e-4."""
    wl = _small(n_req=3, n_steps=4, h_k=h_k, h_v=h_v, seed=47)
    inp = _inputs(wl, wk.F32)
    one = VerifyRun(wl, inp, ONEPAGE, wk.F32)
    o1 = one.run()
    slots = VerifyRun(wl, inp, SLOTS, wk.F32)
    assert torch.equal(o1, slots.run())
    assert torch.equal(one.committed_state(), slots.committed_state())
    dm = ora.dims_of(wl)
    o_ref, win_ref, S_ref = ora.verify(dm, inp["conv_w"], inp["a_log"], inp["dt_bias"], inp["x"], inp["a"],
                                       inp["b"], inp["accepted"], inp["window0"], inp["S0"])
    o = host(o1)
    worst = max(float(np.abs(o[:, r, :, h] - o_ref[:, r, :, h]).max() / np.abs(o_ref[:, r, :, h]).max())
                for r in range(wl.n_req) for h in range(wl.h_v))
    assert worst <= 1e-4, worst
    np.testing.assert_array_equal(host(one.committed_window()), win_ref)
    assert int(one.err.item()) == 0 and int(one.conv.sync.abs().sum()) == 0


@pytest.mark.parametrize("state_dtype", [wk.F32, wk.BF16])
def test_two_column_blocks_per_head(ora, state_dtype):
    """d_v = 256: two 128-column workgroups per value head, of which only the
    first records the key head's q/k rows and the gate inputs, and the done
    counter reaches h_v x 2 before the flag flips; one-page equals slots bit
    for bit and the oracle within 1e-4 (3e-3 with bf16 checkpoints)."""
    wl = _small(n_req=3, n_steps=4, h_k=2, h_v=4, d_k=128, d_v=256, seed=53, state_dtype=state_dtype)
    inp = _inputs(wl, state_dtype)
    one = VerifyRun(wl, inp, ONEPAGE, state_dtype)
    o1 = one.run()
    slots = VerifyRun(wl, inp, SLOTS, state_dtype)
    assert torch.equal(o1, slots.run())
    assert torch.equal(one.committed_state(), slots.committed_state())
    dm = ora.dims_of(wl)
    o_ref, win_ref, S_ref = ora.verify(dm, inp["conv_w"], inp["a_log"], inp["dt_bias"], inp["x"], inp["a"],
                                       inp["b"], inp["accepted"], inp["window0"], inp["S0"],
                                       state_bf16=(state_dtype == wk.BF16))
    o = host(o1)
    worst = max(float(np.abs(o[:, r, :, h] - o_ref[:, r, :, h]).max() / np.abs(o_ref[:, r, :, h]).max())
                for r in range(wl.n_req) for h in range(wl.h_v))
    assert worst <= (1e-4 if state_dtype == wk.F32 else 3e-3), worst
    np.testing.assert_array_equal(host(one.committed_window()), win_ref)
    hdr = one.pages.header()
    assert int(one.err.item()) == 0 and int((hdr[:, 0] >> 8).abs().sum()) == 0  # done counters back to zero


@pytest.mark.parametrize("state_dtype", [wk.F32, wk.BF16])
def test_several_layers_share_one_pool_without_cross_talk(ora, state_dtype):
    """Three layers, each with its own conv weights, gates, inputs and
    initial states, keep their pages in one shared page pool and one shared
    conv pool and are stepped in turn on one stream (layer 0 step s, layer 1
    step s, layer 2 step s, ...): each layer's outputs, committed states and
    windows equal a run of that layer alone bit for bit and the oracle at
    the gate (the pages' own verify tests run several layers,
    "r9700-stack v0.2.4", section "What it does")."""
    g = gdn()
    n_layers, R = 3, 4
    wls = [_small(n_req=R, n_steps=4, seed=91 + i) for i in range(n_layers)]
    inps = [_inputs(w, state_dtype) for w in wls]
    dims = VerifyRun(wls[0], inps[0], ONEPAGE, state_dtype).dims
    pages = g.SpecPages.alloc(dims, ONEPAGE, n_layers * R, DEV)
    conv = g.ConvPool.alloc(dims, n_layers * R, 3 + dims.n_spec, DEV)
    # pages interleaved across layers: layer i, request r on page r * n_layers + i
    runs = [VerifyRun(w, x, ONEPAGE, state_dtype, pages_of=[r * n_layers + i for r in range(R)],
                      n_pages=n_layers * R, pages=pages, conv=conv) for i, (w, x) in enumerate(zip(wls, inps))]
    outs = [[] for _ in runs]
    zero = np.zeros(R, np.int32)
    for s in range(4):
        for i, run in enumerate(runs):
            outs[i].append(run.step(s, inps[i]["accepted"][s - 1] if s else zero))
    for i, run in enumerate(runs):
        run.step(0, inps[i]["accepted"][3], n_cand=0)
    tol = 1e-4 if state_dtype == wk.F32 else 3e-3
    for i, run in enumerate(runs):
        alone = VerifyRun(wls[i], inps[i], ONEPAGE, state_dtype)
        o_alone = alone.run()
        assert torch.equal(torch.stack(outs[i]), o_alone), i
        assert torch.equal(run.committed_state(), alone.committed_state()), i
        assert torch.equal(run.committed_window(), alone.committed_window()), i
        dm = ora.dims_of(wls[i])
        o_ref, win_ref, S_ref = ora.verify(dm, inps[i]["conv_w"], inps[i]["a_log"], inps[i]["dt_bias"], inps[i]["x"],
                                           inps[i]["a"], inps[i]["b"], inps[i]["accepted"], inps[i]["window0"],
                                           inps[i]["S0"], state_bf16=(state_dtype == wk.BF16))
        o = host(o_alone)
        for r in range(R):
            for h in range(wls[i].h_v):
                ref = o_ref[:, r, :, h]
                assert np.abs(o[:, r, :, h] - ref).max() <= tol * np.abs(ref).max(), (i, r, h)
        np.testing.assert_array_equal(host(run.committed_window()), win_ref)
    assert int(conv.sync.abs().sum()) == 0
