"""GPU tests of prefix caching beside the one-page record
(gdn_spec_verify_cached, gdn_prefix_restore).

"r9700-stack v0.2.4: one GDN state page per request", section "What it
does", runs the one-page record only with prefix caching off.  Here a cache
entry coexists with the record: a normal verify step may also leave the
committed prefix that ends at any replayed row in a cache entry, with no
extra launch, and a restore fills fresh pages from an entry.  Checked:
cached steps change nothing else (bit-identical to plain steps), the
one-page and slot designs cache the same bits, every cached prefix equals
the oracle's committed state and window for that prefix, and a restored
request continues as the oracle's committed stream through the cached row
does.
"""
import numpy as np
import pytest
import torch

import gdn_workloads as wk
from gpu_util import DEV, VerifyRun, dev, gdn, host

pytestmark = pytest.mark.gpu

ONEPAGE, SLOTS = 0, 1


def _inputs(wl, state_dtype):
    inp = wk.make_verify_inputs(wl)
    inp["S0"] = wk.round_to(inp["S0"], state_dtype)
    return inp


def _wl(**kw):
    base = dict(n_req=6, n_steps=5, seed=81)
    base.update(kw)
    return wk.SPEC_VERIFY.replace(**base)


def _oracle_prefix(ora, wl, inp, s, rows, state_bf16):
    """The oracle's committed state and window of the prefix that ends at
    candidate rows[r] of step s-1 (request r): the first s-1 steps committed
    with their own acceptances, step s-1 with rows[r]."""
    if s == 0:
        return inp["S0"].astype(np.float64), inp["window0"].astype(np.float64)
    acc = inp["accepted"][:s].copy()
    acc[s - 1] = rows
    dm = ora.dims_of(wl)
    _, win, S = ora.verify(dm, inp["conv_w"], inp["a_log"], inp["dt_bias"], inp["x"][:s], inp["a"][:s],
                           inp["b"][:s], acc, inp["window0"], inp["S0"], state_bf16=state_bf16)
    return S, win


def _rows_for_step(rng, s, prev, R):
    """A random cached row per request: 0..a' when the record holds rows (s > 0); 0 otherwise."""
    return np.array([int(rng.integers(0, int(prev[r]) + 1)) if s > 0 else 0 for r in range(R)], np.int32)


@pytest.mark.parametrize("state_dtype", [wk.F32, wk.BF16])
def test_cached_steps_match_plain_steps_slots_and_oracle(ora, state_dtype):
    g = gdn()
    wl = _wl()
    inp = _inputs(wl, state_dtype)
    R = wl.n_req
    plain = VerifyRun(wl, inp, ONEPAGE, state_dtype)
    one = VerifyRun(wl, inp, ONEPAGE, state_dtype)
    slots = VerifyRun(wl, inp, SLOTS, state_dtype)
    n_entries = wl.n_steps * R
    cache_one = g.PrefixCache.alloc(one.dims, n_entries, DEV)
    cache_slots = g.PrefixCache.alloc(slots.dims, n_entries, DEV)
    rng = np.random.default_rng(82)
    zero = np.zeros(R, np.int32)
    rows_at = []
    for s in range(wl.n_steps):
        prev = inp["accepted"][s - 1] if s else zero
        rows = _rows_for_step(rng, s, prev, R)
        rows_at.append(rows)
        entry = s * R + np.arange(R, dtype=np.int32)
        op = plain.step(s, prev)
        oc = one.step(s, prev, cache=cache_one, cache_entry=entry, cache_row=rows)
        os_ = slots.step(s, prev, cache=cache_slots, cache_entry=entry, cache_row=rows)
        assert not torch.isnan(oc).any()
        assert torch.equal(op, oc) and torch.equal(oc, os_), s
        assert torch.equal(plain.pages.buf, one.pages.buf), s
        assert torch.equal(plain.conv.buf, one.conv.buf), s
    # the two designs cache the same bits
    assert torch.equal(cache_one.state.buf, cache_slots.state.buf)
    assert torch.equal(cache_one.conv.buf, cache_slots.conv.buf)
    assert int(one.err.item()) == 0 and int(slots.err.item()) == 0
    # every cached prefix is the oracle's committed prefix through that row
    tol = 1e-4 if state_dtype == wk.F32 else 3e-3
    cs, cw = host(cache_one.state.buf), host(cache_one.conv.buf)
    for s in range(wl.n_steps):
        S_ref, win_ref = _oracle_prefix(ora, wl, inp, s, rows_at[s], state_dtype == wk.BF16)
        for r in range(R):
            e = s * R + r
            np.testing.assert_array_equal(cw[e], win_ref[r])
            for h in range(wl.h_v):
                ref = S_ref[r, h]
                assert np.abs(cs[e, h] - ref).max() <= tol * np.abs(ref).max(), (s, r, h)
    # a prefix cached at the full replay is the step's checkpoint, bit for bit
    last = wl.n_steps - 1
    full = [r for r in range(R) if rows_at[last][r] == inp["accepted"][last - 1][r]]
    for r in full:
        assert torch.equal(cache_one.state.buf[last * R + r], one.pages.states()[r, 0])


@pytest.mark.parametrize("state_dtype", [wk.F32, wk.BF16])
def test_restored_prefix_continues_like_the_oracle(ora, state_dtype):
    """Cache every request's prefix at a random replayed row of step 3,
    restore the entries into fresh pages, and continue with steps 3.. : the
    outputs and the final committed state follow the oracle's committed
    stream through the cached row, and equal a restore by tensor copies bit
    for bit."""
    g = gdn()
    wl = _wl(n_steps=7, seed=83)
    inp = _inputs(wl, state_dtype)
    R, s_cache = wl.n_req, 3
    A = VerifyRun(wl, inp, ONEPAGE, state_dtype)
    cache = g.PrefixCache.alloc(A.dims, R, DEV)
    zero = np.zeros(R, np.int32)
    for s in range(s_cache):
        A.step(s, inp["accepted"][s - 1] if s else zero)
    prev = inp["accepted"][s_cache - 1]
    rows = np.random.default_rng(84).integers(0, prev + 1).astype(np.int32)
    A.step(s_cache, prev, cache=cache, cache_entry=np.arange(R, dtype=np.int32), cache_row=rows)
    # restore into fresh pages, pages in reverse order to exercise the page map
    B = VerifyRun(wl, inp, ONEPAGE, state_dtype, pages_of=list(range(R))[::-1])
    B.pages.buf.fill_(0x5A)                                   # a stale page: header, checkpoint and record
    B.book.hdr[:] = B.pages.header()[:, :4].cpu().numpy().view(np.uint32)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    g.gdn_prefix_restore(B.dims, B.pages, torch.arange(R, dtype=torch.int32, device=DEV), B.rp, cache, B.conv,
                         err=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    for r, p in enumerate(B.req_page):
        B.book.hdr[p] = 0
        B.book.cbuf[p, :3] = host(cache.conv.buf[r])
    # the same restore by tensor copies
    Cp = VerifyRun(wl, inp, ONEPAGE, state_dtype)
    Cp.pages.states()[:, 0] = cache.state.buf
    Cp.conv.buf[:, :3] = cache.conv.buf
    Cp.book.cbuf[:, :3] = host(cache.conv.buf)
    outs_b, outs_c = [], []
    for s in range(s_cache, wl.n_steps):
        prev_s = inp["accepted"][s - 1] if s > s_cache else zero
        ob = B.step(s, prev_s)
        oc = Cp.step(s, prev_s)
        assert torch.equal(ob, oc), s
        outs_b.append(host(ob))
    B.step(0, inp["accepted"][wl.n_steps - 1], n_cand=0)
    Cp.step(0, inp["accepted"][wl.n_steps - 1], n_cand=0)
    assert torch.equal(B.committed_state(), Cp.committed_state())
    # oracle: the committed stream through step s_cache-1's candidate rows[r], then steps s_cache..
    acc = inp["accepted"].copy()
    acc[s_cache - 1] = rows
    dm = ora.dims_of(wl)
    o_ref, win_ref, S_ref = ora.verify(dm, inp["conv_w"], inp["a_log"], inp["dt_bias"], inp["x"], inp["a"],
                                       inp["b"], acc, inp["window0"], inp["S0"], state_bf16=(state_dtype == wk.BF16))
    tol = 1e-4 if state_dtype == wk.F32 else 3e-3
    got = np.stack(outs_b)                                  # [steps][R][K][h_v][d_v]
    for r in range(R):
        for h in range(wl.h_v):
            ref = o_ref[s_cache:, r, :, h]
            assert np.abs(got[:, r, :, h] - ref).max() <= tol * np.abs(ref).max(), (r, h)
    Sb = host(B.committed_state())
    for r in range(R):
        for h in range(wl.h_v):
            assert np.abs(Sb[r, h] - S_ref[r, h]).max() <= tol * np.abs(S_ref[r, h]).max(), (r, h)
    np.testing.assert_array_equal(host(B.committed_window()), win_ref)


def test_cache_of_an_empty_record_is_the_checkpoint():
    """On a fresh page and after a commit-only step the live record holds no
    rows: the entry receives the checkpoint and conv rows 0..2 as they are,
    whatever the row argument says."""
    g = gdn()
    wl = _wl(n_req=4, n_steps=3, seed=85)
    inp = _inputs(wl, wk.F32)
    R = wl.n_req
    run = VerifyRun(wl, inp, ONEPAGE, wk.F32)
    cache = g.PrefixCache.alloc(run.dims, 2 * R, DEV)
    S0, W0 = run.committed_state().clone(), run.committed_window().clone()
    run.step(0, np.zeros(R, np.int32), cache=cache, cache_entry=np.arange(R, dtype=np.int32),
             cache_row=np.full(R, 5, np.int32))
    assert torch.equal(cache.state.buf[:R], S0) and torch.equal(cache.conv.buf[:R], W0)
    run.step(1, inp["accepted"][0])
    run.step(0, inp["accepted"][1], n_cand=0)                 # commit: the live record is empty again
    S1, W1 = run.committed_state().clone(), run.committed_window().clone()
    run.step(2, np.zeros(R, np.int32), cache=cache, cache_entry=R + np.arange(R, dtype=np.int32),
             cache_row=np.full(R, 7, np.int32))
    assert torch.equal(cache.state.buf[R:], S1) and torch.equal(cache.conv.buf[R:], W1)
    assert int(run.err.item()) == 0


def test_bad_cache_arguments_refuse_the_request():
    """An entry beyond the cache, or a row past the replayed acceptance,
    refuses that request (nothing of it is written, GDN_DEVERR_CACHE);
    a negative entry caches nothing; the other requests step normally."""
    g = gdn()
    wl = _wl(n_req=4, n_steps=3, seed=86)
    inp = _inputs(wl, wk.F32)
    R = wl.n_req
    run = VerifyRun(wl, inp, ONEPAGE, wk.F32)
    cache = g.PrefixCache.alloc(run.dims, 2, DEV)
    run.step(0, np.zeros(R, np.int32))
    prev = np.array([2, 3, 1, 4], np.int32)
    snap_pages, snap_conv = run.pages.buf.clone(), run.conv.buf.clone()
    before = cache.state.buf.clone()
    run.step(1, prev, cache=cache, cache_entry=np.array([5, 0, 1, -1], np.int32),
             cache_row=np.array([0, 4, 1, 9], np.int32), refused=(0, 1))
    assert int(run.err.item()) & g.GDN_DEVERR_CACHE
    for r in (0, 1):
        assert torch.equal(run.pages.buf[r], snap_pages[r]) and torch.equal(run.conv.buf[r], snap_conv[r])
    assert torch.equal(cache.state.buf[0], before[0])         # request 1's entry untouched
    assert not torch.equal(cache.state.buf[1], before[1])     # request 2 cached its prefix


def test_restore_skips_padding_and_reports_bad_entries():
    g = gdn()
    wl = _wl(n_req=3, n_steps=1, seed=87)
    inp = _inputs(wl, wk.F32)
    run = VerifyRun(wl, inp, ONEPAGE, wk.F32)
    cache = g.PrefixCache.alloc(run.dims, 2, DEV)
    cache.state.buf.normal_()
    cache.conv.buf.normal_()
    snap = run.pages.buf.clone()
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    g.gdn_prefix_restore(run.dims, run.pages, torch.tensor([1, -1, 7], dtype=torch.int32, device=DEV),
                         torch.tensor([0, 1, 2], dtype=torch.int32, device=DEV), cache, run.conv, err=err)
    torch.cuda.synchronize()
    assert int(err.item()) == g.GDN_DEVERR_CACHE
    assert torch.equal(run.pages.states()[0, 0], cache.state.buf[1])
    assert torch.equal(run.conv.buf[0, :3], cache.conv.buf[1])
    assert int(run.pages.header()[0].abs().sum()) == 0
    assert torch.equal(run.pages.buf[1:], snap[1:])
