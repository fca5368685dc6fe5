"""GPU parity of the token-by-token core (gdn_recurrent_seq) and the conv
update (gdn_conv_update) against the fp64 oracle, plus the bit-exact
properties between launches.  Tolerance: max relative error 1e-4 per
(tensor, sequence, head) slice for the fp32-state path."""
import numpy as np
import pytest
import torch

import gdn_workloads as wk
from gpu_util import (DEV, dev, dims_of, gdn, host, make_batch, max_slice_rel_S, max_slice_rel_o,
                      oracle_seq, params_of, rel, run_seq, seq_pools)

pytestmark = pytest.mark.gpu

TOL = 1e-4


def _check(ora, wl, inp, pages=None, has_init=None, tol=TOL):
    o, conv, state = run_seq(wl, inp, pages=pages, has_init=has_init)
    o_ref, win_ref, S_ref = oracle_seq(ora, wl, inp, has_init=has_init)
    pages = list(range(len(wl.seqlens))) if pages is None else pages
    idx = [p for p in pages]
    assert max_slice_rel_o(host(o), o_ref, inp["cu_seqlens"]) <= tol
    S = host(state.buf)[idx]
    assert max_slice_rel_S(S, S_ref) <= tol
    np.testing.assert_array_equal(host(conv.buf)[idx], win_ref)  # rolled window: exact data movement
    assert int(conv.sync.abs().sum()) == 0
    return o, conv, state


def test_tiny_parity(ora):
    wl = wk.TINY
    _check(ora, wl, wk.make_sequence_inputs(wl))


def test_decode_parity(ora):
    wl = wk.DECODE
    _check(ora, wl, wk.make_sequence_inputs(wl))


def test_decode_work_counter_repeated_steps(ora):
    """The decode kernel hands out the items past each workgroup's first
    three from the work counter that follows the conv pool's arrival words.
    Three steps in a row on the same pools: each equals the oracle's step
    from the previous step's device state and window, and every sync word,
    the work counter included, is zero after each call.  Outputs are
    compared normwise per head over the batch: a single token's 128-value
    output slice can be thousands of times smaller than the head's typical
    output (q nearly orthogonal to k under strong decay, where o is about
    (k.q) beta v and k.q is itself a cancelling sum), and there a relative
    error per slice measures fp32 rounding of the terms, not the kernel.
    States are compared per (sequence, head) slice as everywhere else."""
    g = gdn()
    wl = wk.DECODE
    base = wk.make_sequence_inputs(wl)
    n = len(wl.seqlens)
    dims, conv, state = seq_pools(wl, base, list(range(n)), n)
    params = params_of(base, wl)
    batch = make_batch(base["cu_seqlens"], list(range(n)), base["x"].shape[0])
    for step in range(3):
        fresh = wk.make_sequence_inputs(wl.replace(seed=wl.seed + 100 + step))
        ref_inp = dict(base, x=fresh["x"], a=fresh["a"], b=fresh["b"],
                       window0=host(conv.buf)[:, :wl.conv_w - 1], S0=host(state.buf))
        x, a, b = (dev(fresh[k], dims.act_torch) for k in ("x", "a", "b"))
        o = torch.full((x.shape[0], wl.h_v, wl.d_v), float("nan"), device=DEV)
        g.gdn_recurrent_seq(dims, params, x, a, b, batch, conv, state, o=o)
        torch.cuda.synchronize()
        o_ref, win_ref, S_ref = oracle_seq(ora, wl, ref_inp)
        oh = host(o)
        assert max(rel(oh[:, h], o_ref[:, h]) for h in range(wl.h_v)) <= TOL, step
        assert max_slice_rel_S(host(state.buf), S_ref) <= TOL, step
        np.testing.assert_array_equal(host(conv.buf), win_ref)
        assert int(conv.sync.abs().sum()) == 0, step


def test_short_prefill_parity(ora):
    wl = wk.SHORT_PREFILL
    _check(ora, wl, wk.make_sequence_inputs(wl))


@pytest.mark.parametrize("lens", [(1, 2, 3, 17, 33), (0, 5, 0, 16), (2,), (47,)])
def test_ragged_edges(ora, lens):
    wl = wk.DECODE.replace(seqlens=lens, seed=7)
    _check(ora, wl, wk.make_sequence_inputs(wl))


def test_has_init_zero_and_padding(ora):
    wl = wk.DECODE.replace(seqlens=(5, 9, 3, 6), seed=8)
    inp = wk.make_sequence_inputs(wl)
    has = np.array([0, 1, 0, 1], np.uint8)
    g = gdn()
    # padding row (-1) skipped: nothing of it read or written
    pages = [3, -1, 0, 2]
    o, conv, state = run_seq(wl, inp, pages=pages, n_pages=5, has_init=has)
    o_ref, win_ref, S_ref = oracle_seq(ora, wl, inp, has_init=has)
    cu = inp["cu_seqlens"]
    oh = host(o)
    for s, p in enumerate(pages):
        rows = slice(int(cu[s]), int(cu[s + 1]))
        if p < 0:
            assert np.isnan(oh[rows]).all()
            continue
        assert max_slice_rel_o(oh[rows], o_ref[rows], [0, cu[s + 1] - cu[s]]) <= TOL
        assert max_slice_rel_S(host(state.buf)[p:p + 1], S_ref[s:s + 1]) <= TOL
        np.testing.assert_array_equal(host(conv.buf)[p], win_ref[s])
    # pages 1 and 4 were never touched
    assert float(state.buf[1].abs().sum()) == 0.0 and float(state.buf[4].abs().sum()) == 0.0


def test_d_k_64_and_scale(ora):
    wl = wk.Workload("d64", h_k=4, h_v=8, d_k=64, d_v=64, conv_w=4, act_dtype=wk.BF16,
                     state_dtype=wk.F32, seqlens=(7, 30), seed=9, scale=64 ** -0.5)
    _check(ora, wl, wk.make_sequence_inputs(wl))


def test_mild_decay_long_memory(ora):
    """Weak decay keeps far history in the state, so state propagation errors
    cannot hide behind the workload's strong decay."""
    wl = wk.DECODE.replace(seqlens=(200, 61), seed=10)
    inp = wk.make_sequence_inputs(wl)
    inp["a_log"] = np.full_like(inp["a_log"], np.log(0.02))
    _check(ora, wl, inp)


def test_bf16_state(ora):
    wl = wk.DECODE.replace(seqlens=(9, 1, 20), state_dtype=wk.BF16, seed=11)
    inp = wk.make_sequence_inputs(wl)
    o, conv, state = run_seq(wl, inp)
    o_ref, win_ref, S_ref = oracle_seq(ora, wl, inp)
    assert max_slice_rel_o(host(o), o_ref, inp["cu_seqlens"]) <= TOL
    # the state is stored once, rounded to bf16 (relative step 2^-8)
    assert max_slice_rel_S(host(state.buf), S_ref) <= 2.0 ** -8


def test_one_launch_equals_token_launches():
    """T tokens in one launch == T launches of one token, bit for bit (fp32
    state): the per-token arithmetic does not depend on how tokens are batched."""
    g = gdn()
    wl = wk.DECODE.replace(seqlens=(21, 6), seed=12)
    inp = wk.make_sequence_inputs(wl)
    o_all, conv_all, st_all = run_seq(wl, inp)
    params = params_of(inp, wl)
    dims, conv, state = seq_pools(wl, inp, [0, 1], 2)
    x = dev(inp["x"], dims.act_torch)
    a = dev(inp["a"], dims.act_torch)
    b = dev(inp["b"], dims.act_torch)
    cu = inp["cu_seqlens"]
    o_tok = torch.full_like(o_all, float("nan"))
    for s in range(2):
        for t in range(int(cu[s]), int(cu[s + 1])):
            batch = make_batch([0, 1], [s], 1)
            g.gdn_recurrent_seq(dims, params, x[t:t + 1], a[t:t + 1], b[t:t + 1], batch, conv, state,
                                o=o_tok[t:t + 1])
    torch.cuda.synchronize()
    assert torch.equal(o_tok, o_all)
    assert torch.equal(state.buf, st_all.buf)
    assert torch.equal(conv.buf, conv_all.buf)


def test_deterministic_and_batch_independent():
    """Two runs agree bit for bit, and a sequence gives the same bits alone
    as inside a batch (identical copies in lockstep agree with the lone run)."""
    wl = wk.DECODE.replace(seqlens=(13, 13, 13), seed=13)
    inp = wk.make_sequence_inputs(wl)
    for k in ("window0", "S0"):
        inp[k][1] = inp[k][0]
        inp[k][2] = inp[k][0]
    T = 13
    inp["x"][T:2 * T] = inp["x"][:T]
    inp["x"][2 * T:] = inp["x"][:T]
    for k in ("a", "b"):
        inp[k][T:2 * T] = inp[k][:T]
        inp[k][2 * T:] = inp[k][:T]
    o1, c1, s1 = run_seq(wl, inp)
    o2, c2, s2 = run_seq(wl, inp)
    assert torch.equal(o1, o2) and torch.equal(s1.buf, s2.buf) and torch.equal(c1.buf, c2.buf)
    assert torch.equal(o1[:T], o1[T:2 * T]) and torch.equal(o1[:T], o1[2 * T:])
    lone = wl.replace(seqlens=(13,))
    inp1 = {k: (v[:1] if k in ("window0", "S0") else v[:T] if k in ("x", "a", "b") else v)
            for k, v in inp.items()}
    inp1["cu_seqlens"] = np.array([0, T], np.int32)
    o3, c3, s3 = run_seq(lone, inp1)
    assert torch.equal(o3, o1[:T]) and torch.equal(s3.buf[0], s1.buf[0])


def test_device_errors_skip_and_report():
    g = gdn()
    wl = wk.DECODE.replace(seqlens=(4, 4), seed=14)
    inp = wk.make_sequence_inputs(wl)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    # page 7 does not exist in a 2-page pool
    o, conv, state = run_seq(wl, inp, pages=[0, 7], n_pages=2, err=err)
    assert int(err.item()) & g.GDN_DEVERR_PAGE
    assert np.isnan(host(o)[4:]).all() and not np.isnan(host(o)[:4]).any()


# ------------------------------------------------------------- conv update
def _conv_call(wl, inp, act, y_dtype, max_seqlen=None, has_init=None):
    g = gdn()
    dims = dims_of(wl)
    n = len(wl.seqlens)
    conv = g.ConvPool.alloc(dims, n, 3, DEV)
    for s in range(n):
        conv.buf[s] = dev(inp["window0"][s], dims.act_torch)
    x = dev(inp["x"], dims.act_torch)
    batch = make_batch(inp["cu_seqlens"], list(range(n)), x.shape[0], has_init, max_seqlen)
    y = g.gdn_conv_update(dims, dev(inp["conv_w"], dims.act_torch), x, batch, conv, activation=act,
                          y_dtype=y_dtype)
    torch.cuda.synchronize()
    return y, conv


@pytest.mark.parametrize("max_seqlen", [None, 0])
def test_conv_update_bit_exact_fp32_model(ora, max_seqlen):
    """activation off, fp32 output: bit-exact against the fp32 op-order model."""
    wl = wk.SHORT_PREFILL.replace(seqlens=(45, 200, 0, 3), act_dtype=wk.F32, seed=15)
    inp = wk.make_sequence_inputs(wl)
    y, conv = _conv_call(wl, inp, False, "f32", max_seqlen)
    cu = inp["cu_seqlens"]
    yh = y.cpu().numpy()
    for s in range(len(wl.seqlens)):
        r0, r1 = int(cu[s]), int(cu[s + 1])
        ref = ora.conv_f32_model(inp["x"][r0:r1], inp["conv_w"], inp["window0"][s])
        np.testing.assert_array_equal(yh[r0:r1], ref)
    _, win_ref = ora.conv_update(inp["x"], inp["conv_w"], cu, inp["window0"])
    np.testing.assert_array_equal(host(conv.buf), win_ref)


def test_conv_update_silu_parity(ora):
    wl = wk.SHORT_PREFILL.replace(seqlens=(45, 83, 159, 1, 2), seed=16)
    inp = wk.make_sequence_inputs(wl)
    has = np.array([1, 0, 1, 1, 0], np.uint8)
    y, conv = _conv_call(wl, inp, True, "f32", has_init=has)
    y_ref, win_ref = ora.conv_update(inp["x"], inp["conv_w"], inp["cu_seqlens"], inp["window0"], has)
    assert rel(host(y), y_ref) <= 1e-6
    np.testing.assert_array_equal(host(conv.buf), win_ref)
    yb, _ = _conv_call(wl, inp, True, "bf16", has_init=has)
    assert rel(host(yb), y_ref) <= 2.0 ** -8
    # the bf16 output is the fp32 output rounded to nearest even, bit for bit
    assert torch.equal(yb.view(torch.int16), y.to(torch.bfloat16).view(torch.int16))


def test_fused_conv_window_equals_conv_update():
    """The fused kernel rolls the window exactly as gdn_conv_update does."""
    wl = wk.SHORT_PREFILL.replace(seqlens=(45, 2, 70), seed=17)
    inp = wk.make_sequence_inputs(wl)
    _, conv_fused, _ = run_seq(wl, inp)
    _, conv_alone = _conv_call(wl, inp, True, "f32")
    assert torch.equal(conv_fused.buf, conv_alone.buf)


def _check_pages(ora, wl, inp, pages, has, n_pages, s_tol=TOL):
    o, conv, state = run_seq(wl, inp, pages=pages, n_pages=n_pages, has_init=has)
    o_ref, win_ref, S_ref = oracle_seq(ora, wl, inp, has_init=has)
    cu = inp["cu_seqlens"]
    oh, Sh, Ch = host(o), host(state.buf), host(conv.buf)
    used = set()
    for s, p in enumerate(pages):
        rows = slice(int(cu[s]), int(cu[s + 1]))
        if p < 0:
            assert np.isnan(oh[rows]).all()
            continue
        used.add(p)
        assert max_slice_rel_o(oh[rows], o_ref[rows], [0, cu[s + 1] - cu[s]]) <= TOL
        if cu[s + 1] == cu[s]:
            continue  # an empty sequence leaves its page as it was
        assert max_slice_rel_S(Sh[p:p + 1], S_ref[s:s + 1]) <= s_tol
        np.testing.assert_array_equal(Ch[p], win_ref[s])
    for p in range(n_pages):
        if p not in used:
            assert float(state.buf[p].abs().sum()) == 0.0
    assert int(conv.sync.abs().sum()) == 0


@pytest.mark.parametrize("state_dtype", [wk.F32, wk.BF16])
def test_decode_stream_many_items(ora, state_dtype):
    """Sequences of at most 4 tokens take the streaming kernel.  With 40
    sequences x 32 heads there are more items than resident workgroups, so
    each workgroup walks several items with the next one's state prefetched;
    lengths 0..4, fresh and continuing states and padding rows are mixed so
    skipped items fall between fetched ones."""
    rng = np.random.default_rng(21)
    n = 40
    lens = tuple(int(x) for x in rng.integers(0, 5, size=n))
    wl = wk.DECODE.replace(seqlens=lens, state_dtype=state_dtype, seed=21)
    inp = wk.make_sequence_inputs(wl)
    has = (rng.random(n) < 0.75).astype(np.uint8)
    pages = list(range(n))
    pages[5] = pages[17] = pages[18] = -1
    _check_pages(ora, wl, inp, pages, has, n, s_tol=TOL if state_dtype == wk.F32 else 2.0 ** -8)


def test_decode_stream_d64_two_blocks(ora):
    """d_k = 64 and d_v = 256: two 128-column items per head share the key
    head's conv window (arrival count 2 r)."""
    wl = wk.Workload("d64v256", h_k=4, h_v=8, d_k=64, d_v=256, conv_w=4, act_dtype=wk.BF16,
                     state_dtype=wk.F32, seqlens=(1, 2, 3, 4, 1, 0, 2) * 12, seed=22, scale=64 ** -0.5)
    inp = wk.make_sequence_inputs(wl)
    n = len(wl.seqlens)
    _check_pages(ora, wl, inp, list(range(n)), None, n)


@pytest.mark.parametrize("state_dtype", [wk.F32, wk.BF16])
def test_decode_stream_one_block_per_head(ora, state_dtype):
    """d_v = 64 takes the streaming kernel with 64-column items (two state
    columns per lane): one item per head, so each key head's window is
    owned by its r value heads alone (arrival count r)."""
    wl = wk.Workload("d64v64", h_k=4, h_v=8, d_k=64, d_v=64, conv_w=4, act_dtype=wk.BF16,
                     state_dtype=state_dtype, seqlens=(1, 4, 2, 0, 3, 1) * 12, seed=26, scale=64 ** -0.5)
    inp = wk.make_sequence_inputs(wl)
    n = len(wl.seqlens)
    _check_pages(ora, wl, inp, list(range(n)), None, n, s_tol=TOL if state_dtype == wk.F32 else 2.0 ** -8)


@pytest.mark.parametrize("state_dtype", [wk.F32, wk.BF16])
def test_decode_stream_d32(ora, state_dtype):
    """d_k = 32 (two state rows per lane in the staged layout) with d_v = 128
    through the streaming kernel, fp32 and bf16 state."""
    wl = wk.Workload("d32v128", h_k=4, h_v=8, d_k=32, d_v=128, conv_w=4, act_dtype=wk.BF16,
                     state_dtype=state_dtype, seqlens=(1, 3, 4, 1, 2, 0, 1) * 10, seed=23)
    inp = wk.make_sequence_inputs(wl)
    n = len(wl.seqlens)
    _check_pages(ora, wl, inp, list(range(n)), None, n, s_tol=TOL if state_dtype == wk.F32 else 2.0 ** -8)


def test_more_sequences_than_threads(ora):
    """More sequences than a workgroup has threads (600 > 512): the
    longest-first ranking is off and workgroups keep the batch order."""
    rng = np.random.default_rng(24)
    lens = tuple(int(x) for x in rng.integers(5, 9, size=600))
    wl = wk.TINY.replace(seqlens=lens, h_k=1, h_v=2, s0_std=0.05, window_std=1.0, seed=24)
    inp = wk.make_sequence_inputs(wl)
    n = len(lens)
    _check_pages(ora, wl, inp, list(range(n)), None, n)


@pytest.mark.parametrize("n", [1, 3])
def test_decode_stream_fewer_items_than_workgroups(ora, n):
    """One and three decode sequences: fewer (sequence, head) items than the
    resident grid, every workgroup takes at most one item."""
    wl = wk.DECODE.replace(seqlens=(1,) * n, seed=25)
    inp = wk.make_sequence_inputs(wl)
    _check_pages(ora, wl, inp, list(range(n)), None, n)


def test_bf16_state_store_rounds_to_nearest_even():
    """One decode token from a start state that bf16 represents exactly runs
    the same fp32 arithmetic with either state dtype, so the bf16 run must
    store exactly the round-to-nearest-even of the fp32 run's new state
    (torch's conversion), and both runs give the same outputs bit for bit.
    Pins the kernels' fp32 -> bf16 conversion to that rounding."""
    wl = wk.DECODE.replace(seqlens=(1,) * 8, seed=27)
    inp = wk.make_sequence_inputs(wl)
    inp["S0"] = wk.round_to(inp["S0"], wk.BF16)
    o32, _, st32 = run_seq(wl, inp)
    o16, _, st16 = run_seq(wl.replace(state_dtype=wk.BF16), inp)
    assert torch.equal(o32, o16)
    ref = st32.buf.to(torch.bfloat16)
    assert torch.equal(st16.buf.view(torch.int16), ref.view(torch.int16))
    # the step moved the state: not every value was already representable
    assert not torch.equal(st32.buf, ref.to(torch.float32))


@pytest.mark.parametrize("h_k,h_v", [(4, 4), (2, 8)])
@pytest.mark.parametrize("lens", [(1, 2, 1, 3), (1, 40, 7)])
def test_gqa_ratios(ora, h_k, h_v, lens):
    """One and four value heads per key head (the workloads use two), through
    the streaming decode kernel (lengths <= 4) and the general one: key-head
    mapping and the q/k window written after r * blocks arrivals."""
    wl = wk.DECODE.replace(h_k=h_k, h_v=h_v, seqlens=lens, seed=28)
    _check(ora, wl, wk.make_sequence_inputs(wl))


def test_decode_stream_many_claims(ora):
    """200 sequences of 1-4 tokens at the decode shape: 6,400 items, about
    twelve per resident workgroup, so most are handed out from the work
    counter; every sequence matches the oracle and the counter returns to
    zero."""
    rng = np.random.default_rng(29)
    lens = tuple(int(x) for x in rng.integers(1, 5, size=200))
    wl = wk.DECODE.replace(seqlens=lens, seed=29)
    _check(ora, wl, wk.make_sequence_inputs(wl))


def _stream_shapes():
    d64v64 = wk.Workload("d64v64", h_k=4, h_v=8, d_k=64, d_v=64, conv_w=4, act_dtype=wk.BF16,
                         state_dtype=wk.F32, seqlens=(1,), seed=31, scale=64 ** -0.5)
    d32v128 = wk.Workload("d32v128", h_k=4, h_v=8, d_k=32, d_v=128, conv_w=4, act_dtype=wk.BF16,
                          state_dtype=wk.F32, seqlens=(1,), seed=32)
    return {"decode": wk.DECODE.replace(seed=30), "d64v64": d64v64, "d32v128": d32v128}


@pytest.mark.parametrize("state_dtype", [wk.F32, wk.BF16])
@pytest.mark.parametrize("shape", ["decode", "d64v64", "d32v128"])
def test_decode_stream_grid_shapes_agree(ora, shape, state_dtype):
    """Above four items per compute unit the decode kernel runs one
    workgroup per CU, each walking many items (most of them claimed from the
    work counter); at four or fewer it fills every resident slot.  The same
    sequences -- 1 to 4 tokens, fresh and continuing states -- run once as
    one batch and once as consecutive calls of at most four items per CU on
    fresh pools: outputs, states and windows agree bit for bit (128- and
    64-column items, d_k = 32 and 128, fp32 and bf16 state), and the batch
    run matches the oracle."""
    base = _stream_shapes()[shape]
    ncu = torch.cuda.get_device_properties(DEV).multi_processor_count
    per_seq = base.h_v * (base.d_v // (128 if base.d_v % 128 == 0 else 64))
    small = max(1, 4 * ncu // per_seq)          # sequences per call at four items per CU or fewer
    n = 3 * small + 5                           # more than four items per CU in one call
    rng = np.random.default_rng(33)
    lens = tuple(int(v) for v in rng.integers(1, 5, size=n))
    wl = base.replace(seqlens=lens, state_dtype=state_dtype)
    inp = wk.make_sequence_inputs(wl)
    has = (rng.random(n) < 0.8).astype(np.uint8)
    pages = list(range(n))
    o1, c1, s1 = run_seq(wl, inp, pages=pages, n_pages=n, has_init=has)

    g = gdn()
    dims, conv, state = seq_pools(wl, inp, pages, n)
    params = params_of(inp, wl)
    x, a, b = (dev(inp[k], dims.act_torch) for k in ("x", "a", "b"))
    o2 = torch.full((x.shape[0], wl.h_v, wl.d_v), float("nan"), device=DEV)
    cu = inp["cu_seqlens"]
    for lo in range(0, n, small):
        hi = min(n, lo + small)
        r0, r1 = int(cu[lo]), int(cu[hi])
        batch = make_batch(cu[lo:hi + 1] - r0, pages[lo:hi], r1 - r0, has[lo:hi])
        g.gdn_recurrent_seq(dims, params, x[r0:r1], a[r0:r1], b[r0:r1], batch, conv, state, o=o2[r0:r1])
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)
    assert torch.equal(s1.buf, state.buf)
    assert torch.equal(c1.buf, conv.buf)
    assert int(c1.sync.abs().sum()) == 0 and int(conv.sync.abs().sum()) == 0

    # Outputs normwise per head over the batch, as in the repeated-steps
    # test: a one-token slice can be orders of magnitude below the head's
    # typical output, and its own relative error then measures fp32 rounding.
    o_ref, win_ref, S_ref = oracle_seq(ora, wl, inp, has_init=has)
    oh = host(o1)
    assert max(rel(oh[:, h], o_ref[:, h]) for h in range(wl.h_v)) <= TOL
    assert max_slice_rel_S(host(s1.buf), S_ref) <= (TOL if state_dtype == wk.F32 else 2.0 ** -8)
    np.testing.assert_array_equal(host(c1.buf), win_ref)
