"""GPU parity of the chunked WY/UT prefill (gdn_chunked_prefill) on bf16
matrix cores: against the fp64 token-by-token oracle and against the
token-by-token kernel, max relative error 3e-3 per (tensor, sequence, head)
slice."""
import numpy as np
import pytest
import torch

import gdn_workloads as wk
from gpu_util import DEV, dev, gdn, host, max_slice_rel_S, max_slice_rel_o, oracle_seq, run_seq

pytestmark = pytest.mark.gpu

TOL = 3e-3


def _small(lens, seed, **kw):
    base = dict(name="chunk_small", h_k=2, h_v=4, d_k=128, d_v=128, conv_w=4, act_dtype=wk.BF16,
                state_dtype=wk.F32, seqlens=lens, chunk=64, seed=seed)
    base.update(kw)
    return wk.Workload(**base)


def _check(ora, wl, inp, tol=TOL, has_init=None, pages=None):
    o, conv, state = run_seq(wl, inp, chunk=64, has_init=has_init, pages=pages)
    o_ref, win_ref, S_ref = oracle_seq(ora, wl, inp, has_init=has_init)
    idx = list(range(len(wl.seqlens))) if pages is None else pages
    eo = max_slice_rel_o(host(o), o_ref, inp["cu_seqlens"])
    eS = max_slice_rel_S(host(state.buf)[idx], S_ref)
    assert eo <= tol and eS <= tol, (eo, eS)
    np.testing.assert_array_equal(host(conv.buf)[idx], win_ref)
    assert int(conv.sync.abs().sum()) == 0
    return eo, eS


@pytest.mark.parametrize("lens", [(64,), (130, 64, 1, 200), (63, 65, 127, 3)])
def test_chunked_parity_ragged(ora, lens):
    wl = _small(lens, seed=41)
    _check(ora, wl, wk.make_sequence_inputs(wl))


def test_chunked_fp32_activations_short_sequences(ora):
    """fp32 activations (rows read as 16-byte vectors of 4 channels) and
    sequences shorter than the conv window, with and without an initial
    state: the first chunk's halo rows come from the window or are zero."""
    wl = _small((1, 2, 3, 66, 129), seed=45, act_dtype=wk.F32)
    inp = wk.make_sequence_inputs(wl)
    _check(ora, wl, inp, has_init=np.array([0, 1, 0, 1, 0], np.uint8))


def test_chunked_bf16_state_and_has_init(ora):
    wl = _small((150, 70), seed=42)
    inp = wk.make_sequence_inputs(wl)
    _check(ora, wl, inp, has_init=np.array([0, 1], np.uint8))
    wlb = wl.replace(state_dtype=wk.BF16)
    inpb = wk.make_sequence_inputs(wlb)
    o, conv, state = run_seq(wlb, inpb, chunk=64)
    o_ref, _, S_ref = oracle_seq(ora, wlb, inpb)
    assert max_slice_rel_o(host(o), o_ref, inpb["cu_seqlens"]) <= TOL
    assert max_slice_rel_S(host(state.buf), S_ref) <= TOL + 2.0 ** -8


def test_chunked_mild_decay(ora):
    """Weak decay lets bf16 operand rounding accumulate over the sequence;
    the bound here is the same 3e-3 on a shorter sequence."""
    wl = _small((256, 190), seed=43)
    inp = wk.make_sequence_inputs(wl)
    inp["a_log"] = np.full_like(inp["a_log"], np.log(0.05))
    _check(ora, wl, inp)


def test_chunked_equals_token_by_token_kernel():
    """The chunked form equals the token-by-token kernel within 3e-3."""
    wl = _small((333, 64, 129), seed=44, h_k=4, h_v=8)
    inp = wk.make_sequence_inputs(wl)
    o_c, conv_c, st_c = run_seq(wl, inp, chunk=64)
    o_s, conv_s, st_s = run_seq(wl, inp)
    assert max_slice_rel_o(host(o_c), host(o_s), inp["cu_seqlens"]) <= TOL
    assert max_slice_rel_S(host(st_c.buf), host(st_s.buf)) <= TOL
    assert torch.equal(conv_c.buf, conv_s.buf)


def test_long_prefill_full_size_sampled_heads(ora):
    """The long-prefill workload at full size (4 x 8192 tokens, 32 value
    heads); the oracle recomputes a sample of (sequence, head) pairs."""
    wl = wk.LONG_PREFILL
    inp = wk.make_sequence_inputs(wl)
    o, conv, state = run_seq(wl, inp, chunk=64)
    sel = np.zeros((len(wl.seqlens), wl.h_v), np.uint8)
    for s, h in ((0, 0), (1, 17), (2, 31), (3, 6)):
        sel[s, h] = 1
    o_ref, win_ref, S_ref = oracle_seq(ora, wl, inp, head_sel=sel)
    oh, Sh = host(o), host(state.buf)
    cu = inp["cu_seqlens"]
    worst = 0.0
    for s, h in zip(*np.nonzero(sel)):
        r0, r1 = int(cu[s]), int(cu[s + 1])
        ref = o_ref[r0:r1, h]
        worst = max(worst, np.abs(oh[r0:r1, h] - ref).max() / np.abs(ref).max())
        worst = max(worst, np.abs(Sh[s, h] - S_ref[s, h]).max() / np.abs(S_ref[s, h]).max())
    assert worst <= TOL, worst
    np.testing.assert_array_equal(host(conv.buf), win_ref)
    assert not torch.isnan(o).any()


def test_identical_launches_are_bit_identical():
    """Repeated launches on the same inputs give the same bits: outputs,
    states and windows (matrix-core results are read only after their
    write-back has settled)."""
    wl = _small((512, 200, 77, 64), seed=45, h_k=4, h_v=8)
    inp = wk.make_sequence_inputs(wl)
    first = run_seq(wl, inp, chunk=64)
    for _ in range(5):
        again = run_seq(wl, inp, chunk=64)
        assert torch.equal(again[0], first[0])
        assert torch.equal(again[1].buf, first[1].buf)
        assert torch.equal(again[2].buf, first[2].buf)


@pytest.mark.parametrize("d_v", [64, 192])
def test_chunked_other_value_widths(ora, d_v):
    """One and three 64-column blocks per value head (the rolled q/k window
    is handed to the last of r * blocks workgroups)."""
    wl = _small((130, 64, 7), seed=46, h_k=2, h_v=4, d_v=d_v)
    inp = wk.make_sequence_inputs(wl)
    _check(ora, wl, inp)


def test_chunked_more_sequences_than_threads(ora):
    """300 sequences (more than the 256 threads that rank them): the
    longest-first ranking is off and workgroups keep the batch order."""
    rng = np.random.default_rng(47)
    lens = tuple(int(x) for x in rng.integers(1, 70, size=300))
    wl = _small(lens, seed=47, h_k=1, h_v=2, d_v=64)
    inp = wk.make_sequence_inputs(wl)
    _check(ora, wl, inp)


def test_chunked_padding_and_bad_page(ora):
    """A padding sequence (page -1) is skipped and writes nothing; a page
    beyond the pools is skipped and reported (GDN_DEVERR_PAGE); the other
    sequences of the launch still match the oracle, and pages no valid
    sequence names stay untouched."""
    g = gdn()
    wl = _small((130, 64, 70, 65), seed=48)
    inp = wk.make_sequence_inputs(wl)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    pages = [2, -1, 0, 9]
    o, conv, state = run_seq(wl, inp, pages=pages, n_pages=4, chunk=64, err=err)
    assert int(err.item()) & g.GDN_DEVERR_PAGE
    o_ref, win_ref, S_ref = oracle_seq(ora, wl, inp)
    cu = inp["cu_seqlens"]
    oh, Sh, Ch = host(o), host(state.buf), host(conv.buf)
    for s, p in enumerate(pages):
        rows = slice(int(cu[s]), int(cu[s + 1]))
        if p < 0 or p >= 4:
            assert np.isnan(oh[rows]).all(), s
            continue
        assert max_slice_rel_o(oh[rows], o_ref[rows], [0, cu[s + 1] - cu[s]]) <= TOL, s
        assert max_slice_rel_S(Sh[p:p + 1], S_ref[s:s + 1]) <= TOL, s
        np.testing.assert_array_equal(Ch[p], win_ref[s])
    for p in (1, 3):
        assert float(state.buf[p].abs().sum()) == 0.0 and float(conv.buf[p].float().abs().sum()) == 0.0
    assert int(conv.sync.abs().sum()) == 0


def test_chunked_max_seqlen_bounds_the_records(ora):
    """batch.max_seqlen sizes the record pass (ceil(max_seqlen / 64) chunks per
    sequence): a sequence longer than it is skipped, leaves its page and rows
    untouched and raises GDN_DEVERR_BATCH; the others match the oracle."""
    g = gdn()
    wl = _small((130, 64, 70), seed=50)
    inp = wk.make_sequence_inputs(wl)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    o, conv, state = run_seq(wl, inp, chunk=64, err=err, max_seqlen=100)
    assert int(err.item()) == g.GDN_DEVERR_BATCH
    o_ref, win_ref, S_ref = oracle_seq(ora, wl, inp)
    cu = inp["cu_seqlens"]
    oh, Sh, Ch = host(o), host(state.buf), host(conv.buf)
    assert np.isnan(oh[:130]).all()
    np.testing.assert_array_equal(Sh[0], host(dev(inp["S0"][0], state.buf.dtype)))
    np.testing.assert_array_equal(Ch[0][:wl.conv_w - 1], host(dev(inp["window0"][0], conv.buf.dtype)))
    for s in (1, 2):
        rows = slice(int(cu[s]), int(cu[s + 1]))
        assert max_slice_rel_o(oh[rows], o_ref[rows], [0, cu[s + 1] - cu[s]]) <= TOL, s
        assert max_slice_rel_S(Sh[s:s + 1], S_ref[s:s + 1]) <= TOL, s
        np.testing.assert_array_equal(Ch[s][:wl.conv_w - 1], win_ref[s])


@pytest.mark.parametrize("h_k,h_v", [(4, 4), (2, 8)])
def test_chunked_gqa_ratios(ora, h_k, h_v):
    """One and four value heads per key head (the workloads use two): the key
    head's K K^T and Q K^T shared by r value heads, and the window hand-off."""
    wl = _small((130, 64, 7), seed=49, h_k=h_k, h_v=h_v)
    _check(ora, wl, wk.make_sequence_inputs(wl))
