"""GPU tests of gdn_prefill, the host-side switch between the token-by-token
and chunked paths ("r9700-stack v0.2.3", section "1. Time to first token"):
whichever path it reports, its outputs, final states and rolled windows
match the fp64 oracle at that path's tolerance (1e-4 token by token, 3e-3
for the bf16 matrix-core chunked form), are bit-identical to a direct call
of that path on the same inputs, and the path agrees with
gdn_prefill_path."""
import numpy as np
import pytest
import torch

import gdn_workloads as wk
from gpu_util import (DEV, dev, gdn, host, make_batch, max_slice_rel_o, max_slice_rel_S, oracle_seq, params_of,
                      run_seq, seq_pools)

pytestmark = pytest.mark.gpu


def _wl(lens, seed, h_k=4, h_v=8):
    return wk.SHORT_PREFILL.replace(name="prefill_switch", h_k=h_k, h_v=h_v, seqlens=tuple(lens), seed=seed)


def run_prefill(wl, inp, token_max=-1):
    g = gdn()
    n = len(wl.seqlens)
    pages = list(range(n))
    dims, conv, state = seq_pools(wl, inp, pages, n)
    params = params_of(inp, wl)
    x = dev(inp["x"], dims.act_torch)
    a = dev(inp["a"], dims.act_torch)
    b = dev(inp["b"], dims.act_torch)
    batch = make_batch(inp["cu_seqlens"], pages, x.shape[0])
    o = torch.full((x.shape[0], wl.h_v, wl.d_v), float("nan"), device=DEV)
    want = g.gdn_prefill_path(dims, batch, token_max)
    o, path = g.gdn_prefill(dims, params, x, a, b, batch, conv, state, token_max=token_max, o=o)
    torch.cuda.synchronize()
    assert path == want
    return o, conv, state, path


def _oracle_parity(ora, wl, inp, got):
    """o, final states and rolled windows of a gdn_prefill run against the
    oracle's layer, at the tolerance of the path it took."""
    o, conv, state, path = got
    tol = 1e-4 if path == gdn().GDN_PATH_TOKEN else 3e-3
    o_ref, win_ref, S_ref = oracle_seq(ora, wl, inp)
    cu = inp["cu_seqlens"]
    assert max_slice_rel_o(host(o), o_ref, cu) <= tol
    lens = np.diff(cu)
    live = [i for i in range(len(lens)) if lens[i] > 0]
    assert max_slice_rel_S(host(state.buf)[live], S_ref[live]) <= tol
    np.testing.assert_array_equal(host(conv.buf[:, :wl.conv_w - 1]), win_ref)


def _same(r1, r2):
    o1, c1, s1 = r1[:3]
    o2, c2, s2 = r2[:3]
    assert torch.equal(o1, o2)
    assert torch.equal(c1.buf, c2.buf)
    assert torch.equal(s1.buf, s2.buf)


@pytest.mark.parametrize("lens", [(16, 9, 1, 16), (32, 5)])
def test_short_batches_run_token_by_token(ora, lens):
    wl = _wl(lens, seed=61)
    inp = wk.make_sequence_inputs(wl)
    got = run_prefill(wl, inp)
    assert got[3] == gdn().GDN_PATH_TOKEN
    _oracle_parity(ora, wl, inp, got)
    _same(got, run_seq(wl, inp))


@pytest.mark.parametrize("lens", [(333, 64, 129), (33,), (17, 3, 2, 9, 5), (30, 5, 3, 20)])
def test_longer_batches_run_chunked(ora, lens):
    wl = _wl(lens, seed=62)
    inp = wk.make_sequence_inputs(wl)
    got = run_prefill(wl, inp)
    assert got[3] == gdn().GDN_PATH_CHUNKED
    _oracle_parity(ora, wl, inp, got)
    _same(got, run_seq(wl, inp, chunk=64))


def test_explicit_threshold_overrides_the_default(ora):
    wl = _wl((200, 77), seed=63)
    inp = wk.make_sequence_inputs(wl)
    got = run_prefill(wl, inp, token_max=1 << 30)
    assert got[3] == gdn().GDN_PATH_TOKEN
    _oracle_parity(ora, wl, inp, got)
    _same(got, run_seq(wl, inp))
    short = _wl((8, 8), seed=64)
    inp = wk.make_sequence_inputs(short)
    got = run_prefill(short, inp, token_max=0)
    assert got[3] == gdn().GDN_PATH_CHUNKED
    _oracle_parity(ora, short, inp, got)
    _same(got, run_seq(short, inp, chunk=64))
    assert not np.isnan(got[0].cpu().numpy()).any()


@pytest.mark.parametrize("token_max,path", [(-1, 1), (1 << 30, 0)])
def test_short_prefill_workload_through_the_selector(ora, token_max, path):
    """The whole short-prefill batch (8 sequences, 45..656 rows, H_k = 16,
    H_v = 32, d = 128) as a server would send it: with the default
    threshold it takes the chunked path (3e-3 against the oracle), with a
    large threshold the token-by-token path (1e-4)."""
    wl = wk.SHORT_PREFILL
    inp = wk.make_sequence_inputs(wl)
    got = run_prefill(wl, inp, token_max=token_max)
    assert got[3] == path
    _oracle_parity(ora, wl, inp, got)
