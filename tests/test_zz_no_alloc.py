"""GPU test of gdn_recurrent_seq_noalloc, the token-by-token entry point for
callers that cannot allocate: its sync words live in the library's own
device array instead of the caller's conv.sync.  Called through the C ABI,
it must give the results of gdn_recurrent_seq bit for bit (the same
kernels), on two calls in a row with the second smaller, for the decode
shape (the streaming kernel and its work counter) and for a ragged prefill
(the arrival counters of shared windows)."""
import numpy as np
import pytest
import torch

import gdn_workloads as wk
from gpu_util import DEV, dev, gdn, make_batch, params_of, seq_pools

pytestmark = pytest.mark.gpu


def _pair(wl, inp):
    """Identical pools for the two entry points, the batch, and both outputs."""
    g = gdn()
    n = len(wl.seqlens)
    pages = list(range(n))
    d1, conv1, st1 = seq_pools(wl, inp, pages, n)
    _, conv2, st2 = seq_pools(wl, inp, pages, n)
    x, a, b = (dev(inp[k], d1.act_torch) for k in ("x", "a", "b"))
    batch = make_batch(inp["cu_seqlens"], pages, x.shape[0])
    o1 = torch.full((x.shape[0], wl.h_v, wl.d_v), float("nan"), device=DEV)
    o2 = o1.clone()
    return g, d1, params_of(inp, wl), x, a, b, batch, (conv1, st1, o1), (conv2, st2, o2)


def _run_and_compare(wl, inp):
    g, dims, params, x, a, b, batch, ref, got = _pair(wl, inp)
    err1 = torch.zeros(1, dtype=torch.int32, device=DEV)
    err2 = torch.zeros(1, dtype=torch.int32, device=DEV)
    g.gdn_recurrent_seq(dims, params, x, a, b, batch, ref[0], ref[1], o=ref[2], err=err1)
    g.gdn_recurrent_seq_noalloc(dims, params, x, a, b, batch, got[0], got[1], got[2], err=err2)
    torch.cuda.synchronize()
    assert not torch.isnan(got[2]).any()
    assert torch.equal(got[2], ref[2])
    assert torch.equal(got[1].buf, ref[1].buf)
    assert torch.equal(got[0].buf, ref[0].buf)
    assert int(err1.item()) == 0 and int(err2.item()) == 0
    assert int(got[0].sync.abs().sum()) == 0     # the caller's sync words were never touched


@pytest.mark.parametrize("shape", ["decode", "prefill"])
def test_noalloc_equals_recurrent_seq_twice_second_smaller(shape):
    if shape == "decode":
        first = wk.DECODE                                         # 64 sequences x 1 token
        second = wk.DECODE.replace(seqlens=(1,) * 24, seed=11)    # fewer sequences and pages
    else:
        first = wk.SHORT_PREFILL.replace(h_k=4, h_v=8, seqlens=(45, 83, 159, 17), seed=12)
        second = first.replace(seqlens=(9, 30), seed=13)
    for wl in (first, second):
        _run_and_compare(wl, wk.make_sequence_inputs(wl))


def test_noalloc_rejects_more_pages_than_its_array_holds():
    g = gdn()
    wl = wk.DECODE.replace(seqlens=(1,) * 2)
    inp = wk.make_sequence_inputs(wl)
    _, dims, params, x, a, b, batch, ref, _ = _pair(wl, inp)
    big = g.ConvPool.alloc(dims, g.GDN_NOALLOC_SYNC_WORDS // dims.h_k + 1, 3, DEV)
    with pytest.raises(g.GdnError) as e:
        g.gdn_recurrent_seq_noalloc(dims, params, x, a, b, batch, big, ref[1], ref[2])
    assert e.value.status == 1
