"""Helpers of the GPU parity tests: upload seeded workloads, run libgdn
through the binding, run the oracle on the same values, compare slices."""
from __future__ import annotations

import numpy as np
import torch

import gdn_workloads as wk

DEV = "cuda:0"
TORCH_DT = {wk.F32: torch.float32, wk.BF16: torch.bfloat16}


def gdn():
    import linear_attention_ssm_gdn_amd as g
    g.load()
    return g


def dims_of(wl: wk.Workload, **kw):
    g = gdn()
    base = dict(h_k=wl.h_k, h_v=wl.h_v, d_k=wl.d_k, d_v=wl.d_v, conv_w=wl.conv_w,
                n_spec=max(wl.n_cand - 1, 0), act_dtype=wl.act_dtype, state_dtype=wl.state_dtype,
                scale=wl.scale, l2_eps=wl.l2_eps)
    base.update(kw)
    return g.Dims(**base)


def dev(arr, dt) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32)).to(DEV).to(dt)


def params_of(inp, wl):
    g = gdn()
    return g.Params(dev(inp["conv_w"], TORCH_DT[wl.act_dtype]), dev(inp["a_log"], torch.float32),
                    dev(inp["dt_bias"], torch.float32))


def host(t: torch.Tensor) -> np.ndarray:
    return t.detach().to(torch.float64).cpu().numpy()


def make_batch(cu, pages, n_rows, has_init=None, max_seqlen=None):
    g = gdn()
    cu = np.asarray(cu, dtype=np.int32)
    lens = np.diff(cu)
    return g.Batch(torch.from_numpy(cu).to(DEV), torch.as_tensor(np.asarray(pages, np.int32)).to(DEV),
                   None if has_init is None else torch.as_tensor(np.asarray(has_init, np.uint8)).to(DEV),
                   int(lens.max()) if max_seqlen is None and len(lens) else int(max_seqlen or 0), int(n_rows))


def seq_pools(wl, inp, pages, n_pages, conv_rows=None, dims=None):
    """Conv and state pools with each sequence's initial window/state at its page."""
    g = gdn()
    dims = dims or dims_of(wl)
    conv = g.ConvPool.alloc(dims, n_pages, conv_rows or wl.conv_w - 1, DEV)
    state = g.StatePool.alloc(dims, n_pages, DEV)
    for s, p in enumerate(pages):
        if p < 0 or p >= n_pages:
            continue
        conv.buf[p, :wl.conv_w - 1] = dev(inp["window0"][s], dims.act_torch)
        state.buf[p] = dev(inp["S0"][s], dims.state_torch)
    return dims, conv, state


def run_seq(wl, inp, pages=None, n_pages=None, has_init=None, chunk=0, err=None, conv_rows=None,
            dims=None, max_seqlen=None):
    g = gdn()
    n = len(wl.seqlens)
    pages = list(range(n)) if pages is None else pages
    n_pages = n_pages or (max(pages) + 1 if len(pages) else 1)
    dims, conv, state = seq_pools(wl, inp, pages, n_pages, conv_rows, dims)
    params = params_of(inp, wl)
    x = dev(inp["x"], dims.act_torch)
    a = dev(inp["a"], dims.act_torch)
    b = dev(inp["b"], dims.act_torch)
    batch = make_batch(inp["cu_seqlens"], pages, x.shape[0], has_init, max_seqlen)
    o = torch.full((x.shape[0], wl.h_v, wl.d_v), float("nan"), device=DEV)
    if chunk:
        g.gdn_chunked_prefill(dims, params, x, a, b, batch, conv, state, chunk=chunk, o=o, err=err)
    else:
        g.gdn_recurrent_seq(dims, params, x, a, b, batch, conv, state, o=o, err=err)
    torch.cuda.synchronize()
    return o, conv, state


def oracle_seq(ora, wl, inp, has_init=None, chunk=0, head_sel=None):
    dm = ora.dims_of(wl)
    return ora.layer(dm, inp["conv_w"], inp["a_log"], inp["dt_bias"], inp["x"], inp["a"], inp["b"],
                     inp["cu_seqlens"], inp["window0"], inp["S0"], has_init=has_init, chunk=chunk,
                     head_sel=head_sel)


def rel(y, ref) -> float:
    y = np.asarray(y, np.float64)
    ref = np.asarray(ref, np.float64)
    den = np.abs(ref).max() if ref.size else 0.0
    num = np.abs(y - ref).max() if ref.size else 0.0
    return float(num / den) if den > 0 else float(num)


def max_slice_rel_o(o, o_ref, cu, heads=None):
    """max over (sequence, head) slices of max|o - ref| / max|ref|."""
    worst = 0.0
    for s in range(len(cu) - 1):
        r0, r1 = int(cu[s]), int(cu[s + 1])
        if r1 == r0:
            continue
        for h in range(o_ref.shape[1]) if heads is None else heads:
            worst = max(worst, rel(o[r0:r1, h], o_ref[r0:r1, h]))
    return worst


def max_slice_rel_S(S, S_ref):
    worst = 0.0
    for s in range(S_ref.shape[0]):
        for h in range(S_ref.shape[1]):
            worst = max(worst, rel(S[s, h], S_ref[s, h]))
    return worst


class BookModel:
    """The oracle's bookkeeping model of verify pages (oracle.book_batch),
    stepped beside a GPU run: headers (flag, n_rows, acceptance echo), the
    whole conv buffer of every page and the sticky error bits, compared bit
    for bit with the GPU's after each step."""

    def __init__(self, dims, n_pages, rows, req_page, window0):
        import oracle
        self.ora = oracle
        self.W, self.n_spec = dims.conv_w, dims.n_spec
        C = dims.c_conv
        self.hdr = np.zeros((n_pages, 4), np.uint32)
        self.cbuf = np.zeros((n_pages, rows, C))
        for r, p in enumerate(req_page):
            if 0 <= p < n_pages:
                self.cbuf[p, :self.W - 1] = window0[r]
        self.own = sorted(p for p in req_page if 0 <= p < n_pages)  # the pages this run's requests use
        self.err = 0

    def step(self, req_page, x, accepted, parity):
        g = gdn()
        errs, self.hdr, self.cbuf = self.ora.book_batch(self.W, self.n_spec, self.hdr, self.cbuf, req_page, x,
                                                        accepted, parity)
        bits = {0: 0, -1: g.GDN_DEVERR_PAGE, self.ora.BOOK_ACCEPTED: g.GDN_DEVERR_ACCEPTED,
                self.ora.BOOK_PARITY: g.GDN_DEVERR_PARITY}
        for e in errs:
            self.err |= bits[e]
        return errs

    def check(self, pages, conv, err):
        own = self.own
        got_hdr = pages.header()[own, :4].cpu().numpy().view(np.uint32)
        np.testing.assert_array_equal(got_hdr, self.hdr[own])
        np.testing.assert_array_equal(host(conv.buf[own]), self.cbuf[own])
        assert int(err.item()) == self.err


class VerifyRun:
    """A request batch stepping through speculative verify on the GPU."""

    def __init__(self, wl, inp, layout, state_dtype, pages_of=None, n_pages=None, pages=None, conv=None):
        """pages / conv: pools shared with other runs (other layers); by
        default the run allocates its own."""
        g = gdn()
        self.g, self.wl, self.inp = g, wl, inp
        self.dims = dims_of(wl, state_dtype=state_dtype, n_spec=wl.n_cand - 1)
        R = wl.n_req
        self.req_page = list(range(R)) if pages_of is None else list(pages_of)
        n_pages = n_pages or (max(self.req_page) + 1)
        self.pages = pages if pages is not None else g.SpecPages.alloc(self.dims, layout, n_pages, DEV)
        self.conv = conv if conv is not None else g.ConvPool.alloc(self.dims, n_pages, 3 + self.dims.n_spec, DEV)
        st = self.pages.states()
        for r, p in enumerate(self.req_page):
            if p < 0:
                continue
            st[p, 0] = dev(inp["S0"][r], self.dims.state_torch)
            self.conv.buf[p, :3] = dev(inp["window0"][r], self.dims.act_torch)
        self.params = params_of(inp, wl)
        self.rp = torch.tensor(self.req_page, dtype=torch.int32, device=DEV)
        self.err = torch.zeros(1, dtype=torch.int32, device=DEV)
        self.step_no = 0
        # the oracle's page bookkeeping, stepped beside the GPU and compared after every step
        self.book = BookModel(self.dims, n_pages, 3 + self.dims.n_spec, self.req_page, inp["window0"])

    def step(self, s, accepted_prev, n_cand=None, parity=None, cache=None, cache_entry=None, cache_row=None,
             refused=()):
        """Step s with the previous step's acceptance counts.  With `cache`
        (a PrefixCache) the step also writes cache_entry[r] <- the prefix that
        ends at replayed row cache_row[r].  `refused`: requests the device is
        expected to refuse for their cache arguments (their pages untouched,
        GDN_DEVERR_CACHE)."""
        wl, inp = self.wl, self.inp
        R, K = wl.n_req, wl.n_cand if n_cand is None else n_cand
        C = wl.c_conv
        acc = torch.tensor(np.asarray(accepted_prev, np.int32), device=DEV)
        par = (self.step_no + 1) & 1 if parity is None else parity
        pt = torch.full((R,), par, dtype=torch.uint8, device=DEV)
        if K > 0:
            x = dev(inp["x"][s][:, :K].reshape(R * K, C), self.dims.act_torch)
            a = dev(inp["a"][s][:, :K].reshape(R * K, wl.h_v), self.dims.act_torch)
            b = dev(inp["b"][s][:, :K].reshape(R * K, wl.h_v), self.dims.act_torch)
            o = torch.full((R * K, wl.h_v, wl.d_v), float("nan"), device=DEV)
        else:
            x = a = b = o = None
        kw = {}
        if cache is not None:
            kw = dict(cache=cache, cache_entry=torch.tensor(np.asarray(cache_entry, np.int32), device=DEV),
                      cache_row=torch.tensor(np.asarray(cache_row, np.int32), device=DEV))
        self.g.gdn_spec_verify(self.dims, self.params, self.pages, x, a, b, R, K, self.rp, acc, pt, self.conv,
                               o=o, err=self.err, **kw)
        if parity is None:
            self.step_no += 1
        torch.cuda.synchronize()
        stepped = [(-1 if r in refused else p) for r, p in enumerate(self.req_page)]
        self.book.step(stepped, inp["x"][s][:, :K] if K > 0 else None, accepted_prev, [par] * R)
        if refused:
            self.book.err |= self.g.GDN_DEVERR_CACHE
        self.book.check(self.pages, self.conv, self.err)
        return None if o is None else o.view(R, K, wl.h_v, wl.d_v)

    def clear_err(self):
        self.err.zero_()
        self.book.err = 0

    def run(self):
        wl, inp = self.wl, self.inp
        outs = []
        for s in range(wl.n_steps):
            prev = inp["accepted"][s - 1] if s > 0 else np.zeros(wl.n_req, np.int32)
            outs.append(self.step(s, prev))
        self.step(0, inp["accepted"][wl.n_steps - 1], n_cand=0)  # commit the last acceptance
        return torch.stack(outs)  # [steps][R][K][h_v][d_v]

    def committed_state(self):
        return self.pages.states()[self.req_page, 0]

    def committed_window(self):
        return self.conv.buf[self.req_page, :3]
