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
