"""Thin torch-facing binding of libgdn: argument marshalling only.

Every function here turns torch tensors into the device pointers, strides and
sizes of the matching C entry point of include/gdn.h, calls it on the current
HIP stream and raises on a non-OK status.  All computation happens in the
library's kernels; nothing here has a CPU path.
"""
from __future__ import annotations

import ctypes
import dataclasses
from typing import Optional

import torch

from . import _lib as L

_DT = {"f32": L.GDN_F32, "bf16": L.GDN_BF16}
_TORCH_DT = {"f32": torch.float32, "bf16": torch.bfloat16}


class GdnError(RuntimeError):
    def __init__(self, fn: str, status: int):
        msg = L.load().gdn_status_str(status).decode()
        super().__init__(f"{fn}: status {status} ({msg})")
        self.status = status


def _check(fn: str, st: int) -> None:
    if st != L.GDN_OK:
        raise GdnError(fn, st)


@dataclasses.dataclass(frozen=True)
class Dims:
    h_k: int
    h_v: int
    d_k: int
    d_v: int
    conv_w: int = 4
    n_spec: int = 0
    act_dtype: str = "bf16"
    state_dtype: str = "f32"
    scale: float = 1.0
    l2_eps: float = 1e-6

    @property
    def c_conv(self) -> int:
        return 2 * self.h_k * self.d_k + self.h_v * self.d_v

    @property
    def act_torch(self) -> torch.dtype:
        return _TORCH_DT[self.act_dtype]

    @property
    def state_torch(self) -> torch.dtype:
        return _TORCH_DT[self.state_dtype]

    def c(self) -> L.GdnDims:
        return L.GdnDims(self.h_k, self.h_v, self.d_k, self.d_v, self.conv_w, self.n_spec,
                         _DT[self.act_dtype], _DT[self.state_dtype], self.scale, self.l2_eps)


@dataclasses.dataclass
class Params:
    conv_w: torch.Tensor   # [C_conv][conv_w], act dtype
    a_log: torch.Tensor    # [h_v] fp32
    dt_bias: torch.Tensor  # [h_v] fp32

    def c(self) -> L.GdnParams:
        return L.GdnParams(self.conv_w.data_ptr(), self.a_log.data_ptr(), self.dt_bias.data_ptr())


@dataclasses.dataclass
class Batch:
    cu_seqlens: torch.Tensor            # [n+1] int32 (device)
    page_idx: torch.Tensor              # [n] int32 (device)
    has_init: Optional[torch.Tensor]    # [n] uint8 (device) or None
    max_seqlen: int                     # host bound of every length, 0 if unknown
    n_rows: int                         # rows of x / a / b / o

    @property
    def n_seqs(self) -> int:
        return int(self.page_idx.numel())

    def c(self) -> L.GdnBatch:
        return L.GdnBatch(self.cu_seqlens.data_ptr(), self.page_idx.data_ptr(),
                          self.has_init.data_ptr() if self.has_init is not None else None,
                          self.n_seqs, self.max_seqlen, self.n_rows)


@dataclasses.dataclass
class ConvPool:
    buf: torch.Tensor    # [n_pages][rows][C_conv], act dtype
    sync: torch.Tensor   # [n_pages * h_k + 1] int32: arrival counters, then the work counter; zero between calls

    @staticmethod
    def alloc(dims: Dims, n_pages: int, rows: int, device) -> "ConvPool":
        return ConvPool(torch.zeros((n_pages, rows, dims.c_conv), dtype=dims.act_torch, device=device),
                        torch.zeros((n_pages * dims.h_k + 1,), dtype=torch.int32, device=device))

    def c(self) -> L.GdnConvPool:
        n, rows, C = self.buf.shape
        return L.GdnConvPool(self.buf.data_ptr(), self.buf.stride(0), rows, n, self.sync.data_ptr())


@dataclasses.dataclass
class StatePool:
    buf: torch.Tensor    # [n_pages][h_v][d_k][d_v], state dtype

    @staticmethod
    def alloc(dims: Dims, n_pages: int, device) -> "StatePool":
        return StatePool(torch.zeros((n_pages, dims.h_v, dims.d_k, dims.d_v), dtype=dims.state_torch,
                                     device=device))

    def c(self) -> L.GdnStatePool:
        return L.GdnStatePool(self.buf.data_ptr(), self.buf.stride(0), self.buf.shape[0])


def _stream(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


def _rows(t: torch.Tensor, name: str) -> int:
    if t.dim() != 2 or t.stride(1) != 1:
        raise ValueError(f"{name} must be a 2-D tensor with unit inner stride")
    return t.stride(0)


def _ptr(t: Optional[torch.Tensor]):
    return t.data_ptr() if t is not None else None


def gdn_abi_version() -> int:
    return L.load().gdn_abi_version()


def gdn_spec_page_layout(dims: Dims, layout: int) -> dict:
    out = L.GdnSpecLayout()
    d = dims.c()
    _check("gdn_spec_page_layout", L.load().gdn_spec_page_layout(ctypes.byref(d), layout, ctypes.byref(out)))
    return {f: int(getattr(out, f)) for f, _ in L.GdnSpecLayout._fields_}


def gdn_chunked_workspace_bytes(dims: Dims, n_seqs: int, n_rows: int, chunk: int) -> int:
    out = ctypes.c_size_t(0)
    d = dims.c()
    _check("gdn_chunked_workspace_bytes",
           L.load().gdn_chunked_workspace_bytes(ctypes.byref(d), n_seqs, n_rows, chunk, ctypes.byref(out)))
    return int(out.value)


def gdn_conv_update(dims: Dims, conv_w: torch.Tensor, x: torch.Tensor, batch: Batch, conv: ConvPool,
                    activation: bool = True, y: Optional[torch.Tensor] = None, y_dtype: str = "f32",
                    err: Optional[torch.Tensor] = None) -> torch.Tensor:
    if y is None:
        y = torch.empty((batch.n_rows, dims.c_conv), dtype=_TORCH_DT[y_dtype], device=x.device)
    d, b = dims.c(), batch.c()
    st = L.load().gdn_conv_update(ctypes.byref(d), conv_w.data_ptr(), x.data_ptr(), _rows(x, "x"),
                                  ctypes.byref(b), conv.c(), 1 if activation else 0, y.data_ptr(),
                                  _DT[y_dtype], _rows(y, "y"), _ptr(err), _stream(x))
    _check("gdn_conv_update", st)
    return y


def gdn_recurrent_seq(dims: Dims, params: Params, x: torch.Tensor, a: torch.Tensor, b: torch.Tensor,
                      batch: Batch, conv: ConvPool, state: StatePool, o: Optional[torch.Tensor] = None,
                      err: Optional[torch.Tensor] = None) -> torch.Tensor:
    if o is None:
        o = torch.empty((batch.n_rows, dims.h_v, dims.d_v), dtype=torch.float32, device=x.device)
    if a.stride() != b.stride():
        raise ValueError("a and b must share their row stride")
    d, p, bt = dims.c(), params.c(), batch.c()
    st = L.load().gdn_recurrent_seq(ctypes.byref(d), ctypes.byref(p), x.data_ptr(), _rows(x, "x"),
                                    a.data_ptr(), b.data_ptr(), _rows(a, "a"), ctypes.byref(bt), conv.c(),
                                    state.c(), o.data_ptr(), _ptr(err), _stream(x))
    _check("gdn_recurrent_seq", st)
    return o


def gdn_recurrent_seq_noalloc(dims: Dims, params: Params, x: torch.Tensor, a: torch.Tensor, b: torch.Tensor,
                              batch: Batch, conv: ConvPool, state: StatePool, o: torch.Tensor,
                              err: Optional[torch.Tensor] = None) -> torch.Tensor:
    """gdn_recurrent_seq with its sync words in the library's own device
    array: conv.sync is not passed, and o must be given (nothing is
    allocated on the way)."""
    if a.stride() != b.stride():
        raise ValueError("a and b must share their row stride")
    d, p, bt = dims.c(), params.c(), batch.c()
    n, rows, C = conv.buf.shape
    cp = L.GdnConvPool(conv.buf.data_ptr(), conv.buf.stride(0), rows, n, None)
    st = L.load().gdn_recurrent_seq_noalloc(ctypes.byref(d), ctypes.byref(p), x.data_ptr(), _rows(x, "x"),
                                            a.data_ptr(), b.data_ptr(), _rows(a, "a"), ctypes.byref(bt), cp,
                                            state.c(), o.data_ptr(), _ptr(err), _stream(x))
    _check("gdn_recurrent_seq_noalloc", st)
    return o


def gdn_chunked_prefill(dims: Dims, params: Params, x: torch.Tensor, a: torch.Tensor, b: torch.Tensor,
                        batch: Batch, conv: ConvPool, state: StatePool, chunk: int = 64,
                        o: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                        err: Optional[torch.Tensor] = None) -> torch.Tensor:
    if o is None:
        o = torch.empty((batch.n_rows, dims.h_v, dims.d_v), dtype=torch.float32, device=x.device)
    if a.stride() != b.stride():
        raise ValueError("a and b must share their row stride")
    need = gdn_chunked_workspace_bytes(dims, batch.n_seqs, batch.n_rows, chunk)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    d, p, bt = dims.c(), params.c(), batch.c()
    st = L.load().gdn_chunked_prefill(ctypes.byref(d), ctypes.byref(p), x.data_ptr(), _rows(x, "x"),
                                      a.data_ptr(), b.data_ptr(), _rows(a, "a"), ctypes.byref(bt), conv.c(),
                                      state.c(), o.data_ptr(), chunk, _ptr(workspace),
                                      workspace.numel() if workspace is not None else 0, _ptr(err), _stream(x))
    _check("gdn_chunked_prefill", st)
    return o


def gdn_prefill_path(dims: Dims, batch: Batch, token_max: int = L.GDN_PREFILL_MAX_DEFAULT) -> int:
    out = ctypes.c_int32(-1)
    d, bt = dims.c(), batch.c()
    _check("gdn_prefill_path", L.load().gdn_prefill_path(ctypes.byref(d), ctypes.byref(bt), token_max,
                                                         ctypes.byref(out)))
    return int(out.value)


def gdn_prefill(dims: Dims, params: Params, x: torch.Tensor, a: torch.Tensor, b: torch.Tensor, batch: Batch,
                conv: ConvPool, state: StatePool, token_max: int = L.GDN_PREFILL_MAX_DEFAULT,
                o: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                err: Optional[torch.Tensor] = None):
    """Returns (o, path): path is GDN_PATH_TOKEN or GDN_PATH_CHUNKED."""
    if o is None:
        o = torch.empty((batch.n_rows, dims.h_v, dims.d_v), dtype=torch.float32, device=x.device)
    if a.stride() != b.stride():
        raise ValueError("a and b must share their row stride")
    if workspace is None:
        need = gdn_chunked_workspace_bytes(dims, batch.n_seqs, batch.n_rows, 64)
        if need > 0:
            workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    path = ctypes.c_int32(-1)
    d, p, bt = dims.c(), params.c(), batch.c()
    st = L.load().gdn_prefill(ctypes.byref(d), ctypes.byref(p), x.data_ptr(), _rows(x, "x"), a.data_ptr(),
                              b.data_ptr(), _rows(a, "a"), ctypes.byref(bt), conv.c(), state.c(), o.data_ptr(),
                              token_max, _ptr(workspace), workspace.numel() if workspace is not None else 0,
                              ctypes.byref(path), _ptr(err), _stream(x))
    _check("gdn_prefill", st)
    return o, int(path.value)


@dataclasses.dataclass
class SpecPages:
    """Speculative pages: raw bytes [n_pages][page_bytes] laid out by
    gdn_spec_page_layout (header, state, record)."""
    buf: torch.Tensor
    layout: int
    lay: dict
    dims: Dims

    @staticmethod
    def alloc(dims: Dims, layout: int, n_pages: int, device) -> "SpecPages":
        lay = gdn_spec_page_layout(dims, layout)
        buf = torch.zeros((n_pages, lay["page_bytes"]), dtype=torch.uint8, device=device)
        return SpecPages(buf, layout, lay, dims)

    @property
    def n_slots(self) -> int:
        return 1 if self.layout == L.GDN_SPEC_ONEPAGE else self.dims.n_spec + 1

    def header(self) -> torch.Tensor:
        """[n_pages][64] uint32 view of every page header."""
        return self.buf[:, self.lay["header_off"]:self.lay["header_off"] + 256].view(torch.int32)

    def checkpoint_pool(self) -> "StatePool":
        """A state pool aliased onto the pages' checkpoints (slot 0): a
        sequence call through it writes its final states into the pages."""
        return StatePool(self.states()[:, 0])

    def states(self) -> torch.Tensor:
        """[n_pages][n_slots][h_v][d_k][d_v] view of the state region."""
        d = self.dims
        es = 2 if d.state_dtype == "bf16" else 4
        nbytes = self.n_slots * d.h_v * d.d_k * d.d_v * es
        off = self.lay["state_off"]
        return self.buf[:, off:off + nbytes].view(d.state_torch).view(
            self.buf.shape[0], self.n_slots, d.h_v, d.d_k, d.d_v)


@dataclasses.dataclass
class PrefixCache:
    """Cached committed prefixes: entry e holds a state (state pool page e)
    and the conv window that ends with it (conv pool page e, rows 0..W-2)."""
    state: StatePool
    conv: ConvPool

    @staticmethod
    def alloc(dims: Dims, n_entries: int, device) -> "PrefixCache":
        return PrefixCache(StatePool.alloc(dims, n_entries, device),
                           ConvPool.alloc(dims, n_entries, dims.conv_w - 1, device))

    def c(self, entry: Optional[torch.Tensor] = None, row: Optional[torch.Tensor] = None) -> L.GdnPrefixCache:
        return L.GdnPrefixCache(_ptr(entry), _ptr(row), self.state.c(), self.conv.c())


def gdn_spec_verify(dims: Dims, params: Params, pages: SpecPages, x: Optional[torch.Tensor],
                    a: Optional[torch.Tensor], b: Optional[torch.Tensor], n_req: int, n_cand: int,
                    req_page: torch.Tensor, num_accepted: torch.Tensor, step_parity: torch.Tensor,
                    conv: ConvPool, o: Optional[torch.Tensor] = None,
                    err: Optional[torch.Tensor] = None, cache: Optional[PrefixCache] = None,
                    cache_entry: Optional[torch.Tensor] = None,
                    cache_row: Optional[torch.Tensor] = None) -> Optional[torch.Tensor]:
    """gdn_spec_verify, or gdn_spec_verify_cached when `cache` is given (with
    int32 device tensors cache_entry and cache_row, one entry per request)."""
    dev = req_page.device
    if o is None and n_cand > 0:
        o = torch.empty((n_req * n_cand, dims.h_v, dims.d_v), dtype=torch.float32, device=dev)
    xs = _rows(x, "x") if x is not None else 0
    abs_ = _rows(a, "a") if a is not None else 0
    d, p = dims.c(), params.c()
    args = (ctypes.byref(d), ctypes.byref(p), pages.layout, _ptr(x), xs, _ptr(a), _ptr(b), abs_, n_req, n_cand,
            req_page.data_ptr(), num_accepted.data_ptr(), step_parity.data_ptr(), pages.buf.data_ptr(),
            pages.buf.stride(0), pages.buf.shape[0], conv.c())
    stream = torch.cuda.current_stream(dev).cuda_stream
    if cache is None:
        st = L.load().gdn_spec_verify(*args, _ptr(o), _ptr(err), stream)
        _check("gdn_spec_verify", st)
    else:
        if cache_entry is None or cache_row is None:
            raise ValueError("a prefix cache needs cache_entry and cache_row")
        pc = cache.c(cache_entry, cache_row)
        st = L.load().gdn_spec_verify_cached(*args, ctypes.byref(pc), _ptr(o), _ptr(err), stream)
        _check("gdn_spec_verify_cached", st)
    return o


def gdn_prefix_restore(dims: Dims, pages: SpecPages, entry: torch.Tensor, req_page: torch.Tensor,
                       cache: PrefixCache, conv: ConvPool, err: Optional[torch.Tensor] = None) -> None:
    """Restore cached prefixes entry[r] into pages req_page[r] (fresh headers)."""
    d = dims.c()
    pc = cache.c()
    st = L.load().gdn_prefix_restore(ctypes.byref(d), pages.layout, int(entry.numel()), entry.data_ptr(),
                                     req_page.data_ptr(), ctypes.byref(pc), pages.buf.data_ptr(),
                                     pages.buf.stride(0), pages.buf.shape[0], conv.c(), _ptr(err),
                                     torch.cuda.current_stream(entry.device).cuda_stream)
    _check("gdn_prefix_restore", st)


def _mixed_parts(seq: Optional[dict], verify: Optional[dict]):
    """ctypes structs of a mixed step's parts (None where a part is absent),
    the objects they point into, and the tensor whose stream is used."""
    sp = vp = None
    keep = []
    stream_of = None
    if seq is not None:
        if seq["a"].stride() != seq["b"].stride():
            raise ValueError("a and b must share their row stride")
        bt = seq["batch"].c()
        keep.append(bt)
        spg = seq.get("spec_pages")
        sp = L.GdnSeqPart(seq["x"].data_ptr(), _rows(seq["x"], "x"), seq["a"].data_ptr(), seq["b"].data_ptr(),
                          _rows(seq["a"], "a"), ctypes.pointer(bt), seq["conv"].c(), seq["state"].c(),
                          seq["o"].data_ptr(), spg.buf.data_ptr() if spg is not None else None,
                          spg.buf.stride(0) if spg is not None else 0, spg.buf.shape[0] if spg is not None else 0)
        stream_of = seq["x"]
    if verify is not None:
        v = verify
        pages = v["pages"]
        x, a, b = v.get("x"), v.get("a"), v.get("b")
        vp = L.GdnVerifyPart(pages.layout, _ptr(x), _rows(x, "x") if x is not None else 0, _ptr(a), _ptr(b),
                             _rows(a, "a") if a is not None else 0, v["n_req"], v["n_cand"],
                             v["req_page"].data_ptr(), v["num_accepted"].data_ptr(), v["step_parity"].data_ptr(),
                             pages.buf.data_ptr(), pages.buf.stride(0), pages.buf.shape[0], v["conv"].c(),
                             _ptr(v.get("o")))
        stream_of = stream_of if stream_of is not None else v["req_page"]
    return sp, vp, keep, stream_of


def gdn_mixed_launches(dims: Dims, seq: Optional[dict] = None, verify: Optional[dict] = None) -> int:
    """The launch count gdn_mixed_step uses for these parts (host only):
    GDN_MIXED_ONE_LAUNCH or GDN_MIXED_TWO_LAUNCHES."""
    d = dims.c()
    sp, vp, keep, _ = _mixed_parts(seq, verify)
    out = ctypes.c_int32(0)
    st = L.load().gdn_mixed_launches(ctypes.byref(d), ctypes.byref(sp) if sp is not None else None,
                                     ctypes.byref(vp) if vp is not None else None, ctypes.byref(out))
    _check("gdn_mixed_launches", st)
    return int(out.value)


def gdn_mixed_step(dims: Dims, params: Params, seq: Optional[dict] = None, verify: Optional[dict] = None,
                   err: Optional[torch.Tensor] = None, launches: int = L.GDN_MIXED_AUTO) -> None:
    """A step mixing token-by-token sequences and verify requests: one
    launch, or two where gdn_mixed_launches picks them (launches overrides:
    GDN_MIXED_ONE_LAUNCH / GDN_MIXED_TWO_LAUNCHES; the results are the same
    bit for bit).

    seq:    dict(x, a, b, batch, conv, state, o) -- the arguments of gdn_recurrent_seq, and
            optionally spec_pages (SpecPages) whose headers the sequences leave fresh
    verify: dict(pages, x, a, b, n_req, n_cand, req_page, num_accepted, step_parity, conv, o)
            -- the arguments of gdn_spec_verify (pages: SpecPages)
    Outputs are written into the o tensors given."""
    d, p = dims.c(), params.c()
    sp, vp, keep, stream_of = _mixed_parts(seq, verify)
    if stream_of is None:
        return
    st = L.load().gdn_mixed_step_launches(ctypes.byref(d), ctypes.byref(p),
                                          ctypes.byref(sp) if sp is not None else None,
                                          ctypes.byref(vp) if vp is not None else None, int(launches), _ptr(err),
                                          torch.cuda.current_stream(stream_of.device).cuda_stream)
    _check("gdn_mixed_step", st)
