"""ctypes front end of the fp64 oracle (``gdn_oracle.c``).

TEST INFRASTRUCTURE ONLY.  Every function takes and returns numpy arrays;
inputs are widened exactly to float64 before the call, so the oracle consumes
the same values the HIP path is given.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

_dp = ctypes.POINTER(ctypes.c_double)
_fp = ctypes.POINTER(ctypes.c_float)
_ip = ctypes.POINTER(ctypes.c_int32)
_up = ctypes.POINTER(ctypes.c_uint8)


class OraDims(ctypes.Structure):
    _fields_ = [("h_k", ctypes.c_int32), ("h_v", ctypes.c_int32), ("d_k", ctypes.c_int32),
                ("d_v", ctypes.c_int32), ("conv_w", ctypes.c_int32),
                ("scale", ctypes.c_double), ("l2_eps", ctypes.c_double)]


def lib():
    global _lib
    if _lib is None:
        src = os.path.join(_HERE, "gdn_oracle.c")
        if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(src):
            from . import build as _b
            _b.build()
        L = ctypes.CDLL(_LIB_PATH)
        for name in ("ora_silu", "ora_softplus", "ora_sigmoid", "ora_round_bf16"):
            getattr(L, name).restype = ctypes.c_double
            getattr(L, name).argtypes = [ctypes.c_double]
        L.ora_decay.restype = ctypes.c_double
        L.ora_decay.argtypes = [ctypes.c_double] * 3
        L.ora_layer.restype = ctypes.c_int
        L.ora_verify.restype = ctypes.c_int
        L.ora_conv_update.restype = ctypes.c_int
        L.ora_book_step.restype = ctypes.c_int
        _lib = L
    return _lib


def _d(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float64)


def _ptr(a: np.ndarray, t=_dp):
    return a.ctypes.data_as(t)


def dims(h_k, h_v, d_k, d_v, conv_w=4, scale=1.0, l2_eps=1e-6) -> OraDims:
    return OraDims(h_k, h_v, d_k, d_v, conv_w, scale, l2_eps)


def dims_of(wl) -> OraDims:
    return dims(wl.h_k, wl.h_v, wl.d_k, wl.d_v, wl.conv_w, wl.scale, wl.l2_eps)


# ----------------------------------------------------------------- scalars
def silu(z: float) -> float:
    return lib().ora_silu(float(z))


def softplus(u: float) -> float:
    return lib().ora_softplus(float(u))


def sigmoid(b: float) -> float:
    return lib().ora_sigmoid(float(b))


def decay(a: float, a_log: float, dt_bias: float) -> float:
    return lib().ora_decay(float(a), float(a_log), float(dt_bias))


def round_bf16(x: float) -> float:
    return lib().ora_round_bf16(float(x))


def round_bf16_array(x) -> np.ndarray:
    x = _d(x).copy()
    lib().ora_round_bf16_array(_ptr(x), ctypes.c_int64(x.size))
    return x


# -------------------------------------------------------------------- conv
def conv_seq(x, w, window=None, act=True):
    """Causal depthwise conv of one sequence: x [T][C], w [C][W], window [W-1][C].
    Returns (y [T][C], window_out [W-1][C])."""
    x, w = _d(x), _d(w)
    T, C = x.shape
    W = w.shape[1]
    y = np.zeros((T, C))
    wo = np.zeros((W - 1, C))
    win = _d(window) if window is not None else None
    lib().ora_conv_seq(ctypes.c_int32(T), ctypes.c_int32(C), ctypes.c_int32(W), _ptr(x), _ptr(w),
                       _ptr(win) if win is not None else None, ctypes.c_int32(1 if act else 0),
                       _ptr(y), _ptr(wo))
    return y, wo


def conv_f32_model(x, w, window=None):
    """fp32 single-FMA-chain conv (no activation), oldest tap first."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    w = np.ascontiguousarray(w, dtype=np.float32)
    T, C = x.shape
    W = w.shape[1]
    y = np.zeros((T, C), dtype=np.float32)
    win = np.ascontiguousarray(window, dtype=np.float32) if window is not None else None
    lib().ora_conv_f32_model(ctypes.c_int32(T), ctypes.c_int32(C), ctypes.c_int32(W),
                             _ptr(x, _fp), _ptr(w, _fp),
                             _ptr(win, _fp) if win is not None else None, _ptr(y, _fp))
    return y


def conv_update(x, conv_w, cu_seqlens, window, has_init=None, act=True):
    """Conv over a ragged batch.  window [n][W-1][C] is rolled in a copy.
    Returns (y [N][C], window_out)."""
    x, conv_w = _d(x), _d(conv_w)
    N, C = x.shape
    W = conv_w.shape[1]
    cu = np.ascontiguousarray(cu_seqlens, dtype=np.int32)
    n = len(cu) - 1
    win = _d(window).copy()
    hi = None if has_init is None else np.ascontiguousarray(has_init, dtype=np.uint8)
    y = np.zeros((N, C))
    rc = lib().ora_conv_update(ctypes.c_int32(C), ctypes.c_int32(W), _ptr(conv_w), _ptr(x),
                               _ptr(cu, _ip), ctypes.c_int32(n),
                               _ptr(hi, _up) if hi is not None else None, _ptr(win),
                               ctypes.c_int32(1 if act else 0), _ptr(y))
    assert rc == 0
    return y, win


# ------------------------------------------------------------ gating, rule
def gate_row(dm: OraDims, y, a, b, a_log, dt_bias):
    y, a, b, a_log, dt_bias = map(_d, (y, a, b, a_log, dt_bias))
    qn = np.zeros((dm.h_k, dm.d_k))
    kn = np.zeros((dm.h_k, dm.d_k))
    v = np.zeros((dm.h_v, dm.d_v))
    g = np.zeros(dm.h_v)
    beta = np.zeros(dm.h_v)
    lib().ora_gate_row(ctypes.byref(dm), _ptr(y), _ptr(a), _ptr(b), _ptr(a_log), _ptr(dt_bias),
                       _ptr(qn), _ptr(kn), _ptr(v), _ptr(g), _ptr(beta))
    return qn, kn, v, g, beta


def delta_rule(q, k, v, g, beta, S0, scale=1.0, chunk=0):
    """One value head: q, k [T][dk], v [T][dv], g, beta [T], S0 [dk][dv].
    chunk == 0: token by token; chunk > 0: chunked WY/UT form.
    Returns (o [T][dv], S [dk][dv])."""
    q, k, v, g, beta = map(_d, (q, k, v, g, beta))
    T, dk = q.shape
    dv = v.shape[1]
    S = _d(S0).copy()
    o = np.zeros((T, dv))
    L = lib()
    if chunk > 0:
        L.ora_chunked_rule(ctypes.c_int32(T), ctypes.c_int32(dk), ctypes.c_int32(dv),
                           ctypes.c_int32(chunk), ctypes.c_double(scale), _ptr(q), _ptr(k),
                           ctypes.c_int64(dk), _ptr(v), ctypes.c_int64(dv), _ptr(g), _ptr(beta),
                           _ptr(S), _ptr(o), ctypes.c_int64(dv))
    else:
        L.ora_delta_rule(ctypes.c_int32(T), ctypes.c_int32(dk), ctypes.c_int32(dv),
                         ctypes.c_double(scale), _ptr(q), _ptr(k), ctypes.c_int64(dk), _ptr(v),
                         ctypes.c_int64(dv), _ptr(g), _ptr(beta), _ptr(S), _ptr(o),
                         ctypes.c_int64(dv))
    return o, S


# ------------------------------------------------------------ whole layer
def layer(dm: OraDims, conv_w, a_log, dt_bias, x, a, b, cu_seqlens, window0, S0,
          has_init=None, chunk=0, head_sel: Optional[np.ndarray] = None):
    """The layer core over a ragged batch.  Returns (o [N][H_v][d_v],
    window [n][W-1][C], S [n][H_v][d_k][d_v])."""
    conv_w, a_log, dt_bias, x, a, b = map(_d, (conv_w, a_log, dt_bias, x, a, b))
    cu = np.ascontiguousarray(cu_seqlens, dtype=np.int32)
    n = len(cu) - 1
    N = x.shape[0]
    win = _d(window0).copy()
    S = _d(S0).copy()
    o = np.zeros((N, dm.h_v, dm.d_v))
    hi = None if has_init is None else np.ascontiguousarray(has_init, dtype=np.uint8)
    hs = None if head_sel is None else np.ascontiguousarray(head_sel, dtype=np.uint8)
    rc = lib().ora_layer(ctypes.byref(dm), _ptr(conv_w), _ptr(a_log), _ptr(dt_bias), _ptr(x),
                         _ptr(a), _ptr(b), _ptr(cu, _ip), ctypes.c_int32(n),
                         _ptr(hi, _up) if hi is not None else None, _ptr(win), _ptr(S), _ptr(o),
                         ctypes.c_int32(chunk), _ptr(hs, _up) if hs is not None else None)
    if rc != 0:
        raise ValueError(f"ora_layer returned {rc}")
    return o, win, S


def verify(dm: OraDims, conv_w, a_log, dt_bias, x, a, b, accepted, window0, S0,
           state_bf16=False):
    """Speculative-verify semantics.  x [steps][req][cand][C], a, b [..][H_v],
    accepted [steps][req].  Returns (o [steps][req][cand][H_v][d_v],
    committed window [req][W-1][C], committed state [req][H_v][d_k][d_v])."""
    conv_w, a_log, dt_bias, x, a, b = map(_d, (conv_w, a_log, dt_bias, x, a, b))
    St, R, K = x.shape[:3]
    acc = np.ascontiguousarray(accepted, dtype=np.int32)
    win = _d(window0).copy()
    S = _d(S0).copy()
    o = np.zeros((St, R, K, dm.h_v, dm.d_v))
    rc = lib().ora_verify(ctypes.byref(dm), _ptr(conv_w), _ptr(a_log), _ptr(dt_bias),
                          ctypes.c_int32(R), ctypes.c_int32(St), ctypes.c_int32(K), _ptr(x),
                          _ptr(a), _ptr(b), _ptr(acc, _ip), ctypes.c_int32(1 if state_bf16 else 0),
                          _ptr(win), _ptr(S), _ptr(o))
    if rc != 0:
        raise ValueError(f"ora_verify returned {rc}")
    return o, win, S


# ------------------------------------------------- verify page bookkeeping
BOOK_ACCEPTED, BOOK_PARITY, BOOK_ARG = 1, 2, 16


def book_step(W: int, n_spec: int, hdr, cbuf, x, num_accepted: int, parity: int):
    """One verify step's page bookkeeping for one request (``ora_book_step``).
    hdr: 4 uint32 {flag, n_rows[0], n_rows[1], accepted}; cbuf [rows][C] conv
    buffer; x [n_cand][C] candidate rows (n_cand may be 0).  Returns
    (err, hdr', cbuf', info) with info = (a, replayed rows, replayed slot,
    written slot); on a refusal hdr' and cbuf' equal the inputs."""
    h = np.ascontiguousarray(hdr, dtype=np.uint32).copy()
    cb = _d(cbuf).copy()
    rows, C = cb.shape
    xx = _d(x).reshape(-1, C) if x is not None else np.zeros((0, C))
    out = np.zeros(4, dtype=np.int32)
    err = lib().ora_book_step(ctypes.c_int32(W), ctypes.c_int32(n_spec), ctypes.c_int32(C), ctypes.c_int32(rows),
                              ctypes.c_int32(xx.shape[0]), ctypes.c_int32(int(num_accepted)),
                              ctypes.c_int32(int(parity)), h.ctypes.data_as(ctypes.POINTER(ctypes.c_uint32)),
                              _ptr(cb), _ptr(xx), _ptr(out, _ip))
    return int(err), h, cb, tuple(int(v) for v in out)


def book_batch(W: int, n_spec: int, hdrs, cbufs, req_page, x, num_accepted, parity):
    """The bookkeeping of one verify step over a request batch: request r
    works on page req_page[r] (< 0: padding, nothing touched; >= the number
    of pages: refused, nothing touched).  hdrs [n_pages][4], cbufs
    [n_pages][rows][C], x [n_req][n_cand][C].  Returns (per-request error
    codes, with -1 for a page out of range, hdrs', cbufs')."""
    hdrs = np.ascontiguousarray(hdrs, dtype=np.uint32).copy()
    cbufs = _d(cbufs).copy()
    errs = []
    for r, p in enumerate(req_page):
        p = int(p)
        if p < 0:
            errs.append(0)
            continue
        if p >= hdrs.shape[0]:
            errs.append(-1)
            continue
        e, h, cb, _ = book_step(W, n_spec, hdrs[p], cbufs[p], x[r] if x is not None else None,
                                num_accepted[r], parity[r])
        errs.append(e)
        if e == 0:
            hdrs[p], cbufs[p] = h, cb
    return errs, hdrs, cbufs


def max_rel(y, ref) -> float:
    """max |y - ref| / max |ref| over the whole array (the tests apply it per
    (tensor, sequence, head) slice)."""
    y = np.asarray(y, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.max(np.abs(ref)) if ref.size else 0.0
    num = np.max(np.abs(y - ref)) if ref.size else 0.0
    if den == 0.0:
        return float(num)
    return float(num / den)
