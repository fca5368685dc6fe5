"""Seeded synthetic workloads for the Gated DeltaNet layer core.

This module only draws numbers and fixes shapes; it holds none of the
method's arithmetic (no convolution, gating or recurrence).  Both the HIP
path (through the package binding) and the fp64 oracle (under ``oracle/``)
consume the arrays it returns, so the two sides see identical input values.

Draw recipe (one ``numpy.random.Generator(PCG64(seed))`` per workload, every
draw made in float32 and then rounded to nearest-even into the activation
dtype, bf16 or fp32):

1. conv weights ``w[C_conv][W]``      ~ N(0, 0.25)   (second parameter = std)
2. ``A_log[H_v]``                     = log U[1, 16]   (kept fp32)
3. ``dt_bias[H_v]``                   ~ N(0, 0.1)      (kept fp32)
4. per sequence: ``S0[H_v][d_k][d_v]`` ~ N(0, 0.05)   (zeros when ``s0_std`` is 0)
   then ``window0[W-1][C_conv]``      ~ N(0, 1)       (zeros when ``window_std`` is 0)
5. per sequence, the whole token block: ``x[T][C_conv]`` ~ N(0, 1), then
   ``a[T][H_v]`` ~ N(0, 1), then ``b[T][H_v]`` ~ N(0, 1)
6. speculative verify only, after 4: per step, per request the candidate block
   ``x[n_cand][C_conv]``, ``a``, ``b`` as in 5; then ``accepted[n_steps][n_req]``
   ~ U{0 .. n_cand-1}.

Channel order within a row of ``x`` is [q | k | v], head-major then dim:
``C_conv = 2*H_k*d_k + H_v*d_v``.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional

import numpy as np

BF16 = "bf16"
F32 = "f32"


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    h_k: int
    h_v: int
    d_k: int
    d_v: int
    conv_w: int
    act_dtype: str
    state_dtype: str
    seqlens: tuple = ()          # token-by-token / chunked workloads
    chunk: int = 0               # chunked WY/UT prefill chunk size (0 = token by token)
    n_req: int = 0               # speculative verify
    n_cand: int = 0
    n_steps: int = 0
    s0_std: float = 0.05
    window_std: float = 1.0
    seed: int = 0
    scale: float = 1.0
    l2_eps: float = 1e-6

    @property
    def c_conv(self) -> int:
        return 2 * self.h_k * self.d_k + self.h_v * self.d_v

    @property
    def n_tokens(self) -> int:
        return int(sum(self.seqlens))

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The five workload shapes.  Lengths of the short ragged prefill are the
# prompt lengths of the r9700-stack v0.2.3 first-token table ("1. Time to
# first token", 45 ... 656 tokens) plus the 256-token default prefill
# threshold named beside it.
TINY = Workload("tiny", h_k=2, h_v=2, d_k=32, d_v=32, conv_w=4, act_dtype=F32,
                state_dtype=F32, seqlens=(64,), s0_std=0.0, window_std=0.0, seed=0)
DECODE = Workload("decode", h_k=16, h_v=32, d_k=128, d_v=128, conv_w=4, act_dtype=BF16,
                  state_dtype=F32, seqlens=(1,) * 64, seed=1)
SHORT_PREFILL = Workload("short_prefill", h_k=16, h_v=32, d_k=128, d_v=128, conv_w=4,
                         act_dtype=BF16, state_dtype=F32,
                         seqlens=(45, 83, 159, 236, 320, 404, 656, 256), seed=2)
LONG_PREFILL = Workload("long_prefill", h_k=16, h_v=32, d_k=128, d_v=128, conv_w=4,
                        act_dtype=BF16, state_dtype=F32, seqlens=(8192,) * 4, chunk=64,
                        seed=3)
SPEC_VERIFY = Workload("spec_verify", h_k=16, h_v=32, d_k=128, d_v=128, conv_w=4,
                       act_dtype=BF16, state_dtype=F32, n_req=32, n_cand=8, n_steps=12,
                       seed=4)

WORKLOADS: Dict[str, Workload] = {w.name: w for w in
                                  (TINY, DECODE, SHORT_PREFILL, LONG_PREFILL, SPEC_VERIFY)}


def round_to(arr: np.ndarray, dtype: str) -> np.ndarray:
    """Round float32 draws into ``dtype`` (nearest-even) and return them widened
    exactly to float32 again, so every consumer sees representable values."""
    arr = np.ascontiguousarray(arr, dtype=np.float32)
    if dtype == F32:
        return arr
    if dtype != BF16:
        raise ValueError(dtype)
    bits = arr.view(np.uint32).astype(np.uint64)
    # nearest-even on the upper 16 bits; inputs here are finite draws
    lsb = (bits >> 16) & 1
    bits = (bits + 0x7FFF + lsb) & 0xFFFF0000
    return bits.astype(np.uint32).view(np.float32)


def _normal(rng: np.random.Generator, shape, std: float) -> np.ndarray:
    if std == 0.0:
        return np.zeros(shape, dtype=np.float32)
    return rng.standard_normal(shape, dtype=np.float32) * np.float32(std)


def make_params(wl: Workload, rng: np.random.Generator) -> Dict[str, np.ndarray]:
    C, W = wl.c_conv, wl.conv_w
    conv_w = round_to(_normal(rng, (C, W), 0.25), wl.act_dtype)
    a_log = np.log(rng.uniform(1.0, 16.0, size=wl.h_v)).astype(np.float32)
    dt_bias = _normal(rng, (wl.h_v,), 0.1)
    return {"conv_w": conv_w, "a_log": a_log, "dt_bias": dt_bias}


def make_sequence_inputs(wl: Workload, seed: Optional[int] = None) -> Dict[str, np.ndarray]:
    """Inputs of a token-by-token or chunked workload: one ragged batch."""
    rng = np.random.default_rng(wl.seed if seed is None else seed)
    out = make_params(wl, rng)
    C, W = wl.c_conv, wl.conv_w
    n = len(wl.seqlens)
    S0 = np.zeros((n, wl.h_v, wl.d_k, wl.d_v), dtype=np.float32)
    win = np.zeros((n, W - 1, C), dtype=np.float32)
    N = wl.n_tokens
    x = np.empty((N, C), dtype=np.float32)
    a = np.empty((N, wl.h_v), dtype=np.float32)
    b = np.empty((N, wl.h_v), dtype=np.float32)
    cu = np.zeros(n + 1, dtype=np.int32)
    for s, T in enumerate(wl.seqlens):
        S0[s] = _normal(rng, (wl.h_v, wl.d_k, wl.d_v), wl.s0_std)
        win[s] = _normal(rng, (W - 1, C), wl.window_std)
        cu[s + 1] = cu[s] + T
        r0, r1 = cu[s], cu[s + 1]
        x[r0:r1] = _normal(rng, (T, C), 1.0)
        a[r0:r1] = _normal(rng, (T, wl.h_v), 1.0)
        b[r0:r1] = _normal(rng, (T, wl.h_v), 1.0)
    out.update(
        S0=round_to(S0, wl.state_dtype),
        window0=round_to(win, wl.act_dtype),
        x=round_to(x, wl.act_dtype),
        a=round_to(a, wl.act_dtype),
        b=round_to(b, wl.act_dtype),
        cu_seqlens=cu,
    )
    return out


def make_verify_inputs(wl: Workload, seed: Optional[int] = None) -> Dict[str, np.ndarray]:
    """Inputs of a speculative-verify workload (n_steps x n_req x n_cand rows)."""
    rng = np.random.default_rng(wl.seed if seed is None else seed)
    out = make_params(wl, rng)
    C, W, R, K, St = wl.c_conv, wl.conv_w, wl.n_req, wl.n_cand, wl.n_steps
    S0 = np.zeros((R, wl.h_v, wl.d_k, wl.d_v), dtype=np.float32)
    win = np.zeros((R, W - 1, C), dtype=np.float32)
    for r in range(R):
        S0[r] = _normal(rng, (wl.h_v, wl.d_k, wl.d_v), wl.s0_std)
        win[r] = _normal(rng, (W - 1, C), wl.window_std)
    x = np.empty((St, R, K, C), dtype=np.float32)
    a = np.empty((St, R, K, wl.h_v), dtype=np.float32)
    b = np.empty((St, R, K, wl.h_v), dtype=np.float32)
    for s in range(St):
        for r in range(R):
            x[s, r] = _normal(rng, (K, C), 1.0)
            a[s, r] = _normal(rng, (K, wl.h_v), 1.0)
            b[s, r] = _normal(rng, (K, wl.h_v), 1.0)
    accepted = rng.integers(0, K, size=(St, R), dtype=np.int64).astype(np.int32)
    out.update(
        S0=S0,  # rounded into the state dtype by the caller (fp32 and bf16 runs share draws)
        window0=round_to(win, wl.act_dtype),
        x=round_to(x, wl.act_dtype),
        a=round_to(a, wl.act_dtype),
        b=round_to(b, wl.act_dtype),
        accepted=accepted,
    )
    return out


def split_lengths(cu_seqlens: np.ndarray) -> List[int]:
    return [int(cu_seqlens[i + 1] - cu_seqlens[i]) for i in range(len(cu_seqlens) - 1)]
