"""Benchmark of the GDN layer core on one MI355X.

Headline: the decode workload (64 sequences x 1 token, H_k=16, H_v=32,
d_k=d_v=128, bf16 activations, fp32 state), one fused conv + gating +
delta-rule launch per step, reported in microseconds per step for one
layer, against the HBM roofline of its algorithmic bytes.  The other
workloads (short ragged prefill, long chunked prefill, speculative verify)
are reported beside it under "other_workloads".

Inputs are seeded synthetic data (gdn_workloads) already resident in HBM when
the timed region starts.  Every workload rotates through enough copies of
its state, page and input buffers that the bytes it touches between two
uses of one copy are at least 512 MiB, twice the 256 MB last-level cache,
so no launch reads what an earlier launch left in that cache.  Kernel time
is taken with HIP events on the stream the kernels are launched on.

usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--only decode,...] [--sweep-dispatch]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import gdn_workloads as wk  # noqa: E402

METRIC = "GDN tokens/s/layer (prefill) + decode/verify µs/step at B=64; % HBM/MFMA roofline"
HBM_PEAK_GBS = 8000.0            # MI355X HBM3E, GB/s
BF16_MFMA_PEAK_TFLOPS = 2500.0   # dense bf16 matrix cores
FP32_VALU_PEAK_TFLOPS = 157.3    # fp32 vector (256 CU x 4 SIMD x 16 lanes x 2 (FMA) x 2 (packed) x 2.4 GHz)
# the build disables packed fp32 instructions, so one lane retires at most
# one fp32 FMA per cycle: half the published figure
FP32_VALU_REACHABLE_TFLOPS = 78.6
ROTATION_BYTES = 512 << 20       # bytes touched between two uses of one buffer copy
MIN_POOLS = 2
POOLS = 4                        # the dispatch sweep's state copies (its inputs are shared)
WARM_S = 0.3                     # least untimed launch time before each secondary workload is timed
LAST_PERCENTILES = {}  # per-launch kernel time percentiles (us) of the last measure()


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def failed(other, name, e):
    """Record a workload that raised, so the JSON line still comes out."""
    log(f"{name}: failed: {type(e).__name__}: {e}")
    other[name] = {"value": None, "error": f"{type(e).__name__}: {e}"}


# ------------------------------------------------------------ byte / flop models
def decode_bytes(wl) -> int:
    """Algorithmic HBM bytes of one token-by-token launch: every byte the
    layer must read or write once."""
    n = len(wl.seqlens)
    N = wl.n_tokens
    act = 2 if wl.act_dtype == wk.BF16 else 4
    st = 2 if wl.state_dtype == wk.BF16 else 4
    state = n * wl.h_v * wl.d_k * wl.d_v * st * 2          # read + write
    x = N * wl.c_conv * act
    window = n * (wl.conv_w - 1) * wl.c_conv * act * 2    # read + write
    o = N * wl.h_v * wl.d_v * 4
    w = wl.c_conv * wl.conv_w * act
    ab = N * wl.h_v * act * 2
    params = wl.h_v * 4 * 2
    return state + x + window + o + w + ab + params


def recurrence_flops(wl) -> int:
    """fp32 flops of the token-by-token recurrence: per token and value head
    7 d_k d_v (S^T k and S^T q: 2 each; decay, outer product, add: 3)."""
    return wl.n_tokens * wl.h_v * 7 * wl.d_k * wl.d_v


def chunked_flops(wl) -> int:
    """Canonical flops of the chunked WY/UT form: per value head and token
    6 d_k d_v + 2C d_k + 4C d_v + 2C^2/3, plus per key head and token 4C d_k."""
    C, dk, dv = wl.chunk, wl.d_k, wl.d_v
    per_v = 6 * dk * dv + 2 * C * dk + 4 * C * dv + 2 * C * C / 3
    per_k = 4 * C * dk
    return int(wl.n_tokens * (wl.h_v * per_v + wl.h_k * per_k))


def chunked_bytes(wl) -> int:
    n = len(wl.seqlens)
    N = wl.n_tokens
    act = 2 if wl.act_dtype == wk.BF16 else 4
    return (N * wl.c_conv * act + N * wl.h_v * wl.d_v * 4 + N * wl.h_v * act * 2
            + n * wl.h_v * wl.d_k * wl.d_v * 4 * 2 + n * (wl.conv_w - 1) * wl.c_conv * act * 2)


def verify_bytes(wl, state_dtype, mean_replay) -> int:
    """Algorithmic bytes of one one-page verify step: checkpoint read+write,
    replayed record rows read, new record rows written, candidate rows, conv
    buffer (window read + rolled buffer written), outputs."""
    R, K = wl.n_req, wl.n_cand
    st = 2 if state_dtype == wk.BF16 else 4
    act = 2 if wl.act_dtype == wk.BF16 else 4
    row = (wl.c_conv + 2 * wl.h_v) * 4
    state = R * wl.h_v * wl.d_k * wl.d_v * st * 2
    rec = R * (mean_replay + K) * row
    x = R * K * (wl.c_conv + 2 * wl.h_v) * act
    conv = R * (3 + 2 + K) * wl.c_conv * act
    o = R * K * wl.h_v * wl.d_v * 4
    return int(state + rec + x + conv + o)


# ------------------------------------------------------------------- runners
class Timer:
    """Per-launch HIP event pairs on the current stream."""

    def __init__(self, torch):
        self.torch = torch
        self.pairs = []

    def time(self, fn):
        t = self.torch
        s, e = t.cuda.Event(enable_timing=True), t.cuda.Event(enable_timing=True)
        s.record()
        fn()
        e.record()
        self.pairs.append((s, e))

    def mean_ms(self):
        return float(np.mean([s.elapsed_time(e) for s, e in self.pairs]))

    def percentiles_us(self):
        t = np.array([s.elapsed_time(e) for s, e in self.pairs]) * 1e3
        return {"p10": round(float(np.percentile(t, 10)), 2), "p50": round(float(np.percentile(t, 50)), 2),
                "p90": round(float(np.percentile(t, 90)), 2)}


def _upload(torch, arr, dt):
    return torch.from_numpy(np.ascontiguousarray(arr, np.float32)).to("cuda").to(dt)


def pools_for(set_bytes: int) -> int:
    """Copies of a workload's buffers so that one rotation touches at least
    ROTATION_BYTES."""
    return max(MIN_POOLS, -(-ROTATION_BYTES // max(int(set_bytes), 1)))


def _nbytes(*ts) -> int:
    return int(sum(t.numel() * t.element_size() for t in ts))


class SeqWorkload:
    """Token-by-token (or chunked) layer over one ragged batch; enough copies
    of inputs, windows, states and outputs to rotate through >= 512 MiB."""

    def __init__(self, g, torch, wl, chunk=0):
        self.g, self.torch, self.wl, self.chunk = g, torch, wl, chunk
        inp = wk.make_sequence_inputs(wl)
        self.inp = inp
        d = g.Dims(wl.h_k, wl.h_v, wl.d_k, wl.d_v, wl.conv_w, 0, wl.act_dtype, wl.state_dtype, wl.scale,
                   wl.l2_eps)
        self.dims = d
        self.params = g.Params(_upload(torch, inp["conv_w"], d.act_torch), _upload(torch, inp["a_log"], torch.float32),
                               _upload(torch, inp["dt_bias"], torch.float32))
        n = len(wl.seqlens)
        lens = np.diff(inp["cu_seqlens"])
        self.batch = g.Batch(torch.from_numpy(inp["cu_seqlens"]).cuda(), torch.arange(n, dtype=torch.int32).cuda(),
                             None, int(lens.max()), int(wl.n_tokens))
        self.sets = []
        x = _upload(torch, inp["x"], d.act_torch)
        a = _upload(torch, inp["a"], d.act_torch)
        b = _upload(torch, inp["b"], d.act_torch)
        S0 = _upload(torch, inp["S0"], d.state_torch)
        W0 = _upload(torch, inp["window0"], d.act_torch)
        o_bytes = wl.n_tokens * wl.h_v * wl.d_v * 4
        self.set_bytes = _nbytes(x, a, b, S0, W0) + o_bytes
        self.pools = pools_for(self.set_bytes)
        for _ in range(self.pools):
            conv = g.ConvPool.alloc(d, n, wl.conv_w - 1, "cuda")
            conv.buf.copy_(W0)
            state = g.StatePool(S0.clone())
            o = torch.empty((wl.n_tokens, wl.h_v, wl.d_v), device="cuda")
            self.sets.append((x.clone(), a.clone(), b.clone(), conv, state, o))
        self.i = 0

    def rotation(self) -> dict:
        return {"pools": self.pools, "bytes_per_pool": self.set_bytes, "rotation_bytes": self.pools * self.set_bytes}

    def launch(self):
        x, a, b, conv, state, o = self.sets[self.i % self.pools]
        self.i += 1
        if self.chunk:
            self.g.gdn_chunked_prefill(self.dims, self.params, x, a, b, self.batch, conv, state, chunk=self.chunk,
                                       o=o)
        else:
            self.g.gdn_recurrent_seq(self.dims, self.params, x, a, b, self.batch, conv, state, o=o)


class VerifyWorkload:
    """Speculative verify steps over n_req requests; enough page sets (pages,
    conv buffers, outputs) to rotate through >= 512 MiB."""

    def __init__(self, g, torch, wl, state_dtype, layout=0):
        self.g, self.torch, self.wl = g, torch, wl
        inp = wk.make_verify_inputs(wl)
        d = g.Dims(wl.h_k, wl.h_v, wl.d_k, wl.d_v, wl.conv_w, wl.n_cand - 1, wl.act_dtype, state_dtype,
                   wl.scale, wl.l2_eps)
        self.dims = d
        self.params = g.Params(_upload(torch, inp["conv_w"], d.act_torch), _upload(torch, inp["a_log"], torch.float32),
                               _upload(torch, inp["dt_bias"], torch.float32))
        R, K, C = wl.n_req, wl.n_cand, wl.c_conv
        self.x = [_upload(torch, inp["x"][s].reshape(R * K, C), d.act_torch) for s in range(wl.n_steps)]
        self.a = [_upload(torch, inp["a"][s].reshape(R * K, wl.h_v), d.act_torch) for s in range(wl.n_steps)]
        self.b = [_upload(torch, inp["b"][s].reshape(R * K, wl.h_v), d.act_torch) for s in range(wl.n_steps)]
        self.acc = [torch.from_numpy(inp["accepted"][s]).cuda() for s in range(wl.n_steps)]
        self.mean_replay = float(np.mean(inp["accepted"]) + 1.0)
        self.rp = torch.arange(R, dtype=torch.int32, device="cuda")
        self.sets = []
        lay = g.gdn_spec_page_layout(d, layout)
        act = 2 if wl.act_dtype == wk.BF16 else 4
        self.set_bytes = R * lay["page_bytes"] + R * (3 + d.n_spec) * C * act + R * K * wl.h_v * wl.d_v * 4
        self.pools = pools_for(self.set_bytes)
        for _ in range(self.pools):
            pages = g.SpecPages.alloc(d, layout, R, "cuda")
            pages.states()[:, 0] = _upload(torch, inp["S0"], d.state_torch)
            conv = g.ConvPool.alloc(d, R, 3 + d.n_spec, "cuda")
            conv.buf[:, :3] = _upload(torch, inp["window0"], d.act_torch)
            o = torch.empty((R * K, wl.h_v, wl.d_v), device="cuda")
            self.sets.append([pages, conv, o, 0])
        self.i = 0
        self.par = [torch.full((R,), p, dtype=torch.uint8, device="cuda") for p in (0, 1)]

    def rotation(self) -> dict:
        return {"pools": self.pools, "bytes_per_pool": self.set_bytes, "rotation_bytes": self.pools * self.set_bytes}

    def launch(self):
        st = self.sets[self.i % self.pools]
        self.i += 1
        pages, conv, o, n = st
        s = n % self.wl.n_steps
        acc = self.acc[(n - 1) % self.wl.n_steps] if n > 0 else self.acc[0] * 0
        self.g.gdn_spec_verify(self.dims, self.params, pages, self.x[s], self.a[s], self.b[s], self.wl.n_req,
                               self.wl.n_cand, self.rp, acc, self.par[(n + 1) & 1], conv, o=o)
        st[3] = n + 1


class MixedWorkload:
    """A serving step mixing the short ragged prefill batch with the verify
    batch (32 requests x 8 candidates, fp32 state): one gdn_mixed_step launch
    (fused) or gdn_recurrent_seq then gdn_spec_verify (separate).  Both
    parts use the verify workload's parameters, so the two forms compute the
    same step."""

    def __init__(self, g, torch, seq_wl=wk.SHORT_PREFILL, ver_wl=wk.SPEC_VERIFY):
        self.g = g
        self.seq = SeqWorkload(g, torch, seq_wl)
        self.ver = VerifyWorkload(g, torch, ver_wl, wk.F32)
        self.fused = True
        self.launches = g.GDN_MIXED_AUTO  # gdn_mixed_step's launch choice when fused

    def chosen_launches(self) -> int:
        sw, vw = self.seq, self.ver
        x, a, b, conv, state, o = sw.sets[0]
        pages, vconv, vo, _ = vw.sets[0]
        return self.g.gdn_mixed_launches(vw.dims, seq=dict(x=x, a=a, b=b, batch=sw.batch, conv=conv, state=state,
                                                           o=o),
                                         verify=dict(pages=pages, x=vw.x[0], a=vw.a[0], b=vw.b[0],
                                                     n_req=vw.wl.n_req, n_cand=vw.wl.n_cand, req_page=vw.rp,
                                                     num_accepted=vw.acc[0], step_parity=vw.par[0], conv=vconv,
                                                     o=vo))

    def launch(self):
        g, sw, vw = self.g, self.seq, self.ver
        x, a, b, conv, state, o = sw.sets[sw.i % sw.pools]
        sw.i += 1
        st = vw.sets[vw.i % vw.pools]
        vw.i += 1
        pages, vconv, vo, n = st
        s = n % vw.wl.n_steps
        acc = vw.acc[(n - 1) % vw.wl.n_steps] if n > 0 else vw.acc[0] * 0
        par = vw.par[(n + 1) & 1]
        if self.fused:
            g.gdn_mixed_step(vw.dims, vw.params, seq=dict(x=x, a=a, b=b, batch=sw.batch, conv=conv, state=state, o=o),
                             verify=dict(pages=pages, x=vw.x[s], a=vw.a[s], b=vw.b[s], n_req=vw.wl.n_req,
                                         n_cand=vw.wl.n_cand, req_page=vw.rp, num_accepted=acc, step_parity=par,
                                         conv=vconv, o=vo), launches=self.launches)
        else:
            g.gdn_recurrent_seq(vw.dims, vw.params, x, a, b, sw.batch, conv, state, o=o)
            g.gdn_spec_verify(vw.dims, vw.params, pages, vw.x[s], vw.a[s], vw.b[s], vw.wl.n_req, vw.wl.n_cand,
                              vw.rp, acc, par, vconv, o=vo)
        st[3] = n + 1


def measure(torch, wload, steps, warmup, min_warm_s=0.0):
    """Time `steps` launches after `warmup` untimed ones; with min_warm_s the
    untimed launches go on until that much wall time has passed too (the
    VALU-bound kernels run several percent slow for their first hundred or so
    launches after the GPU has been idle)."""
    t_w = time.perf_counter()
    n = 0
    while n < warmup or time.perf_counter() - t_w < min_warm_s:
        wload.launch()
        n += 1
        if n % 16 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    timer = Timer(torch)
    t0 = time.perf_counter()
    for _ in range(steps):
        timer.time(wload.launch)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / steps
    LAST_PERCENTILES.clear()
    LAST_PERCENTILES.update(timer.percentiles_us())
    return timer.mean_ms(), wall * 1e3


# --------------------------------------------------------------- traffic file
def kernel_source_hash() -> str:
    """Hash of the device sources (kernels, their launchers and headers; the
    host-side argument checks and path selection do not change a kernel's
    traffic)."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "linear_attention_ssm_gdn_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        if not f.endswith((".hip", ".hpp", ".h")):
            continue
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def read_traffic(kernel: str, workload: str):
    """HBM bytes per launch from profiles/hbm_traffic.txt, if they were taken
    on the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic.txt")
    if not os.path.exists(path):
        return None
    src = kernel_source_hash()
    for line in open(path):
        f = line.split()
        if len(f) < 4 or f[0] != "traffic" or f[1] != kernel or f[2] != workload:
            continue
        kv = dict(t.split("=", 1) for t in f[3:] if "=" in t)
        if kv.get("src") == src:
            return float(kv["bytes"])
    return None


# ---------------------------------------------------------- denominators
def measured_copy_gbs(torch, nbytes=1 << 30, reps=10):
    """Bandwidth of a plain device-to-device copy of nbytes (torch's copy
    kernel), read + write bytes over HIP-event time: the second denominator
    of every HBM fraction."""
    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    t = Timer(torch)
    for _ in range(reps):
        t.time(lambda: dst.copy_(src))
    torch.cuda.synchronize()
    gbs = 2 * nbytes / (t.mean_ms() * 1e-3) / 1e9
    del src, dst
    torch.cuda.empty_cache()
    return {"value": round(gbs, 1), "unit": "GB/s", "kernel": "torch copy_ (device to device)",
            "bytes_moved": 2 * nbytes}


def measured_gemm_tflops(torch, n=8192, reps=10):
    """Dense bf16 matrix-core throughput of a library GEMM (torch.matmul on
    two contiguous n x n bf16 matrices, fp32 accumulation): the measured
    second denominator of the chunked path's matrix-core fraction."""
    a = torch.randn((n, n), device="cuda").to(torch.bfloat16).contiguous()
    b = torch.randn((n, n), device="cuda").to(torch.bfloat16).contiguous()
    for _ in range(3):
        c = torch.matmul(a, b)
    torch.cuda.synchronize()
    t = Timer(torch)
    for _ in range(reps):
        t.time(lambda: torch.matmul(a, b))
    torch.cuda.synchronize()
    tf = 2.0 * n ** 3 / (t.mean_ms() * 1e-3) / 1e12
    del a, b, c
    torch.cuda.empty_cache()
    return {"value": round(tf, 1), "unit": "TFLOP/s", "kernel": f"torch.matmul bf16 {n}x{n}x{n}"}


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


# ---------------------------------------------------------------- cpu leg
def cpu_baseline(wl, budget_s=12.0):
    """The fp64 oracle on the decode workload, repeated for about budget_s."""
    import oracle as ora
    inp = wk.make_sequence_inputs(wl)
    dm = ora.dims_of(wl)
    args = (inp["conv_w"], inp["a_log"], inp["dt_bias"], inp["x"], inp["a"], inp["b"], inp["cu_seqlens"],
            inp["window0"], inp["S0"])
    ora.layer(dm, *args)  # load + warm
    n, t0 = 0, time.perf_counter()
    while time.perf_counter() - t0 < budget_s:
        ora.layer(dm, *args)
        n += 1
    dt = (time.perf_counter() - t0) / n
    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    return {"value": round(dt * 1e6, 1), "unit": "us/step", "cores": threads, "kind": "oracle",
            "cpu_model": cpu_model(), "host_cpus": os.cpu_count(),
            "sample": f"the full decode step ({len(wl.seqlens)} seqs x 1 token, all {wl.h_v} heads), "
                      f"repeated {n} times in {budget_s:.0f} s"}


def cpu_other_workloads(budget_s=4.0):
    """The fp64 oracle on bounded samples of the other workloads (context
    beside each GPU figure; the headline's baseline is cpu_baseline)."""
    import oracle as ora
    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    out = {}

    def timed(fn):
        fn()  # load + warm
        n, t0 = 0, time.perf_counter()
        while n == 0 or time.perf_counter() - t0 < budget_s:
            fn()
            n += 1
        return (time.perf_counter() - t0) / n, n

    # short prefill: the whole ragged batch
    wl = wk.SHORT_PREFILL
    inp = wk.make_sequence_inputs(wl)
    dm = ora.dims_of(wl)
    dt, n = timed(lambda: ora.layer(dm, inp["conv_w"], inp["a_log"], inp["dt_bias"], inp["x"], inp["a"], inp["b"],
                                    inp["cu_seqlens"], inp["window0"], inp["S0"]))
    out["short_prefill"] = {"value": round(wl.n_tokens / dt), "unit": "tokens/s/layer", "cores": threads,
                            "kind": "oracle", "sample": f"the whole batch ({wl.n_tokens} tokens), {n} runs"}
    # long prefill: the first 1024 tokens of one sequence (the oracle's cost is linear in tokens)
    T = 1024
    wl = wk.LONG_PREFILL.replace(seqlens=(T,))
    inp = wk.make_sequence_inputs(wl)
    dm = ora.dims_of(wl)
    dt, n = timed(lambda: ora.layer(dm, inp["conv_w"], inp["a_log"], inp["dt_bias"], inp["x"], inp["a"], inp["b"],
                                    inp["cu_seqlens"], inp["window0"], inp["S0"]))
    out["long_prefill"] = {"value": round(T / dt), "unit": "tokens/s/layer", "cores": threads, "kind": "oracle",
                           "sample": f"one sequence of {T} tokens, all {wl.h_v} heads, {n} runs (sequential form)"}
    # verify: all steps of the workload, per step
    wl = wk.SPEC_VERIFY
    inp = wk.make_verify_inputs(wl)
    dm = ora.dims_of(wl)
    dt, n = timed(lambda: ora.verify(dm, inp["conv_w"], inp["a_log"], inp["dt_bias"], inp["x"], inp["a"], inp["b"],
                                     inp["accepted"], inp["window0"], inp["S0"]))
    out["spec_verify"] = {"value": round(dt / wl.n_steps * 1e6, 1), "unit": "us/step", "cores": threads,
                          "kind": "oracle", "sample": f"{wl.n_steps} steps x {wl.n_req} requests x {wl.n_cand} "
                                                      f"candidates, fp32 state, {n} runs"}
    return out


# ------------------------------------------------------ dispatch sweep
SWEEP_SEQS = (1, 2, 4, 8, 16, 32)
SWEEP_LENS = (16, 32, 64, 96, 128, 192, 256, 384, 512, 768, 1024, 2048, 4096, 8192)
SWEEP_MAX_TOKENS = 32768


class UniformBatch:
    """n sequences of T tokens each, cut from one draw of the long-prefill
    inputs (same shapes and value distributions); POOLS state/window copies."""

    def __init__(self, g, torch, base, n, T):
        self.g, self.torch = g, torch
        d, x, a, b, S0, W0 = base
        self.dims = d
        N = n * T
        cu = torch.arange(0, N + 1, T, dtype=torch.int32, device="cuda")
        self.batch = g.Batch(cu, torch.arange(n, dtype=torch.int32, device="cuda"), None, T, N)
        self.x, self.a, self.b = x[:N], a[:N], b[:N]
        reps = (n + S0.shape[0] - 1) // S0.shape[0]
        s0 = S0.repeat(reps, 1, 1, 1)[:n]
        w0 = W0.repeat(reps, 1, 1)[:n]
        self.sets = []
        for _ in range(POOLS):
            conv = g.ConvPool.alloc(d, n, 3, "cuda")
            conv.buf.copy_(w0)
            self.sets.append((conv, g.StatePool(s0.clone()),
                              torch.empty((N, d.h_v, d.d_v), device="cuda")))
        self.i = 0
        self.chunk = 0

    def launch(self):
        conv, state, o = self.sets[self.i % POOLS]
        self.i += 1
        if self.chunk:
            self.g.gdn_chunked_prefill(self.dims, self.params, self.x, self.a, self.b, self.batch, conv, state,
                                       chunk=self.chunk, o=o)
        else:
            self.g.gdn_recurrent_seq(self.dims, self.params, self.x, self.a, self.b, self.batch, conv, state, o=o)


def sweep_dispatch(g, torch, steps):
    """Kernel time of the token-by-token and chunked paths over uniform
    batches (n sequences x T tokens, n T <= SWEEP_MAX_TOKENS): one JSON line
    per point, then the shortest length at which the chunked path wins for
    each n."""
    wl = wk.LONG_PREFILL
    inp = wk.make_sequence_inputs(wl)
    d = g.Dims(wl.h_k, wl.h_v, wl.d_k, wl.d_v, wl.conv_w, 0, wl.act_dtype, wl.state_dtype, wl.scale, wl.l2_eps)
    params = g.Params(_upload(torch, inp["conv_w"], d.act_torch), _upload(torch, inp["a_log"], torch.float32),
                      _upload(torch, inp["dt_bias"], torch.float32))
    base = (d, _upload(torch, inp["x"], d.act_torch), _upload(torch, inp["a"], d.act_torch),
            _upload(torch, inp["b"], d.act_torch), _upload(torch, inp["S0"], d.state_torch),
            _upload(torch, inp["window0"], d.act_torch))
    cross = {}
    for n in SWEEP_SEQS:
        for T in SWEEP_LENS:
            if n * T > SWEEP_MAX_TOKENS:
                continue
            ub = UniformBatch(g, torch, base, n, T)
            ub.params = params
            # the two paths in turn, twice; the faster round of each (the first
            # path timed on fresh pools ran several percent slow)
            t = {0: [], wl.chunk: []}
            for _ in range(2):
                for ch in t:
                    ub.chunk = ch
                    t[ch].append(measure(torch, ub, steps, 3)[0])
            seq_ms, chk_ms = min(t[0]), min(t[wl.chunk])
            line = {"n_seqs": n, "seqlen": T, "tokens": n * T, "us_token_by_token": round(seq_ms * 1e3, 2),
                    "us_chunked": round(chk_ms * 1e3, 2), "faster": "chunked" if chk_ms < seq_ms else "token_by_token"}
            print(json.dumps(line), flush=True)
            if chk_ms < seq_ms and n not in cross:
                cross[n] = T
            del ub
        torch.cuda.empty_cache()
    print(json.dumps({"sweep": "dispatch", "chunk": wl.chunk,
                      "first_length_where_chunked_wins": {str(k): v for k, v in cross.items()}}), flush=True)


# ---------------------------------------------------------------- main
def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--warm-s", type=float, default=WARM_S,
                    help="least untimed launch time before each secondary workload is timed (0 for profiler runs)")
    ap.add_argument("--only", default="decode,short_prefill,long_prefill,spec_verify,mixed_step")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--sweep-dispatch", action="store_true",
                    help="time token-by-token vs chunked prefill over uniform batches instead of the benchmark")
    ap.add_argument("--copy-calib", action="store_true",
                    help="first run a plain 1 GiB device copy (the byte-counter calibration kernel)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the GDN core shards by head or request with no exchange, "
              "and the benchmark runs on a single MI355X. Use --gpus 1.", file=sys.stderr)
        sys.exit(2)
    import torch
    import linear_attention_ssm_gdn_amd as g
    g.load()
    if args.sweep_dispatch:
        sweep_dispatch(g, torch, max(args.steps // 20, 5))
        return
    only = set(args.only.split(","))
    result = {"metric": METRIC}
    if args.copy_calib:
        src = torch.ones(256 << 20, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copy calibration: 5 x {src.numel() * 4} bytes read and written")
        del src, dst
    other = {}
    log("denominators: device copy and bf16 GEMM")
    copy = measured_copy_gbs(torch)
    gemm = measured_gemm_tflops(torch)
    result["measured_peaks"] = {"copy": copy, "bf16_gemm": gemm,
                                "fp32_valu_reachable": {"value": FP32_VALU_REACHABLE_TFLOPS, "unit": "TFLOP/s",
                                                        "derivation": "256 CU x 4 SIMD x 16 lanes x 2 (FMA) x 2.4 GHz, "
                                                                      "packed fp32 off"}}
    log(f"denominators: copy {copy['value']:.0f} GB/s, bf16 GEMM {gemm['value']:.0f} TFLOP/s")

    def hbm_roofline(achieved_gbs, nbytes, traffic, kernel):
        return {"bound": "hbm", "achieved": round(achieved_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved_gbs / HBM_PEAK_GBS, 4), "traffic": traffic, "kernel": kernel,
                "algorithmic_bytes": nbytes, "frac_of_measured_copy": round(achieved_gbs / copy["value"], 4)}

    # ---- headline: decode
    wl = wk.DECODE
    log("decode: building pools")
    dec = SeqWorkload(g, torch, wl)
    k_ms, wall_ms = measure(torch, dec, args.steps, args.warmup)
    us = k_ms * 1e3
    nbytes = decode_bytes(wl)
    achieved = nbytes / (k_ms * 1e-3) / 1e9
    traffic = read_traffic("k_gdn_seq_stream", "decode")
    log(f"decode: {us:.2f} us/step kernel, {wall_ms * 1e3:.2f} us/step wall, {achieved:.0f} GB/s")
    result.update({
        "value": round(us, 3), "unit": "us/step", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(wall_ms, 5), "higher_is_better": False, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32", "data": "synthetic",
        "config": {"workload": "decode", "n_seqs": len(wl.seqlens), "tokens_per_seq": 1, "h_k": wl.h_k,
                   "h_v": wl.h_v, "d_k": wl.d_k, "d_v": wl.d_v, "conv_w": wl.conv_w, "act_dtype": wl.act_dtype,
                   "state_dtype": wl.state_dtype, "tokens_per_s_per_layer": round(len(wl.seqlens) / (k_ms * 1e-3)),
                   "rotation": dec.rotation(), "us_per_step_percentiles": dict(LAST_PERCENTILES)},
        "roofline": hbm_roofline(achieved, nbytes, traffic, "k_gdn_seq_stream"),
    })
    del dec
    torch.cuda.empty_cache()

    # ---- short ragged prefill (token by token)
    if "short_prefill" in only:
        try:
            wl = wk.SHORT_PREFILL
            log("short_prefill")
            w = SeqWorkload(g, torch, wl)
            k_ms, wall_ms = measure(torch, w, max(args.steps // 4, 10), 5, args.warm_s)
            fl = recurrence_flops(wl)
            tf = fl / (k_ms * 1e-3) / 1e12
            other["short_prefill"] = {
                "value": round(wl.n_tokens / (k_ms * 1e-3)), "unit": "tokens/s/layer", "us_per_call": round(k_ms * 1e3, 2),
                "us_per_token_critical_path": round(k_ms * 1e3 / max(wl.seqlens), 4),
                "us_per_call_percentiles": dict(LAST_PERCENTILES),
                "roofline": {"bound": "alu", "achieved": round(tf, 2), "peak": FP32_VALU_PEAK_TFLOPS, "unit": "TFLOP/s",
                             "frac": round(tf / FP32_VALU_PEAK_TFLOPS, 4),
                             "peak_reachable": FP32_VALU_REACHABLE_TFLOPS,
                             "frac_reachable": round(tf / FP32_VALU_REACHABLE_TFLOPS, 4),
                             "traffic": read_traffic("k_gdn_seq", "short_prefill"),
                             "kernel": "k_gdn_seq", "algorithmic_flops": fl},
                "config": {"seqlens": list(wl.seqlens), "rotation": w.rotation()}}
            log(f"short_prefill: {k_ms * 1e3:.1f} us, {tf:.2f} TFLOP/s")
            # the same batch through the chunked kernel, the path gdn_prefill
            # selects for it (its longest sequence is above the token-by-token limit)
            path = g.gdn_prefill_path(w.dims, w.batch)
            del w
            torch.cuda.empty_cache()
            try:
                w = SeqWorkload(g, torch, wl, chunk=64)
                c_ms, _ = measure(torch, w, max(args.steps // 4, 10), 5, args.warm_s)
                other["short_prefill"]["chunked_path"] = {
                    "value": round(wl.n_tokens / (c_ms * 1e-3)), "unit": "tokens/s/layer",
                    "us_per_call": round(c_ms * 1e3, 2), "us_per_call_percentiles": dict(LAST_PERCENTILES),
                    "kernel": "k_chunk_prep + k_chunk_state", "chunk": 64,
                    "selected_by_gdn_prefill": path == g.GDN_PATH_CHUNKED}
                log(f"short_prefill, chunked kernel: {c_ms * 1e3:.1f} us")
                del w
                torch.cuda.empty_cache()
            except g.GdnError as e:
                other["short_prefill"]["chunked_path"] = {"value": None, "note": f"not available: {e}"}
        except Exception as e:  # a failure here must not cost the headline line
            failed(other, "short_prefill", e)

    # ---- long chunked prefill
    if "long_prefill" in only:
        try:
            wl = wk.LONG_PREFILL
            try:
                g.gdn_chunked_workspace_bytes(g.Dims(wl.h_k, wl.h_v, wl.d_k, wl.d_v), len(wl.seqlens), wl.n_tokens,
                                              wl.chunk)
                log("long_prefill")
                w = SeqWorkload(g, torch, wl, chunk=wl.chunk)
                k_ms, wall_ms = measure(torch, w, max(args.steps // 20, 5), 2, args.warm_s)
                fl = chunked_flops(wl)
                tf = fl / (k_ms * 1e-3) / 1e12
                other["long_prefill"] = {
                    "value": round(wl.n_tokens / (k_ms * 1e-3)), "unit": "tokens/s/layer", "us_per_call": round(k_ms * 1e3, 1),
                    "us_per_call_percentiles": dict(LAST_PERCENTILES),
                    "roofline": {"bound": "mfma", "achieved": round(tf, 1), "peak": BF16_MFMA_PEAK_TFLOPS,
                                 "unit": "TFLOP/s", "frac": round(tf / BF16_MFMA_PEAK_TFLOPS, 4),
                                 "frac_of_measured_gemm": round(tf / gemm["value"], 4),
                                 "traffic": read_traffic("k_chunk_prep+k_chunk_state", "long_prefill"),
                                 "kernel": "k_chunk_prep + k_chunk_state",
                                 "algorithmic_flops": fl,
                                 "hbm_frac": round(chunked_bytes(wl) / (k_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)},
                    "config": {"n_seqs": len(wl.seqlens), "seqlen": wl.seqlens[0], "chunk": wl.chunk,
                               "rotation": w.rotation()}}
                log(f"long_prefill: {k_ms * 1e3:.1f} us, {tf:.1f} TFLOP/s")
                del w
                torch.cuda.empty_cache()
            except g.GdnError as e:
                other["long_prefill"] = {"value": None, "note": f"not available: {e}"}
        except Exception as e:  # a failure here must not cost the headline line
            failed(other, "long_prefill", e)

    # ---- speculative verify (one page), fp32 and bf16 state
    if "spec_verify" in only:
        try:
            wl = wk.SPEC_VERIFY
            res = {}
            for sd in (wk.F32, wk.BF16):
                log(f"spec_verify {sd}")
                w = VerifyWorkload(g, torch, wl, sd)
                k_ms, wall_ms = measure(torch, w, max(args.steps // 2, 10), 10, args.warm_s)
                nb = verify_bytes(wl, sd, w.mean_replay)
                gbs = nb / (k_ms * 1e-3) / 1e9
                res[sd] = {"value": round(k_ms * 1e3, 2), "unit": "us/step", "us_per_step_percentiles": dict(LAST_PERCENTILES),
                           "roofline": hbm_roofline(gbs, nb, read_traffic("k_gdn_verify", "spec_verify_" + sd),
                                                    "k_gdn_verify"),
                           "rotation": w.rotation()}
                log(f"spec_verify {sd}: {k_ms * 1e3:.2f} us/step, {gbs:.0f} GB/s")
                del w
                torch.cuda.empty_cache()
            lay1 = g.gdn_spec_page_layout(g.Dims(wl.h_k, wl.h_v, wl.d_k, wl.d_v, n_spec=wl.n_cand - 1), 0)["page_bytes"]
            lay8 = g.gdn_spec_page_layout(g.Dims(wl.h_k, wl.h_v, wl.d_k, wl.d_v, n_spec=wl.n_cand - 1), 1)["page_bytes"]
            other["spec_verify"] = {"state_f32": res[wk.F32], "state_bf16": res[wk.BF16],
                                    "page_bytes_onepage_f32": lay1, "page_bytes_slots_f32": lay8,
                                    "config": {"n_req": wl.n_req, "n_cand": wl.n_cand}}
        except Exception as e:  # a failure here must not cost the headline line
            failed(other, "spec_verify", e)

    # ---- mixed steps: a prefill batch + a verify batch, one launch vs two
    if "mixed_step" in only:
        try:
            res = {}
            small_seq = wk.SHORT_PREFILL.replace(name="small_prefill", seqlens=(45, 17, 9, 3))
            small_ver = wk.SPEC_VERIFY.replace(name="small_verify", n_req=8)
            dec_seq = wk.SHORT_PREFILL.replace(name="decode_rows", seqlens=(1,) * 32)
            for name, sw, vw in (("short_prefill_plus_verify", wk.SHORT_PREFILL, wk.SPEC_VERIFY),
                                 ("small_prefill_plus_verify", small_seq, small_ver),
                                 ("decode_rows_plus_verify", dec_seq, wk.SPEC_VERIFY)):
                log(f"mixed_step {name}")
                w = MixedWorkload(g, torch, sw, vw)
                n = max(args.steps // 8, 10)
                # the three forms in turn, three rounds, median of each form's
                # rounds (the first form timed on fresh pools ran 6-9% slow)
                forms = ((True, g.GDN_MIXED_AUTO), (True, g.GDN_MIXED_ONE_LAUNCH), (False, g.GDN_MIXED_AUTO))
                runs = {f: [] for f in forms}
                for _ in range(3):
                    for f in forms:
                        w.fused, w.launches = f
                        runs[f].append(measure(torch, w, n, 5, args.warm_s)[0])
                f_ms, one_ms, s_ms = (float(np.median(runs[f])) for f in forms)
                res[name] = {"value": round(f_ms * 1e3, 1), "unit": "us/step",
                             "launches": w.chosen_launches(), "us_one_launch": round(one_ms * 1e3, 1),
                             "us_separate_launches": round(s_ms * 1e3, 1),
                             "speedup_vs_separate": round(s_ms / f_ms, 3),
                             "config": {"prefill_seqlens": list(sw.seqlens), "verify_n_req": vw.n_req,
                                        "verify_n_cand": vw.n_cand, "state_dtype": "f32"}}
                log(f"mixed_step {name}: {f_ms * 1e3:.1f} us (gdn_mixed_step), {one_ms * 1e3:.1f} us one launch, "
                    f"{s_ms * 1e3:.1f} us as two separate calls")
                del w
                torch.cuda.empty_cache()
            other["mixed_step"] = res
        except Exception as e:  # a failure here must not cost the headline line
            failed(other, "mixed_step", e)

    result["other_workloads"] = other
    if not args.no_cpu:
        log("cpu baseline (oracle)")
        result["cpu_baseline"] = cpu_baseline(wk.DECODE)
        log("cpu oracle on the other workloads")
        try:
            for name, base in cpu_other_workloads().items():
                if name in other and isinstance(other[name], dict):
                    other[name]["cpu_baseline"] = base
        except Exception as e:  # the oracle legs are context; the line still comes out
            log(f"cpu oracle on the other workloads: failed: {type(e).__name__}: {e}")
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
