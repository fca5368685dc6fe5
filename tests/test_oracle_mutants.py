"""Mutation run of the oracle's pins (CPU only).

Each mutant below is a copy of oracle/gdn_oracle.c with one plausible
mistake planted in it -- a dropped term, a wrong sign, index or bound, a
transposed operand, a skipped step -- built into its own library.  The
oracle's pin tests (test_oracle.py, test_oracle_book.py, test_golden.py) then
run against that library in a child process, and at least one of them must
fail: a mutant they all accept would mean the pins cannot tell that mistake
from the correct oracle.  The oracle's own source is never changed.
"""
import concurrent.futures as cf
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "gdn_oracle.c")

# (name, text in gdn_oracle.c, replacement); each text occurs exactly once.
MUTANTS = [
    ("silu: sign of the exponent", "return z / (1.0 + exp(-z));", "return z / (1.0 + exp(z));"),
    ("softplus: dropped u for u > 0", "if (u > 0.0) return u + log1p(exp(-u));",
     "if (u > 0.0) return log1p(exp(-u));"),
    ("decay: sign", "return -exp(a_log) * ora_softplus(a + dt_bias);",
     "return exp(a_log) * ora_softplus(a + dt_bias);"),
    ("decay: dt_bias dropped", "return -exp(a_log) * ora_softplus(a + dt_bias);",
     "return -exp(a_log) * ora_softplus(a);"),
    ("beta: sigmoid of -b", "beta[h] = ora_sigmoid(b[h]);", "beta[h] = ora_sigmoid(-b[h]);"),
    ("conv: taps reversed", "z += w[(int64_t)c * W + j] * xr;", "z += w[(int64_t)c * W + (W - 1 - j)] * xr;"),
    ("conv: rolled window one row late", "int32_t r = T - (W - 1) + j;", "int32_t r = T - (W - 2) + j;"),
    ("fp32 conv model: newest tap first",
     "for (int32_t j = 0; j < W; ++j) {\n                int32_t r = t - (W - 1) + j;\n                float xr;",
     "for (int32_t j = W - 1; j >= 0; --j) {\n                int32_t r = t - (W - 1) + j;\n                float xr;"),
    ("gating: k not normalised", "kn[(int64_t)i * d->d_k + e] = k[e] / nk;", "kn[(int64_t)i * d->d_k + e] = k[e];"),
    ("delta rule: S transposed in k^T S", "for (int32_t i = 0; i < dk; ++i) p += kt[i] * S[(int64_t)i * dv + j];",
     "for (int32_t i = 0; i < dk; ++i) p += kt[i] * S[(int64_t)j * dk + i];"),
    ("delta rule: decay outside the correction",
     "eg * (S[(int64_t)i * dv + j] - bt * kt[i] * P[j]) + bt * kt[i] * vt[j];",
     "eg * S[(int64_t)i * dv + j] - bt * kt[i] * P[j] + bt * kt[i] * vt[j];"),
    ("delta rule: output scale dropped", "o[(int64_t)t * o_stride + j] = scale * acc;",
     "o[(int64_t)t * o_stride + j] = acc;"),
    # (A's diagonal is never read by the solve, so "i >= j" in A's mask is an
    # equivalent mutant; the masks and signs below do change the result.)
    ("chunked: A masked above the diagonal", "if (i > j) {", "if (i < j) {"),
    ("chunked: output mask drops the diagonal", "for (int32_t j = 0; j <= i; ++j) {",
     "for (int32_t j = 0; j < i; ++j) {"),
    ("chunked: solve of (I - A)", "t -= A[(int64_t)i * n + m] * Tm[(int64_t)m * n + j];",
     "t += A[(int64_t)i * n + m] * Tm[(int64_t)m * n + j];"),
    ("chunked: decay ratio inverted", "aij = bc[i] * exp(G[i] - G[j]) * kk;", "aij = bc[i] * exp(G[j] - G[i]) * kk;"),
    ("chunked: end state not decayed", "double acc = exp(G[n - 1]) * S[(int64_t)m * dv + e];",
     "double acc = S[(int64_t)m * dv + e];"),
    ("verify: commits the state one candidate late", "if (i == acc) memcpy(Sacc, Srun,",
     "if (i == (acc + 1 < n_cand ? acc + 1 : acc)) memcpy(Sacc, Srun,"),
    ("verify: window rolled by acc rows",
     "ora_conv_seq(acc + 1, (int32_t)C, d->conv_w, tmp, conv_w, wr, 0, ydummy, wnext);",
     "ora_conv_seq(acc, (int32_t)C, d->conv_w, tmp, conv_w, wr, 0, ydummy, wnext);"),
    ("verify: bf16 commit not rounded", "if (state_bf16) ora_round_bf16_array(Sacc, Sreq);", ""),
    ("bf16 rounding: ties away from zero", "return ldexp(nearbyint(ldexp(m, 8)), e - 8);",
     "return ldexp(round(ldexp(m, 8)), e - 8);"),
    ("bookkeeping: parity not stored", "hdr[0] = (uint32_t)(1 - L) | ((uint32_t)parity << 1);",
     "hdr[0] = (uint32_t)(1 - L);"),
    ("bookkeeping: window from row a+1", "memcpy(win + (int64_t)j * C, cbuf + (int64_t)(a + j) * C,",
     "memcpy(win + (int64_t)j * C, cbuf + (int64_t)(a + 1 + j) * C,"),
    ("bookkeeping: acceptance bound off by one", "if (num_accepted < 0 || num_accepted >= held ||",
     "if (num_accepted < 0 || num_accepted > held ||"),
    ("layer: key head of a value head", "const int32_t i = h / r;", "const int32_t i = h % d->h_k;"),
    ("layer: has_init ignored", "if (!init) {\n            memset(win + s * ws, 0,",
     "if (0) {\n            memset(win + s * ws, 0,"),
    ("layer: state of a fresh sequence kept", "memset(S + s * (int64_t)d->h_v * hs, 0,",
     "(void)(S + s * (int64_t)d->h_v * hs), memset(win + s * ws, 0,"),
]


def _survives(name, text, repl, src, workdir):
    """Build the mutant and run the pins against it; True if every pin passes."""
    assert text == repl or src.count(text) == 1, (name, src.count(text))
    tag = "".join(ch if ch.isalnum() else "_" for ch in name)[:60]
    c = os.path.join(workdir, tag + ".c")
    so = os.path.join(workdir, tag + ".so")
    with open(c, "w") as f:
        f.write(src.replace(text, repl))
    r = subprocess.run(["gcc", "-O1", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-o", so, c, "-lm"],
                       capture_output=True, text=True)
    assert r.returncode == 0, (name, r.stderr)
    driver = (
        "import sys; sys.path[:0] = [%r, %r]\n"
        "import oracle.oracle as O; O._LIB_PATH = %r\n"
        "import pytest\n"
        "rc = pytest.main(['-q', '-x', '-p', 'no:cacheprovider', '-m', 'not gpu', 'tests/test_oracle.py',\n"
        "                  'tests/test_oracle_book.py', 'tests/test_golden.py'])\n"
        "assert O.lib()._name == %r\n"
        "sys.exit(int(rc))\n" % (ROOT, os.path.join(ROOT, "tests"), so, so))
    env = dict(os.environ, OMP_NUM_THREADS="2")
    r = subprocess.run([sys.executable, "-c", driver], cwd=ROOT, capture_output=True, text=True, env=env,
                       timeout=600)
    return r.returncode == 0


def test_every_planted_mistake_fails_a_pin(tmp_path):
    src = open(SRC).read()
    # control: the unchanged source, built and run the same way, passes every pin,
    # so a failing mutant fails because of its mistake and not of the harness
    assert _survives("control", "", "", src, str(tmp_path)), "the unchanged oracle fails its pins"
    with cf.ThreadPoolExecutor(max_workers=4) as pool:
        futs = {pool.submit(_survives, n, t, r, src, str(tmp_path)): n for n, t, r in MUTANTS}
        survivors = sorted(futs[f] for f in cf.as_completed(futs) if f.result())
    assert not survivors, f"mutants no pin catches: {survivors}"
