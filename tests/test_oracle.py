"""Pins of the fp64 oracle against closed forms, special cases, library
routines and brute-force cross-checks (CPU only).

Each test names the definition it pins (Gated DeltaNet as stated by the
method: conv (a), gating (b), delta rule and chunked form (c); one-page
verify semantics from "r9700-stack v0.2.4: one GDN state page per request",
section "What it does").
"""
import math

import numpy as np
import pytest

import gdn_workloads as wk


def rng(seed=0):
    return np.random.default_rng(seed)


# ------------------------------------------------------------- scalars (a)(b)
def test_silu_closed_forms(ora):
    assert ora.silu(0.0) == 0.0
    # sigmoid(ln 3) = 3/4 exactly, so SiLU(ln 3) = 0.75 ln 3
    assert abs(ora.silu(math.log(3.0)) - 0.75 * math.log(3.0)) < 1e-15
    # SiLU(z) - SiLU(-z) = z for every z
    for z in (-30.0, -2.5, -0.1, 0.7, 3.0, 40.0):
        assert abs(ora.silu(z) - ora.silu(-z) - z) < 1e-13 * max(1.0, abs(z))
    assert ora.silu(-800.0) == 0.0 or abs(ora.silu(-800.0)) < 1e-300


def test_softplus_sigmoid_decay_closed_forms(ora):
    assert abs(ora.softplus(0.0) - math.log(2.0)) < 1e-16
    assert abs(ora.softplus(math.log(3.0)) - math.log(4.0)) < 1e-15
    for u in (-40.0, -3.0, -0.5, 0.5, 3.0, 40.0):
        assert abs(ora.softplus(u) - ora.softplus(-u) - u) < 1e-13 * max(1.0, abs(u))
    assert abs(ora.softplus(-50.0) - math.exp(-50.0)) < 1e-30
    assert ora.softplus(800.0) == 800.0
    assert ora.sigmoid(0.0) == 0.5
    assert abs(ora.sigmoid(math.log(3.0)) - 0.75) < 1e-16
    assert ora.sigmoid(-math.inf) == 0.0
    for A in (1.0, 2.5, 16.0):
        assert abs(ora.decay(0.0, math.log(A), 0.0) + A * math.log(2.0)) < 1e-14
        # a and dt_bias enter only through their sum
        assert abs(ora.decay(0.3, math.log(A), -0.1) - ora.decay(0.1, math.log(A), 0.1)) < 1e-14
    assert ora.decay(-math.inf, 0.0, 0.0) == 0.0


def test_round_bf16_matches_library_conversion(ora):
    torch = pytest.importorskip("torch")
    r = rng(1)
    vals = np.concatenate([
        r.standard_normal(4000).astype(np.float32),
        (r.standard_normal(1000) * 1e-30).astype(np.float32),
        np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -(1.0 + 2 ** -8), 2 ** -130, 0.0],
                 dtype=np.float32),  # exact ties and a subnormal
    ])
    ref = torch.from_numpy(vals).to(torch.bfloat16).to(torch.float64).numpy()
    got = ora.round_bf16_array(vals.astype(np.float64))
    np.testing.assert_array_equal(got, ref)
    # the shared input generator's rounding agrees with the library too
    np.testing.assert_array_equal(wk.round_to(vals, wk.BF16).astype(np.float64), ref)


# ----------------------------------------------------------------- conv (a)
def test_conv_against_numpy_convolve(ora):
    r = rng(2)
    T, C, W = 23, 7, 4
    x = r.standard_normal((T, C))
    w = r.standard_normal((C, W))
    win = r.standard_normal((W - 1, C))
    y, wo = ora.conv_seq(x, w, win, act=False)
    full = np.concatenate([win, x], axis=0)
    for c in range(C):
        # np.convolve flips its kernel: tap w[c][W-1] meets the newest row
        ref = np.convolve(full[:, c], w[c][::-1], mode="valid")
        np.testing.assert_allclose(y[:, c], ref, rtol=1e-13, atol=1e-13)
    np.testing.assert_array_equal(wo, full[-(W - 1):])


def test_conv_one_hot_tap_and_impulse(ora):
    r = rng(3)
    T, C, W = 12, 5, 4
    x = r.standard_normal((T, C))
    w = np.zeros((C, W))
    w[:, W - 1] = 1.0  # newest-row tap only
    y, _ = ora.conv_seq(x, w, None, act=True)
    np.testing.assert_allclose(y, x / (1.0 + np.exp(-x)), rtol=1e-15)
    # an impulse at t0 reproduces the taps reversed in time
    w = r.standard_normal((C, W))
    x = np.zeros((T, C))
    t0 = 5
    x[t0, :] = 1.0
    y, _ = ora.conv_seq(x, w, None, act=False)
    for lag in range(W):
        np.testing.assert_array_equal(y[t0 + lag], w[:, W - 1 - lag])
    assert np.all(y[:t0] == 0.0) and np.all(y[t0 + W:] == 0.0)


def test_conv_streaming_equals_one_call(ora):
    r = rng(4)
    C, W = 6, 4
    x = r.standard_normal((20, C))
    w = r.standard_normal((C, W))
    win = r.standard_normal((W - 1, C))
    y_all, wo_all = ora.conv_seq(x, w, win)
    for cut in (0, 1, 2, 3, 7, 20):
        y1, w1 = ora.conv_seq(x[:cut], w, win)
        y2, w2 = ora.conv_seq(x[cut:], w, w1)
        np.testing.assert_array_equal(np.concatenate([y1, y2]), y_all)
        np.testing.assert_array_equal(w2, wo_all)
    # a missing window is a zero window
    np.testing.assert_array_equal(ora.conv_seq(x, w, None)[0], ora.conv_seq(x, w, np.zeros_like(win))[0])


def test_conv_f32_model_within_rounding(ora):
    r = rng(5)
    T, C, W = 30, 64, 4
    x = r.standard_normal((T, C)).astype(np.float32)
    w = r.standard_normal((C, W)).astype(np.float32)
    win = r.standard_normal((W - 1, C)).astype(np.float32)
    y32 = ora.conv_f32_model(x, w, win)
    y64, _ = ora.conv_seq(x.astype(np.float64), w.astype(np.float64), win.astype(np.float64), act=False)
    full = np.concatenate([win, x]).astype(np.float64)
    bound = np.zeros((T, C))
    for j in range(W):
        bound += np.abs(w[:, j][None, :] * full[j:j + T])
    assert np.all(np.abs(y32 - y64) <= W * 2.0 ** -24 * bound + 1e-45)
    assert y32.dtype == np.float32


def _round_f32_exact(v):
    """Round an exact rational to the nearest binary32 value, ties to even
    (normal and subnormal range; the inputs here never overflow)."""
    from fractions import Fraction
    if v == 0:
        return 0.0
    sign = -1.0 if v < 0 else 1.0
    a = abs(v)
    e = a.numerator.bit_length() - a.denominator.bit_length()   # 2^e <= a < 2^(e+1), within one
    if Fraction(2) ** e > a:
        e -= 1
    elif Fraction(2) ** (e + 1) <= a:
        e += 1
    quantum = Fraction(2) ** (max(e, -126) - 23)
    m = a / quantum
    n = m.numerator // m.denominator
    rem = m - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    r = n * quantum
    assert r < Fraction(2) ** 128
    return sign * float(r)   # exact: r is a binary32 value


def _conv_chain_exact(x, w, win, order, fused=True):
    """The conv without activation evaluated in exact rationals, rounded to
    binary32 after every operation of a chain acc = 0, acc = fma(w_j, x_j, acc)
    over the taps in `order` (fused: one rounding per tap; unfused: the
    product rounded, then the sum)."""
    from fractions import Fraction
    T, C = x.shape
    Wd = w.shape[1]
    full = np.concatenate([win, x]).astype(np.float32)
    y = np.zeros((T, C), np.float32)
    for t in range(T):
        for c in range(C):
            acc = Fraction(0)
            for j in order:
                prod = Fraction(float(w[c, j])) * Fraction(float(full[t + j, c]))
                if not fused:
                    prod = Fraction(_round_f32_exact(prod))
                acc = Fraction(_round_f32_exact(prod + acc))
            y[t, c] = float(acc)
    return y


def test_round_f32_exact_helper():
    """The exact-rounding helper of the next test against numpy's binary64 ->
    binary32 conversion (exact for these values: they are binary64 numbers
    whose rounding to binary32 is not a double rounding)."""
    from fractions import Fraction
    r = rng(50)
    vals = np.concatenate([r.standard_normal(2000), r.standard_normal(200) * 1e-40,
                           [1.0 + 2.0 ** -24, 1.0 + 3 * 2.0 ** -24, -(1.0 + 2.0 ** -24), 2.0 ** -150,
                            3 * 2.0 ** -150, 2.0 ** -149]])
    for v in vals:
        assert _round_f32_exact(Fraction(float(v))) == float(np.float32(v)), v


@pytest.mark.parametrize("dtype_in", ["f32", "bf16"])
def test_conv_f32_model_equals_exact_fma_chain(ora, dtype_in):
    """ora_conv_f32_model fixes the bits the single-precision conv must
    produce: acc = 0, one fused multiply-add per tap, oldest tap first.  It is
    checked here bit for bit against that chain evaluated in exact rationals
    with one rounding per tap (inputs drawn in fp32 and in bf16, the two
    activation dtypes).  The same inputs separate the chain from its
    plausible variants (newest tap first; with fp32 inputs also product and
    sum rounded separately), so the pin decides the order, not only the
    rounding bound."""
    r = rng(51)
    T, C, Wd = 9, 12, 4
    x = r.standard_normal((T, C)).astype(np.float32)
    w = (0.25 * r.standard_normal((C, Wd))).astype(np.float32)
    win = r.standard_normal((Wd - 1, C)).astype(np.float32)
    if dtype_in == "bf16":
        x, w, win = (wk.round_to(a, wk.BF16) for a in (x, w, win))
    got = ora.conv_f32_model(x, w, win)
    oldest_first = _conv_chain_exact(x, w, win, range(Wd))
    np.testing.assert_array_equal(got, oldest_first)
    newest_first = _conv_chain_exact(x, w, win, range(Wd - 1, -1, -1))
    unfused = _conv_chain_exact(x, w, win, range(Wd), fused=False)
    assert np.any(newest_first != oldest_first)
    if dtype_in == "f32":
        assert np.any(unfused != oldest_first)
    else:
        # a product of two bf16 values has at most 16 significant bits, so it
        # is exact in binary32 and fusing makes no difference
        np.testing.assert_array_equal(unfused, oldest_first)


def test_conv_update_ragged_and_has_init(ora):
    r = rng(6)
    C, W = 5, 4
    lens = [0, 1, 2, 9]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    x = r.standard_normal((cu[-1], C))
    w = r.standard_normal((C, W))
    win = r.standard_normal((len(lens), W - 1, C))
    has = np.array([1, 1, 0, 1], dtype=np.uint8)
    y, wo = ora.conv_update(x, w, cu, win, has)
    for s, T in enumerate(lens):
        w0 = win[s] if has[s] else np.zeros((W - 1, C))
        ys, ws = ora.conv_seq(x[cu[s]:cu[s + 1]], w, w0)
        np.testing.assert_array_equal(y[cu[s]:cu[s + 1]], ys)
        np.testing.assert_array_equal(wo[s], ws)
    np.testing.assert_array_equal(wo[0], win[0])  # empty sequence: window unchanged


# --------------------------------------------------------------- gating (b)
def test_gate_row_norms_and_split(ora):
    r = rng(7)
    dm = ora.dims(2, 4, 8, 3, 4, 1.0, 1e-6)
    C = 2 * 2 * 8 + 4 * 3
    y = r.standard_normal(C)
    a, b = r.standard_normal(4), r.standard_normal(4)
    a_log, dt = np.log(r.uniform(1, 16, 4)), r.standard_normal(4) * 0.1
    qn, kn, v, g, beta = ora.gate_row(dm, y, a, b, a_log, dt)
    q = y[:16].reshape(2, 8)
    k = y[16:32].reshape(2, 8)
    for i in range(2):
        for src, dst in ((q[i], qn[i]), (k[i], kn[i])):
            s = float(np.sum(src * src))
            assert abs(np.sum(dst * dst) - s / (s + 1e-6)) < 1e-14
            # same direction
            assert abs(np.dot(dst, src) - math.sqrt(s) * math.sqrt(np.sum(dst * dst))) < 1e-12
    np.testing.assert_array_equal(v, y[32:].reshape(4, 3))
    for h in range(4):
        assert g[h] == ora.decay(a[h], a_log[h], dt[h])
        assert beta[h] == ora.sigmoid(b[h])
        assert g[h] < 0.0 and 0.0 < beta[h] < 1.0


# ------------------------------------------------------------ delta rule (c)
def _unit(v):
    return v / np.linalg.norm(v, axis=-1, keepdims=True)


def test_delta_identity_beta0_g0(ora):
    r = rng(8)
    T, dk, dv = 9, 6, 5
    q, k = r.standard_normal((T, dk)), r.standard_normal((T, dk))
    v = r.standard_normal((T, dv))
    S0 = r.standard_normal((dk, dv))  # not symmetric: catches a transposed operand
    o, S = ora.delta_rule(q, k, v, np.zeros(T), np.zeros(T), S0, scale=0.7)
    np.testing.assert_array_equal(S, S0)
    np.testing.assert_allclose(o, 0.7 * q @ S0, rtol=1e-13, atol=1e-13)


def test_delta_reset(ora):
    r = rng(9)
    T, dk, dv = 6, 5, 4
    q, k = _unit(r.standard_normal((T, dk))), _unit(r.standard_normal((T, dk)))
    v = r.standard_normal((T, dv))
    beta = r.uniform(0.1, 0.9, T)
    S0 = r.standard_normal((dk, dv)) * 10
    o, S = ora.delta_rule(q, k, v, np.full(T, -1e4), beta, S0, scale=1.3)
    np.testing.assert_allclose(S, beta[-1] * np.outer(k[-1], v[-1]), rtol=1e-14, atol=1e-15)
    for t in range(T):
        np.testing.assert_allclose(o[t], 1.3 * beta[t] * np.dot(k[t], q[t]) * v[t], rtol=1e-13, atol=1e-15)


def test_delta_retrieval(ora):
    r = rng(10)
    T, dk, dv = 7, 8, 5
    q, k = r.standard_normal((T, dk)), _unit(r.standard_normal((T, dk)))
    v = r.standard_normal((T, dv))
    g = -r.uniform(0, 2, T)
    S = r.standard_normal((dk, dv))
    for t in range(T):
        _, S = ora.delta_rule(q[t:t + 1], k[t:t + 1], v[t:t + 1], g[t:t + 1], np.ones(1), S)
        np.testing.assert_allclose(S.T @ k[t], v[t], rtol=1e-12, atol=1e-12)


def test_delta_gla_closed_form_orthonormal_keys(ora):
    r = rng(11)
    dk, dv, T = 8, 4, 8
    Qm, _ = np.linalg.qr(r.standard_normal((dk, dk)))
    k = Qm.T[:T]  # orthonormal rows
    q = r.standard_normal((T, dk))
    v = r.standard_normal((T, dv))
    g = -r.uniform(0.0, 1.5, T)
    beta = r.uniform(0.05, 0.95, T)
    o, _ = ora.delta_rule(q, k, v, g, beta, np.zeros((dk, dv)), scale=0.5)
    G = np.cumsum(g)
    for t in range(T):
        ref = sum(math.exp(G[t] - G[j]) * beta[j] * np.dot(q[t], k[j]) * v[j] for j in range(t + 1))
        np.testing.assert_allclose(o[t], 0.5 * ref, rtol=1e-12, atol=1e-14)


def test_delta_single_step_closed_form(ora):
    r = rng(12)
    dk, dv = 6, 7
    q, k = r.standard_normal(dk), _unit(r.standard_normal(dk))
    v = r.standard_normal(dv)
    S0 = r.standard_normal((dk, dv))
    g, beta, s = -0.37, 0.61, 1.7
    o, S1 = ora.delta_rule(q[None], k[None], v[None], np.array([g]), np.array([beta]), S0, scale=s)
    eg, kq = math.exp(g), float(np.dot(k, q))
    ref = s * (eg * (S0.T @ q - beta * kq * (S0.T @ k)) + beta * kq * v)
    np.testing.assert_allclose(o[0], ref, rtol=1e-13, atol=1e-14)
    # decay applies to the state before the delta update
    ref_S = eg * (S0 - beta * np.outer(k, k @ S0)) + beta * np.outer(k, v)
    np.testing.assert_allclose(S1, ref_S, rtol=1e-13, atol=1e-14)


def test_delta_linear_in_values_and_state(ora):
    r = rng(13)
    T, dk, dv = 10, 5, 4
    q, k = r.standard_normal((T, dk)), _unit(r.standard_normal((T, dk)))
    g, beta = -r.uniform(0, 1, T), r.uniform(0, 1, T)
    V1, V2 = r.standard_normal((T, dv)), r.standard_normal((T, dv))
    S1, S2 = r.standard_normal((dk, dv)), r.standard_normal((dk, dv))
    al = -1.7
    o1, _ = ora.delta_rule(q, k, V1, g, beta, S1)
    o2, _ = ora.delta_rule(q, k, V2, g, beta, S2)
    o12, _ = ora.delta_rule(q, k, al * V1 + V2, g, beta, al * S1 + S2)
    np.testing.assert_allclose(o12, al * o1 + o2, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("C", [1, 2, 3, 8, 16, 64])
@pytest.mark.parametrize("decay", ["config", "mild", "none"])
def test_chunked_equals_sequential(ora, C, decay):
    r = rng(100 + C)
    T, dk, dv = 131, 16, 12  # ragged last chunk for every C > 1 here
    q = _unit(r.standard_normal((T, dk)))
    k = _unit(r.standard_normal((T, dk)))
    v = r.standard_normal((T, dv))
    if decay == "config":
        g = np.array([ora.decay(a, math.log(A), d) for a, A, d in
                      zip(r.standard_normal(T), r.uniform(1, 16, T), r.standard_normal(T) * 0.1)])
    elif decay == "mild":
        g = -r.uniform(0.0, 0.2, T)
    else:
        g = np.zeros(T)
    beta = 1.0 / (1.0 + np.exp(-r.standard_normal(T)))
    S0 = r.standard_normal((dk, dv))
    o_s, S_s = ora.delta_rule(q, k, v, g, beta, S0, scale=0.9)
    o_c, S_c = ora.delta_rule(q, k, v, g, beta, S0, scale=0.9, chunk=C)
    assert ora.max_rel(o_c, o_s) < 1e-12
    assert ora.max_rel(S_c, S_s) < 1e-12


# ---------------------------------------------------------------- the layer
def _small_wl(**kw):
    base = dict(name="t", h_k=2, h_v=4, d_k=8, d_v=6, conv_w=4, act_dtype=wk.F32,
                state_dtype=wk.F32, seqlens=(5, 0, 11, 1), seed=21)
    base.update(kw)
    return wk.Workload(**base)


def test_layer_single_token_end_to_end(ora):
    """T = 1 end to end with independently computed conv (np.convolve),
    gating (numpy) and the single-step closed form."""
    wl = _small_wl(seqlens=(1,))
    inp = wk.make_sequence_inputs(wl)
    dm = ora.dims_of(wl)
    o, win, S = ora.layer(dm, inp["conv_w"], inp["a_log"], inp["dt_bias"], inp["x"], inp["a"],
                          inp["b"], inp["cu_seqlens"], inp["window0"], inp["S0"])
    x = inp["x"].astype(np.float64)
    full = np.concatenate([inp["window0"][0], x]).astype(np.float64)
    z = np.array([np.convolve(full[:, c], inp["conv_w"][c][::-1].astype(np.float64), "valid")[0]
                  for c in range(wl.c_conv)])
    y = z / (1 + np.exp(-z))
    qk = wl.h_k * wl.d_k
    q = y[:qk].reshape(wl.h_k, wl.d_k)
    k = y[qk:2 * qk].reshape(wl.h_k, wl.d_k)
    v = y[2 * qk:].reshape(wl.h_v, wl.d_v)
    q = q / np.sqrt(np.sum(q * q, -1, keepdims=True) + 1e-6)
    k = k / np.sqrt(np.sum(k * k, -1, keepdims=True) + 1e-6)
    u = inp["a"][0].astype(np.float64) + inp["dt_bias"]
    g = -np.exp(inp["a_log"].astype(np.float64)) * np.log1p(np.exp(u))
    beta = 1 / (1 + np.exp(-inp["b"][0].astype(np.float64)))
    r = wl.h_v // wl.h_k
    for h in range(wl.h_v):
        i = h // r
        S0 = inp["S0"][0, h].astype(np.float64)
        kq = float(np.dot(k[i], q[i]))
        eg = math.exp(g[h])
        ref = eg * (S0.T @ q[i] - beta[h] * kq * (S0.T @ k[i])) + beta[h] * kq * v[h]
        np.testing.assert_allclose(o[0, h], ref, rtol=1e-12, atol=1e-13)
    np.testing.assert_array_equal(win[0], full[-3:])


def test_layer_gqa_mapping(ora):
    """v-head h reads key head h // (H_v/H_k): perturbing key head 1's q/k
    channels changes only v-heads 2 and 3."""
    wl = _small_wl(seqlens=(7,))
    inp = wk.make_sequence_inputs(wl)
    dm = ora.dims_of(wl)
    args = (inp["conv_w"], inp["a_log"], inp["dt_bias"])
    o1, _, _ = ora.layer(dm, *args, inp["x"], inp["a"], inp["b"], inp["cu_seqlens"], inp["window0"], inp["S0"])
    x2 = inp["x"].copy()
    x2[:, wl.d_k:2 * wl.d_k] += 0.5                      # q of key head 1
    x2[:, wl.h_k * wl.d_k + wl.d_k:2 * wl.h_k * wl.d_k] -= 0.5  # k of key head 1
    o2, _, _ = ora.layer(dm, *args, x2, inp["a"], inp["b"], inp["cu_seqlens"], inp["window0"], inp["S0"])
    np.testing.assert_array_equal(o1[:, :2], o2[:, :2])
    assert np.all(np.abs(o1[:, 2:] - o2[:, 2:]).max(axis=(0, 2)) > 1e-6)


def test_layer_streaming_and_has_init(ora):
    wl = _small_wl(seqlens=(19,))
    inp = wk.make_sequence_inputs(wl)
    dm = ora.dims_of(wl)
    P = (inp["conv_w"], inp["a_log"], inp["dt_bias"])
    x, a, b = inp["x"], inp["a"], inp["b"]
    o, win, S = ora.layer(dm, *P, x, a, b, inp["cu_seqlens"], inp["window0"], inp["S0"])
    for cut in (1, 2, 3, 10):
        o1, w1, S1 = ora.layer(dm, *P, x[:cut], a[:cut], b[:cut], [0, cut], inp["window0"], inp["S0"])
        o2, w2, S2 = ora.layer(dm, *P, x[cut:], a[cut:], b[cut:], [0, 19 - cut], w1, S1)
        assert ora.max_rel(np.concatenate([o1, o2]), o) < 1e-13
        assert ora.max_rel(S2, S) < 1e-13
        np.testing.assert_array_equal(w2, win)
    # has_init = 0 equals a zero window and a zero state
    oz, _, Sz = ora.layer(dm, *P, x, a, b, inp["cu_seqlens"], np.zeros_like(inp["window0"]),
                          np.zeros_like(inp["S0"]))
    on, _, Sn = ora.layer(dm, *P, x, a, b, inp["cu_seqlens"], inp["window0"], inp["S0"],
                          has_init=np.array([0], np.uint8))
    np.testing.assert_array_equal(on, oz)
    np.testing.assert_array_equal(Sn, Sz)


def test_layer_chunked_matches_token_by_token(ora):
    wl = _small_wl()
    inp = wk.make_sequence_inputs(wl)
    dm = ora.dims_of(wl)
    P = (inp["conv_w"], inp["a_log"], inp["dt_bias"], inp["x"], inp["a"], inp["b"], inp["cu_seqlens"],
         inp["window0"], inp["S0"])
    o, win, S = ora.layer(dm, *P)
    for C in (1, 4, 64):
        oc, wc, Sc = ora.layer(dm, *P, chunk=C)
        assert ora.max_rel(oc, o) < 1e-12 and ora.max_rel(Sc, S) < 1e-12
        np.testing.assert_array_equal(wc, win)


def test_layer_head_selection_skips(ora):
    wl = _small_wl(seqlens=(4, 3))
    inp = wk.make_sequence_inputs(wl)
    dm = ora.dims_of(wl)
    P = (inp["conv_w"], inp["a_log"], inp["dt_bias"], inp["x"], inp["a"], inp["b"], inp["cu_seqlens"],
         inp["window0"], inp["S0"])
    o, _, S = ora.layer(dm, *P)
    sel = np.zeros((2, wl.h_v), np.uint8)
    sel[1, 2] = 1
    o2, _, S2 = ora.layer(dm, *P, head_sel=sel)
    np.testing.assert_array_equal(o2[4:, 2], o[4:, 2])
    np.testing.assert_array_equal(S2[1, 2], S[1, 2])
    assert np.all(o2[:4] == 0) and np.all(S2[0] == inp["S0"][0])


# ------------------------------------------------------------------ verify
def _committed_stream_check(ora, wl, inp, o, state_bf16):
    """o^{(s)}_i must equal the layer output at c_i on the committed stream
    ++ c_0..c_i, where the committed stream holds 1 + accepted rows of every
    earlier step.  Uses ora.layer on explicitly concatenated streams."""
    dm = ora.dims_of(wl)
    St, R, K = wl.n_steps, wl.n_req, wl.n_cand
    P = (inp["conv_w"], inp["a_log"], inp["dt_bias"])
    for r in range(R):
        S_com = inp["S0"][r:r + 1].astype(np.float64)
        w_com = inp["window0"][r:r + 1]
        for s in range(St):
            xs, as_, bs = inp["x"][s, r], inp["a"][s, r], inp["b"][s, r]
            for i in range(K):
                oi, _, _ = ora.layer(dm, *P, xs[:i + 1], as_[:i + 1], bs[:i + 1], [0, i + 1], w_com, S_com)
                assert ora.max_rel(o[s, r, i], oi[-1]) < 1e-13
            acc = int(inp["accepted"][s, r])
            _, w_com, S_com = ora.layer(dm, *P, xs[:acc + 1], as_[:acc + 1], bs[:acc + 1], [0, acc + 1],
                                        w_com, S_com)
            if state_bf16:
                S_com = ora.round_bf16_array(S_com)
        yield r, w_com, S_com


@pytest.mark.parametrize("state_bf16", [False, True])
def test_verify_equals_committed_stream(ora, state_bf16):
    wl = _small_wl(n_req=3, n_cand=4, n_steps=5, seqlens=(), act_dtype=wk.BF16)
    inp = wk.make_verify_inputs(wl)
    S0 = inp["S0"]
    if state_bf16:
        S0 = wk.round_to(S0, wk.BF16)
    inp["S0"] = S0
    dm = ora.dims_of(wl)
    o, win, S = ora.verify(dm, inp["conv_w"], inp["a_log"], inp["dt_bias"], inp["x"], inp["a"], inp["b"],
                           inp["accepted"], inp["window0"], S0, state_bf16=state_bf16)
    for r, w_com, S_com in _committed_stream_check(ora, wl, inp, o, state_bf16):
        np.testing.assert_array_equal(win[r], w_com[0])
        assert ora.max_rel(S[r], S_com[0]) < 1e-13


def test_verify_lockstep_copies_equal_lone_request(ora):
    wl = _small_wl(n_req=1, n_cand=4, n_steps=4, seqlens=())
    inp = wk.make_verify_inputs(wl)
    dm = ora.dims_of(wl)
    P = (inp["conv_w"], inp["a_log"], inp["dt_bias"])
    o1, w1, S1 = ora.verify(dm, *P, inp["x"], inp["a"], inp["b"], inp["accepted"], inp["window0"], inp["S0"])
    rep = lambda t: np.repeat(t, 3, axis=1)
    o3, w3, S3 = ora.verify(dm, *P, rep(inp["x"]), rep(inp["a"]), rep(inp["b"]), rep(inp["accepted"]),
                            np.repeat(inp["window0"], 3, 0), np.repeat(inp["S0"], 3, 0))
    for j in range(3):
        np.testing.assert_array_equal(o3[:, j], o1[:, 0])
        np.testing.assert_array_equal(S3[j], S1[0])
        np.testing.assert_array_equal(w3[j], w1[0])


def test_max_rel_definition(ora):
    assert ora.max_rel(np.array([1.0, 2.0]), np.array([1.0, 4.0])) == 0.5
    assert ora.max_rel(np.zeros(3), np.zeros(3)) == 0.0
