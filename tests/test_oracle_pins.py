"""Pins for the CPU oracle (runs without a GPU).

The sequential fp64 recurrence (oracle.scan / oracle.decode) is checked
against things other than itself:
  * hand-derived values (tests/golden/scalar_by_hand.json, tests/golden/conv1d_by_hand.json),
  * the brute-force quadratic (duality) form, built from explicit decay
    products ("Engineering hybrid state-space models", section 2),
  * scipy.signal.lfilter in the linear time-invariant special case
    (lesty.tech Mamba explainer, section 3, convolution mode),
  * closed forms in the limits the explainer's section 4 describes
    (dt -> 0 keeps the state, large dt flushes it), A = 0 (causal linear
    attention, the blog's section 3 state S_t = S_{t-1} + k v^T), x = 0,
  * algebraic invariants: linearity, group broadcast, packed sequences ==
    separate runs, head permutation, prefill + decode == longer prefill.
The fp64 chunked regrouping (oracle.chunked) is pinned against the
sequential oracle for many chunk sizes, including ragged tails.
The conv1d oracle (oracle.conv) is pinned against numpy.convolve and
scipy.signal.lfilter per channel, its impulse response (tap order, no channel
mixing), SiLU closed forms and scipy.special.expit, and the continuation of
its state across segments of 0, 1 and more tokens.
"""
import json
import os

import numpy as np
import pytest
import scipy.signal

import oracle
from oracle.chunked import chunked_scan
from oracle.quadratic import quadratic_scan_sequence

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rand_case(seed, L=23, H=4, P=3, N=5, G=2, nseq=1, init=True, A_scale=1.0):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((nseq, L, H, P))
    dt = rng.uniform(0.01, 0.6, (nseq, L, H))
    A = -rng.uniform(0.2, 3.0, H) * A_scale
    B = rng.standard_normal((nseq, L, G, N))
    C = rng.standard_normal((nseq, L, G, N))
    D = rng.standard_normal(H)
    h0 = rng.standard_normal((nseq, H, P, N)) if init else None
    return x, dt, A, B, C, D, h0


def close(a, b, tol=1e-12):
    a = np.asarray(a)
    b = np.asarray(b)
    scale = max(1.0, float(np.max(np.abs(b))) if b.size else 1.0)
    assert a.shape == b.shape
    err = float(np.max(np.abs(a - b))) / scale if a.size else 0.0
    assert err <= tol, err


# ------------------------------------------------------------------ golden
def test_golden_hand_values():
    g = json.load(open(os.path.join(GOLDEN, "scalar_by_hand.json")))
    L = len(g["dt"])
    x = np.array(g["x"]).reshape(1, L, 1, 1)
    dt = np.array(g["dt"]).reshape(1, L, 1)
    B = np.array(g["B"]).reshape(1, L, 1, 2)
    C = np.array(g["C"]).reshape(1, L, 1, 2)
    for case in g["cases"]:
        h0 = np.array(case["h0"]).reshape(1, 1, 1, 2)
        y, fin = oracle.scan(x, dt, g["A"], B, C, g["D"], init=h0)
        close(y.reshape(-1), case["y"], 1e-15)
        close(fin.reshape(-1), case["final"], 1e-15)
        if "decode" in case:
            d = case["decode"]
            yd, st = oracle.decode(fin.reshape(1, 1, 1, 2), np.full((1, 1, 1), d["x"]),
                                   np.full((1, 1), d["dt"]), g["A"],
                                   np.array(d["B"]).reshape(1, 1, 2),
                                   np.array(d["C"]).reshape(1, 1, 2), g["D"])
            close(yd.reshape(-1), [d["y"]], 1e-15)
            close(st.reshape(-1), d["state"], 1e-15)


# ------------------------------------------------------------------ quadratic form
@pytest.mark.parametrize("seed", range(6))
@pytest.mark.parametrize("init", [False, True])
def test_matches_quadratic_form(seed, init):
    L = [1, 2, 7, 23, 37, 64][seed]
    x, dt, A, B, C, D, h0 = rand_case(seed, L=L, init=init)
    y, fin = oracle.scan(x, dt, A, B, C, D, init=h0)
    yq, fq = quadratic_scan_sequence(x[0], dt[0], A, B[0], C[0], D,
                                     None if h0 is None else h0[0])
    close(y[0], yq, 1e-12)
    close(fin[0], fq, 1e-12)


# ------------------------------------------------------------------ LTI == lfilter
def test_lti_is_first_order_iir():
    """Constant dt, B, C and zero h0: every (h, p) channel is the IIR filter
    y = (B.C) * lfilter([dt], [1, -exp(dt*A)], x) + D x."""
    rng = np.random.default_rng(7)
    L, H, P, N = 50, 3, 4, 6
    x = rng.standard_normal((1, L, H, P))
    dtv = rng.uniform(0.05, 0.5, H)
    dt = np.broadcast_to(dtv, (1, L, H)).copy()
    A = -rng.uniform(0.1, 2.0, H)
    b = rng.standard_normal(N)
    c = rng.standard_normal(N)
    B = np.broadcast_to(b, (1, L, 1, N)).copy()
    C = np.broadcast_to(c, (1, L, 1, N)).copy()
    D = rng.standard_normal(H)
    y, _ = oracle.scan(x, dt, A, B, C, D)
    for h in range(H):
        filt = scipy.signal.lfilter([dtv[h]], [1.0, -np.exp(dtv[h] * A[h])], x[0, :, h, :], axis=0)
        close(y[0, :, h, :], float(b @ c) * filt + D[h] * x[0, :, h, :], 1e-12)


# ------------------------------------------------------------------ limits / closed forms
def test_A_zero_is_causal_linear_attention():
    x, dt, A, B, C, D, h0 = rand_case(3, L=30)
    A = np.zeros_like(A)
    y, fin = oracle.scan(x, dt, A, B, C, D, init=h0)
    H = x.shape[2]
    G = B.shape[2]
    for h in range(H):
        g = h // (H // G)
        kv = (dt[0, :, h, None] * x[0, :, h, :])[:, :, None] * B[0, :, g, None, :]
        S = h0[0, h][None] + np.cumsum(kv, axis=0)            # S_t = S_{t-1} + k v^T
        yy = np.einsum("tpn,tn->tp", S, C[0, :, g, :]) + D[h] * x[0, :, h, :]
        close(y[0, :, h, :], yy, 1e-12)
        close(fin[0, h], S[-1], 1e-12)


def test_memoryless_limit():
    """exp(dt*A) underflows to exactly 0: only the current token remains."""
    x, dt, A, B, C, D, h0 = rand_case(4, L=12)
    A = np.full_like(A, -1e6)
    y, fin = oracle.scan(x, dt, A, B, C, D, init=h0)
    H = x.shape[2]
    G = B.shape[2]
    for h in range(H):
        g = h // (H // G)
        cb = np.sum(C[0, :, g, :] * B[0, :, g, :], axis=1)
        close(y[0, :, h, :], (dt[0, :, h] * cb)[:, None] * x[0, :, h, :] + D[h] * x[0, :, h, :])
        close(fin[0, h], dt[0, -1, h] * np.outer(x[0, -1, h], B[0, -1, g]))


def test_dt_to_zero_keeps_state():
    x, dt, A, B, C, D, h0 = rand_case(5, L=9)
    dt = np.full_like(dt, 1e-30)
    y, fin = oracle.scan(x, dt, A, B, C, D, init=h0)
    H = x.shape[2]
    G = B.shape[2]
    for h in range(H):
        g = h // (H // G)
        close(y[0, :, h, :], C[0, :, g, :] @ h0[0, h].T + D[h] * x[0, :, h, :])
    close(fin, h0)


def test_zero_input_decays_initial_state():
    x, dt, A, B, C, D, h0 = rand_case(6, L=15)
    x = np.zeros_like(x)
    y, fin = oracle.scan(x, dt, A, B, C, D, init=h0)
    H = x.shape[2]
    G = B.shape[2]
    for h in range(H):
        g = h // (H // G)
        decay = np.exp(A[h] * np.cumsum(dt[0, :, h]))
        close(y[0, :, h, :], decay[:, None] * (C[0, :, g, :] @ h0[0, h].T))
        close(fin[0, h], decay[-1] * h0[0, h])


# ------------------------------------------------------------------ invariants
def test_linearity_in_x_and_h0():
    x1, dt, A, B, C, D, h1 = rand_case(8)
    x2, _, _, _, _, _, h2 = rand_case(9)
    a, b = 0.7, -1.3
    y, f = oracle.scan(a * x1 + b * x2, dt, A, B, C, D, init=a * h1 + b * h2)
    y1, f1 = oracle.scan(x1, dt, A, B, C, D, init=h1)
    y2, f2 = oracle.scan(x2, dt, A, B, C, D, init=h2)
    close(y, a * y1 + b * y2)
    close(f, a * f1 + b * f2)


def test_group_broadcast_equals_expanded_heads():
    x, dt, A, B, C, D, h0 = rand_case(10, H=6, G=3)
    y, f = oracle.scan(x, dt, A, B, C, D, init=h0)
    rep = 6 // 3
    Be = np.repeat(B, rep, axis=2)
    Ce = np.repeat(C, rep, axis=2)
    ye, fe = oracle.scan(x, dt, A, Be, Ce, D, init=h0)
    close(y, ye, 1e-14)
    close(f, fe, 1e-14)


def test_head_permutation_equivariance():
    x, dt, A, B, C, D, h0 = rand_case(11, H=5, G=1)
    perm = np.array([3, 0, 4, 1, 2])
    y, f = oracle.scan(x, dt, A, B, C, D, init=h0)
    yp, fp = oracle.scan(x[:, :, perm], dt[:, :, perm], A[perm], B, C, D[perm], init=h0[:, perm])
    close(yp, y[:, :, perm], 0)
    close(fp, f[:, perm], 0)


def test_packed_sequences_equal_separate_runs():
    rng = np.random.default_rng(12)
    lens = [5, 0, 17, 1, 9]
    H, P, N, G = 4, 3, 5, 2
    T = sum(lens)
    x = rng.standard_normal((T, H, P))
    dt = rng.uniform(0.01, 0.5, (T, H))
    A = -rng.uniform(0.2, 2, H)
    B = rng.standard_normal((T, G, N))
    C = rng.standard_normal((T, G, N))
    D = rng.standard_normal(H)
    h0 = rng.standard_normal((len(lens), H, P, N))
    cu = np.concatenate([[0], np.cumsum(lens)])
    y, f = oracle.scan(x, dt, A, B, C, D, init=h0, cu_seqlens=cu)
    for s, l in enumerate(lens):
        a, b = cu[s], cu[s + 1]
        ys, fs = oracle.scan(x[None, a:b], dt[None, a:b], A, B[None, a:b], C[None, a:b], D,
                             init=h0[s:s + 1])
        close(y[a:b], ys[0], 0)
        close(f[s], fs[0], 0)
    close(f[1], h0[1], 0)  # empty sequence: the state passes through


def test_prefill_then_decode_equals_longer_prefill():
    x, dt, A, B, C, D, h0 = rand_case(13, L=21)
    y, f = oracle.scan(x, dt, A, B, C, D, init=h0)
    L = x.shape[1]
    k = 4
    _, f_short = oracle.scan(x[:, :L - k], dt[:, :L - k], A, B[:, :L - k], C[:, :L - k], D,
                             init=h0)
    st = f_short
    for t in range(L - k, L):
        yd, st = oracle.decode(st, x[:, t], dt[:, t], A, B[:, t], C[:, t], D)
        close(yd, y[:, t], 1e-13)
    close(st, f, 1e-13)
    # a one-token prefill is a decode step from the initial state
    y1, f1 = oracle.scan(x[:, :1], dt[:, :1], A, B[:, :1], C[:, :1], D, init=h0)
    yd, sd = oracle.decode(h0, x[:, 0], dt[:, 0], A, B[:, 0], C[:, 0], D)
    close(y1[:, 0], yd, 0)
    close(f1, sd, 0)


def test_thread_count_does_not_change_result():
    x, dt, A, B, C, D, h0 = rand_case(14, L=40, nseq=3)
    y1, f1 = oracle.scan(x, dt, A, B, C, D, init=h0, nthreads=1)
    y4, f4 = oracle.scan(x, dt, A, B, C, D, init=h0, nthreads=4)
    assert np.array_equal(y1, y4) and np.array_equal(f1, f4)


# ------------------------------------------------------------------ chunked regrouping
@pytest.mark.parametrize("Q", [1, 2, 3, 4, 8, 16, 37, 50])
def test_chunked_equals_sequential(Q):
    x, dt, A, B, C, D, h0 = rand_case(15, L=37, nseq=2)
    y, f = oracle.scan(x, dt, A, B, C, D, init=h0)
    yc, fc = chunked_scan(x, dt, A, B, C, D, Q, init=h0)
    close(yc, y, 1e-12)
    close(fc, f, 1e-12)


def test_chunked_packed_restart_at_sequence_start():
    rng = np.random.default_rng(16)
    lens = [7, 12, 0, 3]
    H, P, N, G = 4, 2, 3, 2
    T = sum(lens)
    x = rng.standard_normal((T, H, P))
    dt = rng.uniform(0.01, 0.5, (T, H))
    A = -rng.uniform(0.2, 2, H)
    B = rng.standard_normal((T, G, N))
    C = rng.standard_normal((T, G, N))
    D = rng.standard_normal(H)
    h0 = rng.standard_normal((len(lens), H, P, N))
    cu = np.concatenate([[0], np.cumsum(lens)])
    y, f = oracle.scan(x, dt, A, B, C, D, init=h0, cu_seqlens=cu)
    yc, fc, inter = chunked_scan(x, dt, A, B, C, D, 4, init=h0, cu_seqlens=cu,
                                 return_intermediates=True)
    close(yc, y, 1e-12)
    close(fc, f, 1e-12)
    # chunks never straddle a sequence boundary
    for c in inter:
        assert cu[c["seq"]] <= c["start"] and c["start"] + c["len"] <= cu[c["seq"] + 1]


# ------------------------------------------------------------------ dt activation
def test_dt_activation_closed_forms():
    """softplus(0) = ln 2; softplus(v) - softplus(-v) = v; softplus(v) ~ exp(v)
    far below 0 and ~ v far above; positive and increasing everywhere."""
    assert oracle.dt_activation(np.array([0.0]))[0] == pytest.approx(np.log(2.0), rel=1e-15)
    v = np.linspace(-30.0, 30.0, 601)
    sp = oracle.dt_activation(v)
    sm = oracle.dt_activation(-v)
    np.testing.assert_allclose(sp - sm, v, rtol=0, atol=1e-12)
    assert np.all(sp > 0) and np.all(np.diff(sp) > 0)
    far = np.array([-40.0, -60.0, -700.0])
    np.testing.assert_allclose(oracle.dt_activation(far), np.exp(far), rtol=1e-15)
    big = np.array([40.0, 300.0, 1e6])
    np.testing.assert_allclose(oracle.dt_activation(big), big, rtol=1e-15)


def test_dt_activation_bias_per_head_and_clamp():
    rng = np.random.default_rng(3)
    raw = rng.normal(-4.0, 1.0, size=(5, 7, 3))
    bias = np.array([0.0, 2.0, -1.5])
    out = oracle.dt_activation(raw, bias)
    for h in range(3):
        np.testing.assert_array_equal(out[..., h], oracle.dt_activation(raw[..., h] + bias[h]))
    lo, hi = 0.01, 0.05
    cl = oracle.dt_activation(raw, bias, (lo, hi))
    free = oracle.dt_activation(raw, bias)
    assert cl.min() >= lo and cl.max() <= hi
    inside = (free >= lo) & (free <= hi)
    np.testing.assert_array_equal(cl[inside], free[inside])
    assert np.all(cl[free < lo] == lo) and np.all(cl[free > hi] == hi)


# ------------------------------------------------------------------ windowed decode
@pytest.mark.parametrize("W,G", [(1, 1), (5, 2), (16, 3)])
def test_decode_window_equals_sequential_steps(W, G):
    """The windowed form of every window position equals that many sequential
    decode steps of the C oracle from the window-start state."""
    rng = np.random.default_rng(40 + W)
    b, H, P, N = 2, 6, 5, 7
    S0 = rng.normal(size=(b, H, P, N))
    xw = rng.normal(size=(b, W, H, P))
    dtw = rng.uniform(0.001, 0.3, size=(b, W, H))
    A = -rng.uniform(0.1, 3.0, size=H)
    Bw = rng.normal(size=(b, W, G, N))
    Cw = rng.normal(size=(b, W, G, N))
    D = rng.normal(size=H)
    st = S0.copy()
    for t in range(W):
        y_seq, st = oracle.decode(st, xw[:, t], dtw[:, t], A, Bw[:, t], Cw[:, t], D)
        y_win, s_win = oracle.decode_window(S0, xw, dtw, A, Bw, Cw, D, t)
        np.testing.assert_allclose(y_win, y_seq, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(s_win, st, rtol=1e-12, atol=1e-12)


# ------------------------------------------------------------------ conv1d (row f-4)
from oracle import conv as oconv  # noqa: E402
import scipy.special  # noqa: E402


def test_silu_closed_forms_and_library_sigmoid():
    v = np.array([-800.0, -30.0, -2.5, -1e-9, 0.0, 1e-9, 0.7, 3.0, 40.0, 800.0])
    s = oconv.silu(v)
    assert s[4] == 0.0
    # silu(v) - silu(-v) = v (odd part of v * sigmoid(v))
    assert np.allclose(oconv.silu(v) - oconv.silu(-v), v, rtol=1e-15, atol=1e-300)
    # against the library logistic function
    assert np.allclose(s, v * scipy.special.expit(v), rtol=1e-14, atol=0)
    # tails: silu(v) -> v above, -> 0 below; derivative 1/2 at 0
    assert s[-1] == 800.0 and abs(s[0]) < 1e-300
    assert abs(oconv.silu(1e-9) / 1e-9 - 0.5) < 1e-9
    # silu(ln 2-ish) exact: silu(log(3)) = log(3) * 3/4
    assert abs(oconv.silu(np.log(3.0)) - np.log(3.0) * 0.75) < 1e-15


@pytest.mark.parametrize("K", [2, 3, 4])
def test_conv1d_equals_library_convolution_per_channel(K):
    rng = np.random.default_rng(100 + K)
    L, C = 37, 24
    x = rng.normal(size=(L, C))
    w = rng.uniform(-1, 1, size=(C, K))
    bias = rng.normal(size=C)
    st = rng.normal(size=(K - 1, C))
    y, fin = oconv.causal_conv1d(x, w, bias, st, activation=False)
    xp = np.concatenate([st, x])
    for c in range(C):
        # numpy's convolution flips the kernel; the reversed taps give the
        # correlation with tap K-1 on the newest sample
        ref = np.convolve(xp[:, c], w[c, ::-1], mode="valid") + bias[c]
        assert np.allclose(y[:, c], ref, rtol=1e-13, atol=1e-13)
        # the same FIR filter through scipy, zero state: first K-1 outputs see zeros
        ref0 = scipy.signal.lfilter(w[c, ::-1], [1.0], x[:, c]) + bias[c]
        y0, _ = oconv.causal_conv1d(x[:, c:c + 1], w[c:c + 1], bias[c:c + 1], None, activation=False)
        assert np.allclose(y0[:, 0], ref0, rtol=1e-13, atol=1e-13)
    ya, _ = oconv.causal_conv1d(x, w, bias, st, activation=True)
    assert np.allclose(ya, y * scipy.special.expit(y), rtol=1e-13, atol=1e-15)


def test_conv1d_impulse_response_orients_the_taps():
    K, C, L, t0 = 4, 3, 10, 2
    w = np.arange(1.0, 1.0 + C * K).reshape(C, K)
    x = np.zeros((L, C))
    x[t0, 1] = 1.0
    y, _ = oconv.causal_conv1d(x, w, None, None, activation=False)
    # the impulse reaches outputs t0 .. t0+K-1 with the taps newest first
    assert np.array_equal(y[t0:t0 + K, 1], w[1, ::-1])
    assert not y[:t0].any() and not y[t0 + K:].any()
    assert not y[:, 0].any() and not y[:, 2].any()  # depthwise: no channel mixing


def test_conv1d_state_continuation_and_short_segments():
    rng = np.random.default_rng(7)
    K, C = 4, 16
    w = rng.uniform(-1, 1, size=(C, K))
    bias = rng.normal(size=C)
    x = rng.normal(size=(12, C))
    st0 = rng.normal(size=(K - 1, C))
    y_all, fin_all = oconv.causal_conv1d(x, w, bias, st0)
    # split into segments of 1, 2, 0, 5, 4 tokens, each continuing from the last state
    st = st0
    ys = []
    for a, b in [(0, 1), (1, 3), (3, 3), (3, 8), (8, 12)]:
        yseg, st = oconv.causal_conv1d(x[a:b], w, bias, st)
        ys.append(yseg)
    assert np.allclose(np.concatenate(ys), y_all, rtol=1e-14, atol=1e-14)
    assert np.array_equal(st, fin_all)
    assert np.array_equal(fin_all, x[-(K - 1):])
    # a sequence shorter than K-1 keeps the tail of its incoming state
    _, fin1 = oconv.causal_conv1d(x[:1], w, bias, st0)
    assert np.array_equal(fin1, np.concatenate([st0[1:], x[:1]]))
    _, fin0 = oconv.causal_conv1d(x[:0], w, bias, st0)
    assert np.array_equal(fin0, st0)


def test_conv1d_steps_equal_prefill_and_packed_batch():
    rng = np.random.default_rng(8)
    K, C = 4, 8
    w = rng.uniform(-1, 1, size=(C, K))
    bias = rng.normal(size=C)
    lens = [5, 0, 1, 9]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    x = rng.normal(size=(cu[-1], C))
    st0 = rng.normal(size=(len(lens), K - 1, C))
    y, fin = oconv.causal_conv1d_batch(x, w, bias, st0, cu_seqlens=cu)
    for i, n in enumerate(lens):
        ys, fs = oconv.causal_conv1d(x[cu[i]:cu[i + 1]], w, bias, st0[i])
        assert np.array_equal(y[cu[i]:cu[i + 1]], ys) and np.array_equal(fin[i], fs)
    # token-by-token decode steps reproduce the prefill of one sequence
    xs = x[cu[3]:cu[4]]
    st = st0[3:4]
    for t in range(lens[3]):
        yt, st = oconv.conv1d_step(st, xs[t:t + 1], w, bias)
        assert np.allclose(yt[0], y[cu[3] + t], rtol=1e-14, atol=1e-14)
    assert np.array_equal(st[0], fin[3])


def test_conv1d_hand_values():
    g = json.load(open(os.path.join(GOLDEN, "conv1d_by_hand.json")))
    w, bias, st = np.array(g["weight"]), np.array(g["bias"]), np.array(g["state"])
    for case in g["cases"]:
        y, fin = oconv.causal_conv1d(np.array(case["x"]), w, bias, st, activation=False)
        assert np.array_equal(y, np.array(case["y"])), case["steps"]
        assert np.array_equal(fin, np.array(case["final"]))
        if "decode" in case:
            d = case["decode"]
            yd, sd = oconv.conv1d_step(fin[None], np.array(d["x"])[None], w, bias, activation=False)
            assert np.array_equal(yd[0], np.array(d["y"])) and np.array_equal(sd[0], np.array(d["state"]))


def test_decode_in_place_equals_copying_decode():
    """The in-place form of the decode glue updates the given fp64 state and
    returns the same values as the copying form (same C routine)."""
    rng = np.random.default_rng(3)
    b, H, P, N, G = 3, 4, 8, 16, 2
    st = rng.normal(size=(b, H, P, N))
    x, dt = rng.normal(size=(b, H, P)), rng.uniform(0.001, 0.1, size=(b, H))
    A, D = -rng.uniform(1, 16, size=H), rng.normal(size=H)
    B, C = rng.normal(size=(b, G, N)), rng.normal(size=(b, G, N))
    y1, s1 = oracle.decode(st, x, dt, A, B, C, D)
    st2 = st.copy()
    y2, s2 = oracle.decode(st2, x, dt, A, B, C, D, inplace=True)
    assert s2 is st2
    assert np.array_equal(y1, y2) and np.array_equal(s1, s2)
    assert not np.array_equal(st, st2)
