"""Pins of the Mamba-2 decode-step oracle (oracle/mamba2.py) to facts outside itself.

The step is the published Mamba-2 single-token update (the pages name Mamba-2 and the
stateful shift register / SSM recurrence kernels: DF-SSM technical summary, section 2C,
Stateful Ops).  Each test below would fail on a plausible slip in the oracle:
  * special values of softplus and silu (their textbook definitions);
  * the convolution with one-hot taps, which must return the activation of one
    window position: the newest value for the last tap, the oldest for the first
    (a reversed window or a wrong shift fails);
  * one step from a zero state in closed form, and pure decay when B = 0;
  * T steps of the recurrence against the SSM's quadratic (attention-like) form, an
    independent route: y_t = sum_{s <= t} (prod_{s < r <= t} dA_r) dt_s (C_t . B_s) x_s
    + (prod_{r <= t} dA_r) (h_0 C_t) + D x_t;
  * the gated norm: invariance under scaling y, unit mean square of out / w when
    eps = 0, and the gate applied before the norm;
  * the layout of the in_proj output (z | xBC | dt, then x | B | C inside xBC) on a
    hand-sized example computed here with plain floats.
"""
import math

import numpy as np

from oracle import mamba2 as m2


def test_softplus_silu_special_values():
    assert m2.softplus(0.0) == math.log(2.0)
    assert m2.softplus(25.0) == 25.0                       # threshold: identity above 20
    assert abs(m2.softplus(-30.0) - math.exp(-30.0)) < 1e-25
    assert m2.silu(0.0) == 0.0
    assert abs(m2.silu(1.0) - 1.0 / (1.0 + math.exp(-1.0))) < 1e-16
    assert abs(m2.silu(-40.0)) < 1e-15
    v = np.linspace(-10, 10, 41)
    assert np.allclose(m2.silu(v) - m2.silu(-v), v, atol=1e-13)     # silu(v) - silu(-v) = v


def test_conv_one_hot_taps_select_window_positions():
    rng = np.random.default_rng(0)
    S, C = 2, 5
    new = rng.standard_normal((S, C))
    state = rng.standard_normal((S, C, 4))
    for j, expect in [(3, new), (2, state[:, :, 3]), (1, state[:, :, 2]), (0, state[:, :, 1])]:
        w = np.zeros((C, 4))
        w[:, j] = 1.0
        act, window = m2.conv_step(new, state, w, np.zeros(C))
        assert np.allclose(act, expect / (1.0 + np.exp(-expect)), rtol=1e-14, atol=0)
        assert np.array_equal(window[:, :, 3], new) and np.array_equal(window[:, :, :3], state[:, :, 1:])
    # bias adds before the activation
    w = np.zeros((C, 4))
    act, _ = m2.conv_step(new, state, w, np.full(C, 0.75))
    assert np.allclose(act, 0.75 / (1.0 + math.exp(-0.75)))


def test_ssm_one_step_from_zero_state_and_pure_decay():
    rng = np.random.default_rng(1)
    S, H, P, N = 2, 3, 4, 5
    x = rng.standard_normal((S, H, P))
    B = rng.standard_normal((S, N))
    C = rng.standard_normal((S, N))
    dt_raw = rng.standard_normal((S, H))
    dt_bias, A_log, D = rng.standard_normal(H), rng.uniform(0, 2, H), rng.standard_normal(H)
    dt = np.log1p(np.exp(dt_raw + dt_bias))
    y, st = m2.ssm_step(x, B, C, dt_raw, np.zeros((S, H, P, N)), dt_bias, A_log, D)
    bc = (B * C).sum(axis=1)
    assert np.allclose(y, dt[:, :, None] * x * bc[:, None, None] + D[None, :, None] * x, rtol=1e-13, atol=1e-14)
    assert np.allclose(st, dt[:, :, None, None] * x[..., None] * B[:, None, None, :], rtol=1e-14, atol=0)
    # B = 0: the state only decays, by exp(-dt exp(A_log))
    h0 = rng.standard_normal((S, H, P, N))
    y, st = m2.ssm_step(x, np.zeros((S, N)), C, dt_raw, h0, dt_bias, A_log, D)
    decay = np.exp(-dt * np.exp(A_log)[None])
    assert np.allclose(st, h0 * decay[:, :, None, None], rtol=1e-14, atol=0)
    assert np.allclose(y, (st * C[:, None, None, :]).sum(axis=3) + D[None, :, None] * x, rtol=1e-13, atol=1e-14)


def test_recurrence_matches_quadratic_form():
    rng = np.random.default_rng(2)
    T, H, P, N = 7, 2, 3, 4
    xs = rng.standard_normal((T, H, P))
    Bs = rng.standard_normal((T, N))
    Cs = rng.standard_normal((T, N))
    dts_raw = rng.standard_normal((T, H))
    dt_bias, A_log, D = rng.standard_normal(H), rng.uniform(0, 1.5, H), rng.standard_normal(H)
    h0 = rng.standard_normal((1, H, P, N))
    # recurrence through the oracle
    h, ys = h0, []
    for t in range(T):
        y, h = m2.ssm_step(xs[t][None], Bs[t][None], Cs[t][None], dts_raw[t][None], h, dt_bias, A_log, D)
        ys.append(y[0])
    # quadratic form, written out with explicit loops
    dt = [[math.log1p(math.exp(dts_raw[t, k] + dt_bias[k])) for k in range(H)] for t in range(T)]
    dA = [[math.exp(-dt[t][k] * math.exp(A_log[k])) for k in range(H)] for t in range(T)]
    for t in range(T):
        for k in range(H):
            for p in range(P):
                acc = D[k] * xs[t, k, p]
                decay0 = 1.0
                for r in range(t + 1):
                    decay0 *= dA[r][k]
                acc += decay0 * sum(h0[0, k, p, n] * Cs[t, n] for n in range(N))
                for s in range(t + 1):
                    decay = 1.0
                    for r in range(s + 1, t + 1):
                        decay *= dA[r][k]
                    cb = sum(Cs[t, n] * Bs[s, n] for n in range(N))
                    acc += decay * dt[s][k] * cb * xs[s, k, p]
                assert abs(ys[t][k, p] - acc) <= 1e-12 * (1 + abs(acc)), (t, k, p)


def test_gated_rmsnorm_properties():
    rng = np.random.default_rng(3)
    y = rng.standard_normal((3, 64))
    z = rng.standard_normal((3, 64))
    w = rng.uniform(0.5, 1.5, 64)
    out = m2.gated_rmsnorm(y, z, w, 0.0)
    assert np.allclose(m2.gated_rmsnorm(7.5 * y, z, w, 0.0), out, rtol=1e-13)   # scale invariance (eps = 0)
    assert np.allclose(((out / w) ** 2).mean(axis=1), 1.0, rtol=1e-13)
    # the gate multiplies before the norm: a gate of silu(z) = 0 on half the channels
    # leaves the other half with mean square 2 (eps = 0)
    z2 = z.copy()
    z2[:, :32] = 0.0
    out2 = m2.gated_rmsnorm(y, z2, np.ones(64), 0.0)
    assert np.all(out2[:, :32] == 0.0)
    assert np.allclose((out2[:, 32:] ** 2).mean(axis=1), 2.0, rtol=1e-13)
    # eps enters under the square root
    g = y * z / (1 + np.exp(-z))
    ms = (g * g).mean(axis=1, keepdims=True)
    assert np.allclose(m2.gated_rmsnorm(y, z, w, 0.25), g / np.sqrt(ms + 0.25) * w, rtol=1e-13)


def test_decode_step_layout_hand_sized():
    # nheads 2, headdim 2, d_state 2: d_inner 4, conv_dim 8, width 4 + 8 + 2 = 14.
    # Taps pick the newest value (no bias), the SSM state starts at a known value, eps 0.
    H, P, N = 2, 2, 2
    z = [0.5, -1.0, 2.0, 1.5]
    xv = [0.3, -0.7, 1.1, 0.2]
    Bv = [0.9, -0.4]
    Cv = [-0.6, 1.3]
    dtr = [0.1, -0.8]
    zxbcdt = np.array([z + xv + Bv + Cv + dtr])
    conv_w = np.zeros((8, 4))
    conv_w[:, 3] = 1.0
    h0 = np.arange(H * P * N, dtype=np.float64).reshape(1, H, P, N) / 10.0
    dt_bias, A_log, Dp = np.array([0.2, -0.3]), np.array([0.4, 1.0]), np.array([1.5, 0.5])
    nw = np.array([1.0, 2.0, 0.5, 1.0])
    out, window, state = m2.decode_step(zxbcdt, np.zeros((1, 8, 4)), h0, conv_w, np.zeros(8), dt_bias, A_log, Dp,
                                        nw, H, P, N, eps=0.0)

    def silu(v):
        return v / (1.0 + math.exp(-v))

    x = [[silu(xv[2 * k + p]) for p in range(P)] for k in range(H)]
    B = [silu(v) for v in Bv]
    C = [silu(v) for v in Cv]
    ys = []
    for k in range(H):
        dt = math.log(1.0 + math.exp(dtr[k] + dt_bias[k]))
        dA = math.exp(-dt * math.exp(A_log[k]))
        for p in range(P):
            hs = [h0[0, k, p, n] * dA + dt * x[k][p] * B[n] for n in range(N)]
            for n in range(N):
                assert abs(state[0, k, p, n] - hs[n]) < 1e-14
            ys.append(sum(hs[n] * C[n] for n in range(N)) + Dp[k] * x[k][p])
    g = [ys[i] * silu(z[i]) for i in range(4)]
    r = 1.0 / math.sqrt(sum(v * v for v in g) / 4)
    for i in range(4):
        assert abs(out[0, i] - g[i] * r * nw[i]) < 1e-13
    assert np.array_equal(window[0, :, 3], np.array(xv + Bv + Cv))
