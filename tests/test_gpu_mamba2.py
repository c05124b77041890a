"""GPU parity of the Mamba-2 decode step (dfssm_mamba2_decode_step) against the CPU oracle.

The oracle (oracle/mamba2.py) runs in fp64 on the same fp32 inputs; the kernels run in
fp32 with the library's exp / log1p.  Each fp32 operation adds at most a few 2^-24 of
the magnitude of its operands, so the bar follows the magnitudes through the step:
  * convolution channel c: A_c = |b| + sum_j |w_j window_j| (its terms can cancel, and
    the error is a fraction of the terms, not of the sum); its activation's magnitude
    is |silu(a)| + 1.1 A_c (silu' stays below 1.1);
  * decay dA = exp(-E), E = dt exp(A_log): an error of a fraction of E in the exponent
    is E times that in dA, so the decay term counts (1 + E) |h dA|;
  * state: H = (1 + E) |h dA| + dt X B_m (X, B_m the activation magnitudes);
  * y: Y = sum_n (|h'| + H_n) C_m[n] + |D| X;  out: Y |silu(z)| r |w| + |out|, r the
    oracle's norm factor;
and every element must lie within TOL = 1e-5 of its magnitude (x the step count over
several steps, where the GPU keeps its fp32 state and the oracle its fp64 state).  The
advanced convolution windows are a shift and a copy: bit-exact.
"""
import numpy as np
import pytest

import synth_inputs as si
from oracle import mamba2 as m2
from test_gpu_parity import torch_cuda  # noqa: F401  (fixture)

pytestmark = pytest.mark.gpu

TOL = 1e-5
EPS = 1e-5


def _layer_to_gpu(layer):
    import torch
    return {k: torch.from_numpy(getattr(layer, k)).cuda() for k in ("conv_w", "conv_b", "dt_bias", "A_log", "D", "norm_w")}


def _gpu_steps(layer, zxbcdts, conv_state, ssm_state, eps=EPS):
    """Run len(zxbcdts) steps on the GPU; returns per step (out, conv_state, ssm_state)."""
    import torch
    from bit_scaffold_int8_amd import dfssm
    L = _layer_to_gpu(layer)
    S = conv_state.shape[0]
    d_inner = ssm_state.shape[1] * ssm_state.shape[2]
    conv = [torch.from_numpy(conv_state).cuda(), torch.empty_like(torch.from_numpy(conv_state)).cuda()]
    ssm = torch.from_numpy(ssm_state.copy()).cuda()
    out = torch.empty((S, d_inner), dtype=torch.float32, device="cuda")
    res = []
    for i, z in enumerate(zxbcdts):
        zx = torch.from_numpy(z).cuda()
        dfssm.dfssm_mamba2_decode_step(zx, conv[i % 2], conv[(i + 1) % 2], ssm, L["conv_w"], L["conv_b"],
                                       L["dt_bias"], L["A_log"], L["D"], L["norm_w"], eps, out)
        torch.cuda.synchronize()
        res.append((out.cpu().numpy().copy(), conv[(i + 1) % 2].cpu().numpy().copy(), ssm.cpu().numpy().copy()))
    return res


def _oracle_step_with_magnitudes(layer, zxbcdt, conv_state, ssm_state, nheads, headdim, d_state, eps):
    """The oracle step, plus the magnitudes the bar uses."""
    out, window, state = m2.decode_step(zxbcdt, conv_state, ssm_state, layer.conv_w, layer.conv_b, layer.dt_bias,
                                        layer.A_log, layer.D, layer.norm_w, nheads, headdim, d_state, eps)
    S = zxbcdt.shape[0]
    d_inner = nheads * headdim
    conv_dim = d_inner + 2 * d_state
    f64 = np.float64
    z = zxbcdt[:, :d_inner].astype(f64)
    act, win = m2.conv_step(zxbcdt[:, d_inner:d_inner + conv_dim], conv_state, layer.conv_w, layer.conv_b)
    a_terms = np.abs(win * layer.conv_w.astype(f64)[None]).sum(axis=2) + np.abs(layer.conv_b.astype(f64))[None]
    act_mag = np.abs(act) + 1.1 * a_terms
    X = act_mag[:, :d_inner].reshape(S, nheads, headdim)
    Bm = act_mag[:, d_inner:d_inner + d_state]
    Cm = act_mag[:, d_inner + d_state:]
    dt = m2.softplus(zxbcdt[:, d_inner + conv_dim:].astype(f64) + layer.dt_bias.astype(f64)[None])
    E = dt * np.exp(layer.A_log.astype(f64))[None]
    dA = np.exp(-E)
    H = (1.0 + E)[:, :, None, None] * np.abs(ssm_state.astype(f64) * dA[:, :, None, None]) + \
        (dt[:, :, None] * X)[..., None] * Bm[:, None, None, :]
    Y = ((np.abs(state) + H) * Cm[:, None, None, :]).sum(axis=3) + np.abs(layer.D.astype(f64))[None, :, None] * X
    y = (state * act[:, None, None, d_inner + d_state:]).sum(axis=3) + \
        layer.D.astype(f64)[None, :, None] * act[:, :d_inner].reshape(S, nheads, headdim)
    g = y.reshape(S, d_inner) * m2.silu(z)
    r = 1.0 / np.sqrt((g * g).mean(axis=1, keepdims=True) + eps)
    out_mag = Y.reshape(S, d_inner) * np.abs(m2.silu(z)) * r * np.abs(layer.norm_w.astype(f64))[None] + np.abs(out)
    return out, window, state, H, out_mag


def _check(layer, zxbcdts, conv_state, ssm_state, eps=EPS):
    S, nheads, headdim, d_state = ssm_state.shape
    got = _gpu_steps(layer, zxbcdts, conv_state, ssm_state, eps)
    cs, hs = conv_state, ssm_state.astype(np.float64)
    for i, z in enumerate(zxbcdts):
        out, window, state, state_mag, out_mag = _oracle_step_with_magnitudes(layer, z, cs, hs, nheads, headdim,
                                                                              d_state, eps)
        g_out, g_conv, g_ssm = got[i]
        assert np.array_equal(g_conv, window.astype(np.float32)), f"step {i}: windows"
        k = i + 1
        err = np.abs(g_ssm.astype(np.float64) - state)
        bad = err > k * TOL * state_mag + 1e-30
        assert not bad.any(), f"step {i}: {bad.sum()} state values outside the bar, worst " \
                              f"{(err / np.maximum(state_mag, 1e-300)).max():.2e}"
        err = np.abs(g_out.astype(np.float64) - out)
        lim = k * TOL * out_mag + 1e-30
        bad = err > lim
        assert not bad.any(), f"step {i}: {bad.sum()} outputs outside the bar, worst {(err / lim).max():.2e} of it"
        cs, hs = window, state


@pytest.mark.parametrize("S", [1, 3, 64])
def test_mamba2_step_matches_oracle(torch_cuda, S):
    rng = np.random.default_rng(si.CONFIGS["mamba2_decode_step"]["seed"] + S)
    layer = si.draw_mamba2_layer(rng)
    zx, conv, ssm = si.draw_mamba2_inputs(rng, S)
    _check(layer, [zx], conv, ssm)


def test_mamba2_steps_carry_state(torch_cuda):
    # four tokens in a row: the windows ping-pong, the state is updated in place
    rng = np.random.default_rng(41)
    layer = si.draw_mamba2_layer(rng)
    zx0, conv, ssm = si.draw_mamba2_inputs(rng, 2)
    zxs = [zx0] + [si.draw_mamba2_inputs(rng, 2)[0] for _ in range(3)]
    _check(layer, zxs, conv, ssm)


@pytest.mark.parametrize("nheads", [1, 3, 24])
def test_mamba2_step_other_head_counts(torch_cuda, nheads):
    rng = np.random.default_rng(50 + nheads)
    layer = si.draw_mamba2_layer(rng, nheads=nheads)
    zx, conv, ssm = si.draw_mamba2_inputs(rng, 2, nheads=nheads)
    _check(layer, [zx], conv, ssm)


def test_mamba2_step_dt_extremes_and_zero_state(torch_cuda):
    # dt above the softplus threshold (identity, the state is all but replaced) and far
    # below it (dt ~ 1e-9: the state barely moves), from a zero state on one sequence
    rng = np.random.default_rng(60)
    layer = si.draw_mamba2_layer(rng)
    zx, conv, ssm = si.draw_mamba2_inputs(rng, 3)
    d_inner, conv_dim = 4096, 4096 + 256
    zx[0, d_inner + conv_dim:] = 40.0
    zx[1, d_inner + conv_dim:] = -15.0
    ssm[2] = 0.0
    _check(layer, [zx], conv, ssm)


def test_mamba2_step_eps_zero_and_large_inputs(torch_cuda):
    rng = np.random.default_rng(61)
    layer = si.draw_mamba2_layer(rng)
    zx, conv, ssm = si.draw_mamba2_inputs(rng, 2)
    zx *= 30.0        # large pre-activations: silu saturates on both sides
    _check(layer, [zx], conv, ssm, eps=0.0)


def test_mamba2_steps_33_sequences_5_heads(torch_cuda):
    # two steps at 33 sequences of 5 heads
    rng = np.random.default_rng(70)
    layer = si.draw_mamba2_layer(rng, nheads=5)
    zx0, conv, ssm = si.draw_mamba2_inputs(rng, 33, nheads=5)
    zx1 = si.draw_mamba2_inputs(rng, 33, nheads=5)[0]
    _check(layer, [zx0, zx1], conv, ssm)
