"""CPU oracle for the Mamba-2 decode step around the projections -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this module; the product path never imports it, and it
never imports the product path.

The pages name the step but not its arithmetic: DF-SSM technical summary
(gist.science), section 2C "Optimized Inference Pipeline", Stateful Ops -- custom
kernels for the stateful shift register (the causal convolution) and the SSM
recurrence (with a reduction), on Mamba-2 1.3B (abstract; d_model 2048, d_inner
4096, in_proj width 8512 = 2 * 4096 + 2 * 128 + 64).  The arithmetic below is the
published Mamba-2 single-token step, restated from its definition, in fp64 numpy:

  in_proj output (one token)  = [z (d_inner) | xBC (d_inner + 2 d_state) | dt (nheads)]
  conv (depthwise, width 4)   : the channel's window shifts left by one and takes the
                                new value; c = sum_j w[c, j] window[c, j] + b[c];
                                xBC = silu(c)
  split                       : x (nheads x headdim), B (d_state), C (d_state)  (one group)
  dt = softplus(dt_raw + dt_bias),  A = -exp(A_log),  dA = exp(dt A)      (per head)
  state[h, p, n] <- state[h, p, n] dA[h] + dt[h] x[h, p] B[n]
  y[h, p] = sum_n state[h, p, n] C[n] + D[h] x[h, p]
  gated RMS norm (gate first)  : g = y silu(z);  out = g / sqrt(mean(g^2) + eps) w

softplus(v) = log(1 + exp(v)), returned as v itself for v > 20 (the threshold the
reference implementation uses; the two differ there by < exp(-20) relative).
silu(v) = v / (1 + exp(-v)).

Parity status: pinned by ``tests/test_oracle_mamba2_pins.py`` -- closed forms of one step
from a zero state, pure decay with B = 0, a one-hot convolution that reproduces the
shifted window, the recurrence against the quadratic (attention-like) form of the same
SSM over several steps computed independently, and the norm's scale invariance.
"""
from __future__ import annotations

import numpy as np

D_CONV = 4
SOFTPLUS_THRESHOLD = 20.0


def softplus(v):
    v = np.asarray(v, dtype=np.float64)
    return np.where(v > SOFTPLUS_THRESHOLD, v, np.log1p(np.exp(np.minimum(v, SOFTPLUS_THRESHOLD))))


def silu(v):
    v = np.asarray(v, dtype=np.float64)
    return v / (1.0 + np.exp(-v))


def conv_step(xbc_new, conv_state, conv_w, conv_b):
    """Causal depthwise convolution, one token: the shift register advances by one.

    xbc_new [S, C] the new values; conv_state [S, C, 4] the previous window (oldest
    first); conv_w [C, 4]; conv_b [C].  Returns (silu(conv) [S, C], new window)."""
    xbc_new = np.asarray(xbc_new, np.float64)
    window = np.concatenate([np.asarray(conv_state, np.float64)[:, :, 1:], xbc_new[:, :, None]], axis=2)
    c = (window * np.asarray(conv_w, np.float64)[None]).sum(axis=2) + np.asarray(conv_b, np.float64)[None]
    return silu(c), window


def ssm_step(x, B, C, dt_raw, ssm_state, dt_bias, A_log, D):
    """Selective state update, one token.

    x [S, H, P]; B, C [S, N]; dt_raw [S, H]; ssm_state [S, H, P, N]; dt_bias, A_log,
    D [H].  Returns (y [S, H, P], new state)."""
    x = np.asarray(x, np.float64)
    B = np.asarray(B, np.float64)
    C = np.asarray(C, np.float64)
    dt = softplus(np.asarray(dt_raw, np.float64) + np.asarray(dt_bias, np.float64)[None])   # [S, H]
    A = -np.exp(np.asarray(A_log, np.float64))                                              # [H]
    dA = np.exp(dt * A[None])                                                               # [S, H]
    state = np.asarray(ssm_state, np.float64) * dA[:, :, None, None] + \
        (dt[:, :, None] * x)[:, :, :, None] * B[:, None, None, :]
    y = (state * C[:, None, None, :]).sum(axis=3) + np.asarray(D, np.float64)[None, :, None] * x
    return y, state


def gated_rmsnorm(y, z, w, eps):
    """g = y silu(z); g / sqrt(mean(g^2) + eps) * w, per token over the last axis."""
    g = np.asarray(y, np.float64) * silu(z)
    r = 1.0 / np.sqrt((g * g).mean(axis=-1, keepdims=True) + eps)
    return g * r * np.asarray(w, np.float64)[None]


def decode_step(zxbcdt, conv_state, ssm_state, conv_w, conv_b, dt_bias, A_log, D, norm_w,
                nheads: int, headdim: int, d_state: int, eps: float = 1e-5):
    """One Mamba-2 token step between in_proj and out_proj.

    zxbcdt [S, 2 d_inner + 2 d_state + nheads] (fp32 in_proj output); conv_state
    [S, d_inner + 2 d_state, 4]; ssm_state [S, nheads, headdim, d_state].  Returns
    (out [S, d_inner] fp64: the out_proj input, new conv_state, new ssm_state)."""
    S = zxbcdt.shape[0]
    d_inner = nheads * headdim
    conv_dim = d_inner + 2 * d_state
    zxbcdt = np.asarray(zxbcdt, np.float64)
    z = zxbcdt[:, :d_inner]
    xbc = zxbcdt[:, d_inner:d_inner + conv_dim]
    dt_raw = zxbcdt[:, d_inner + conv_dim:d_inner + conv_dim + nheads]
    act, window = conv_step(xbc, conv_state, conv_w, conv_b)
    x = act[:, :d_inner].reshape(S, nheads, headdim)
    B = act[:, d_inner:d_inner + d_state]
    C = act[:, d_inner + d_state:]
    y, state = ssm_step(x, B, C, dt_raw, ssm_state, dt_bias, A_log, D)
    out = gated_rmsnorm(y.reshape(S, d_inner), z, norm_w, eps)
    return out, window, state
