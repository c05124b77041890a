"""Pins of the decode-chain oracle (oracle/decode_chain.py) that do not come from the
oracle itself (CPU only).

The chain only wires pinned oracles together (quantizer and projection:
tests/test_oracle_pins.py; the Mamba-2 step: tests/test_oracle_mamba2_pins.py), so
these pins target the wiring:
  * all-zero convolution weights and biases make every convolution output silu(0) = 0,
    so x, B and C are zero, y = 0, the gated norm's output is exactly zero, its
    quantization gives s_x = 0, and the out_proj output is exactly zero -- for any
    projection weights and any state; the next layer then sees an all-zero input and
    its in_proj output is exactly zero too;
  * permuting the heads consistently (in_proj's z, x and dt rows, the Mamba-2 per-head
    parameters, the windows of the x channels, the state, norm_w and out_proj's input
    columns) permutes the intermediate rows but leaves each layer's output x' as it
    was: a head's dt, decay, D, state or gate taken from another head fails it;
  * layer l's output does not depend on any later layer's weights.
"""
import numpy as np

import synth_inputs as si
from oracle import decode_chain as dc


def _small_stack(seed, L=2):
    return si.draw_decode_stack(np.random.default_rng(seed), L)


def test_zero_convolution_makes_every_output_exactly_zero():
    st = _small_stack(1)
    st.conv_w[:] = 0.0
    st.conv_b[:] = 0.0
    x_out, recs = dc.decode_token(st, st.x, st.conv_state, st.ssm_state, nthreads=8)
    assert not recs[0]["out"].any() and recs[0]["sx_out"] == 0.0
    assert not recs[0]["x_next"].any()
    # the second layer's input is all zero: its in_proj output is exactly zero
    assert recs[1]["sx_in"] == 0.0 and not recs[1]["zx"].any()
    assert not x_out.any()


def _permute_heads(st, perm):
    """The same model with its heads reordered by perm (new head i = old head perm[i])."""
    d_inner = 4096
    ch = (perm[:, None] * 64 + np.arange(64)[None, :]).reshape(-1)          # channel order within d_inner
    rows = np.concatenate([ch, d_inner + ch, np.arange(2 * d_inner, 2 * d_inner + 256),
                           2 * d_inner + 256 + perm])                        # z | x | B, C | dt
    conv_rows = np.concatenate([ch, np.arange(d_inner, d_inner + 256)])      # x channels | B, C
    out_bits = np.unpackbits(st.out_P, axis=2, bitorder="little")[:, :, ch]
    out = si.DecodeStack(**{k: v.copy() for k, v in vars(st).items()})
    out.in_P = st.in_P[:, rows]
    out.in_s_w = st.in_s_w[:, rows]
    out.in_W_A = st.in_W_A[:, rows]
    out.in_s_A = st.in_s_A[:, rows]
    out.conv_w = st.conv_w[:, conv_rows]
    out.conv_b = st.conv_b[:, conv_rows]
    out.conv_state = st.conv_state[:, conv_rows]
    out.dt_bias = st.dt_bias[:, perm]
    out.A_log = st.A_log[:, perm]
    out.D = st.D[:, perm]
    out.norm_w = st.norm_w[:, ch]
    out.ssm_state = st.ssm_state[:, perm]
    out.out_P = np.packbits(out_bits, axis=2, bitorder="little")
    out.out_W_B = st.out_W_B[:, :, ch]
    return out, ch


def test_head_permutation_leaves_layer_outputs_unchanged():
    st = _small_stack(2, L=1)
    perm = np.random.default_rng(3).permutation(64)
    ps, ch = _permute_heads(st, perm)
    _, r0 = dc.decode_token(st, st.x, st.conv_state, st.ssm_state, nthreads=8)
    _, r1 = dc.decode_token(ps, ps.x, ps.conv_state, ps.ssm_state, nthreads=8)
    a, b = r0[0], r1[0]
    # the intermediates are the same values in the new order (the projection is exact
    # up to its one rounding; the Mamba-2 step is computed per head in fp64)
    np.testing.assert_array_equal(a["zx"][ch], b["zx"][:4096])
    np.testing.assert_allclose(a["out"][ch], b["out"], rtol=1e-6, atol=1e-12)
    np.testing.assert_allclose(a["ssm_state"][perm], b["ssm_state"], rtol=1e-12, atol=1e-300)
    # the layer's output: the norm's mean square sums in another order, so the out
    # values (and, at a rare tie, a code) may move by an ulp; the output stays within
    # the projection's bar
    scale = np.abs(a["x_next"]).max()
    assert np.abs(a["x_next"].astype(np.float64) - b["x_next"]).max() <= 1e-4 * scale


def test_layer_output_does_not_depend_on_later_layers():
    st = _small_stack(4, L=2)
    _, r0 = dc.decode_token(st, st.x, st.conv_state, st.ssm_state, nthreads=8)
    st.in_P[1] = ~st.in_P[1]
    st.out_W_A[1] = 0
    st.D[1] = 5.0
    _, r1 = dc.decode_token(st, st.x, st.conv_state, st.ssm_state, nthreads=8)
    for k in ("zx", "out", "x_next", "xq_out"):
        np.testing.assert_array_equal(r0[0][k], r1[0][k])
    assert not np.array_equal(r0[1]["x_next"], r1[1]["x_next"])
