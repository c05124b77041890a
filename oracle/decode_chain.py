"""CPU oracle of one decode token through a stack of DF-SSM layers -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this module; the product path never imports it, and it
never imports the product path.

DF-SSM technical summary (gist.science), section 2C "Optimized Inference Pipeline":
a decode step runs every layer's in_proj (1-bit scaffold + int8 LoRA), the stateful
convolution and SSM recurrence, and out_proj (section 2B: LoRA on both projections
of all 48 layers).  This module only chains the oracles that define those steps, in
that order, for one sequence:

  x_q, s_x      = quantize_act(x)                               (dfssm_oracle.c)
  zxbcdt        = scaffold_lora_gemm(x_q, s_x, in_proj of l)    (dfssm_oracle.c; fp64, rounded to fp32)
  out           = mamba2.decode_step(zxbcdt, windows, state)    (mamba2.py, fp64)
  x_q', s_x'    = quantize_act(fl32(out))
  x'            = scaffold_lora_gemm(x_q', s_x', out_proj of l)
and x' is layer l + 1's input.  The Mamba-2 step's output is rounded to fp32 before it
is quantized, as a device would hold it.

Parity status: the steps are the pinned oracles above; the chaining is pinned by
``tests/test_oracle_decode_chain_pins.py`` (all-zero convolution parameters make every
layer's output exactly zero whatever the weights; a permutation of the heads --
in_proj rows, Mamba-2 parameters, state, out_proj columns -- leaves every layer's
output unchanged; layer l's output does not depend on later layers).
"""
from __future__ import annotations

import numpy as np

from . import mamba2, quantize_act, scaffold_lora_gemm

NHEADS, HEADDIM, DSTATE = 64, 64, 128


def layer_step(stack, l, x, conv_state, ssm_state, eps=1e-5, nthreads=1):
    """One layer for one token.  x fp32 [2048]; conv_state [4352, 4]; ssm_state
    [64, 64, 128].  Returns a dict of the layer's intermediates and new state."""
    xq, sx = quantize_act(np.asarray(x, np.float32)[None])
    zx, acc_in, t_in = scaffold_lora_gemm(xq, sx, stack.in_P[l], stack.in_s_w[l], stack.in_W_A[l], stack.in_s_A[l],
                                          stack.in_W_B[l], stack.in_s_B[l], nthreads=nthreads)
    out, window, state = mamba2.decode_step(zx, conv_state[None], ssm_state[None], stack.conv_w[l], stack.conv_b[l],
                                            stack.dt_bias[l], stack.A_log[l], stack.D[l], stack.norm_w[l],
                                            NHEADS, HEADDIM, DSTATE, eps)
    out32 = out.astype(np.float32)
    xq2, sx2 = quantize_act(out32)
    xn, acc_out, t_out = scaffold_lora_gemm(xq2, sx2, stack.out_P[l], stack.out_s_w[l], stack.out_W_A[l],
                                            stack.out_s_A[l], stack.out_W_B[l], stack.out_s_B[l], nthreads=nthreads)
    return dict(xq_in=xq[0], sx_in=sx[0], zx=zx[0], acc_in=acc_in[0], t_in=t_in[0], out=out32[0],
                xq_out=xq2[0], sx_out=sx2[0], x_next=xn[0], acc_out=acc_out[0], t_out=t_out[0],
                conv_state=window[0], ssm_state=state[0])


def decode_token(stack, x, conv_state, ssm_state, eps=1e-5, nthreads=1):
    """One token through all layers.  conv_state [L, 4352, 4], ssm_state [L, 64, 64, 128]
    (fp64 or fp32).  Returns (x_out, per-layer records)."""
    records = []
    for l in range(stack.L):
        rec = layer_step(stack, l, x, conv_state[l], ssm_state[l], eps, nthreads)
        records.append(rec)
        x = rec["x_next"]
    return x, records
