"""Seeded synthetic inputs for the DF-SSM scaffold projection.

This module only draws random numbers: it holds none of the projection's
arithmetic (no quantization, no sign packing, no products), so both the HIP
path's tests/benchmark and the CPU oracle can consume the same buffers.

Shapes follow the Mamba-2 1.3B layout the pages name (DF-SSM technical summary,
section 2B: LoRA on in_proj and out_proj of all 48 layers; d_model 2048,
d_inner 4096, in_proj width 2*4096 + 2*128 + 64 = 8512).  Distributions:
sign bits are uniform random bytes (iid Bernoulli(1/2) signs), the scaffold
scale s_w ~ U[0.01, 0.05], activations x ~ N(0, 1) fp32 with a few outlier
input channels scaled by 20, LoRA matrices uniform int8 in [-127, 127] with
per-row scales ~ U[1e-4, 1e-3].

Draw order per problem (numpy PCG64 via default_rng(seed)):
  1. P   = integers(0, 256, (N, K/8), uint8)
  2. s_w = uniform(0.01, 0.05, N)           -> float32
  3. x   = standard_normal((M, K), float32)
  4. idx = choice(K, n_outliers, replace=False); x[:, idx] *= 20
  5. W_A = integers(-127, 128, (N, r), int8), s_A = uniform(1e-4, 1e-3, N)
  6. W_B = integers(-127, 128, (r, K), int8), s_B = uniform(1e-4, 1e-3, r)
Further copies (rotated weight sets) continue the same generator stream.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

RANK = 16


@dataclass
class Problem:
    """One projection's inputs (host numpy arrays)."""
    x: np.ndarray      # float32 [M, K]
    P: np.ndarray      # uint8   [N, K/8]  sign bits, LSB = lowest k, 1 = +1
    s_w: np.ndarray    # float32 [N]
    W_A: np.ndarray    # int8    [N, r]
    s_A: np.ndarray    # float32 [N]
    W_B: np.ndarray    # int8    [r, K]
    s_B: np.ndarray    # float32 [r]

    @property
    def M(self):
        return self.x.shape[0]

    @property
    def K(self):
        return self.x.shape[1]

    @property
    def N(self):
        return self.P.shape[0]


def draw_problem(rng: np.random.Generator, M: int, N: int, K: int, n_outliers: int,
                 rank: int = RANK) -> Problem:
    if K % 8:
        raise ValueError("K must be a multiple of 8")
    P = rng.integers(0, 256, (N, K // 8), dtype=np.uint8)
    s_w = rng.uniform(0.01, 0.05, N).astype(np.float32)
    x = rng.standard_normal((M, K), dtype=np.float32)
    if n_outliers:
        idx = rng.choice(K, n_outliers, replace=False)
        x[:, idx] *= np.float32(20.0)
    W_A = rng.integers(-127, 128, (N, rank), dtype=np.int8)
    s_A = rng.uniform(1e-4, 1e-3, N).astype(np.float32)
    W_B = rng.integers(-127, 128, (rank, K), dtype=np.int8)
    s_B = rng.uniform(1e-4, 1e-3, rank).astype(np.float32)
    return Problem(x, P, s_w, W_A, s_A, W_B, s_B)


def make_problem(M: int, N: int, K: int, n_outliers: int, seed: int, rank: int = RANK) -> Problem:
    return draw_problem(np.random.default_rng(seed), M, N, K, n_outliers, rank)


def make_copies(M: int, N: int, K: int, n_outliers: int, seed: int, copies: int,
                rank: int = RANK) -> list[Problem]:
    """`copies` independent problems drawn back to back from one seeded stream."""
    rng = np.random.default_rng(seed)
    return [draw_problem(rng, M, N, K, n_outliers, rank) for _ in range(copies)]


@dataclass
class HeadProblem:
    """The int8 embedding / LM head's inputs: tokens' fp32 activations and the int8
    matrix with its per-row scales (host numpy arrays)."""
    x: np.ndarray      # float32 [M, K]
    E: np.ndarray      # int8    [N, K]
    s_e: np.ndarray    # float32 [N]


def draw_head(rng: np.random.Generator, M: int, N: int, K: int) -> HeadProblem:
    """Rows of per-row absmax int8 codes (uniform in [-127, 127]) with scales in
    [1e-3, 1e-2], and N(0, 1) activations (the final hidden state of a token)."""
    E = rng.integers(-127, 128, (N, K), dtype=np.int8)
    s_e = rng.uniform(1e-3, 1e-2, N).astype(np.float32)
    x = rng.standard_normal((M, K), dtype=np.float32)
    return HeadProblem(x, E, s_e)


def make_head(M: int, N: int, K: int, seed: int) -> HeadProblem:
    return draw_head(np.random.default_rng(seed), M, N, K)


# Mamba-2 1.3B mixer sizes around the projections (in_proj width 8512 = 2 * 4096 +
# 2 * 128 + 64): 64 heads of 64 channels, state size 128, one group, convolution width 4.
MAMBA2_NHEADS, MAMBA2_HEADDIM, MAMBA2_DSTATE, MAMBA2_DCONV = 64, 64, 128, 4


@dataclass
class Mamba2Layer:
    """One layer's decode-step parameters (host numpy arrays, float32)."""
    conv_w: np.ndarray    # [conv_dim, 4]
    conv_b: np.ndarray    # [conv_dim]
    dt_bias: np.ndarray   # [nheads]
    A_log: np.ndarray     # [nheads]
    D: np.ndarray         # [nheads]
    norm_w: np.ndarray    # [d_inner]


def draw_mamba2_layer(rng: np.random.Generator, nheads: int = MAMBA2_NHEADS, headdim: int = MAMBA2_HEADDIM,
                      d_state: int = MAMBA2_DSTATE) -> Mamba2Layer:
    """Draw order: conv_w U(-0.5, 0.5), conv_b U(-0.5, 0.5), dt_bias U(-7, -2) (softplus
    of it spans ~1e-3 .. 0.13), A_log U(0, log 16), D U(0.5, 1.5), norm_w 1 + 0.1 N(0, 1)."""
    d_inner = nheads * headdim
    conv_dim = d_inner + 2 * d_state
    f32 = np.float32
    conv_w = rng.uniform(-0.5, 0.5, (conv_dim, MAMBA2_DCONV)).astype(f32)
    conv_b = rng.uniform(-0.5, 0.5, conv_dim).astype(f32)
    dt_bias = rng.uniform(-7.0, -2.0, nheads).astype(f32)
    A_log = rng.uniform(0.0, np.log(16.0), nheads).astype(f32)
    D = rng.uniform(0.5, 1.5, nheads).astype(f32)
    norm_w = (1.0 + 0.1 * rng.standard_normal(d_inner)).astype(f32)
    return Mamba2Layer(conv_w, conv_b, dt_bias, A_log, D, norm_w)


def draw_mamba2_inputs(rng: np.random.Generator, S: int, nheads: int = MAMBA2_NHEADS,
                       headdim: int = MAMBA2_HEADDIM, d_state: int = MAMBA2_DSTATE):
    """One step's (zxbcdt [S, 2 d_inner + 2 d_state + nheads], conv_state [S, conv_dim, 4],
    ssm_state [S, nheads, headdim, d_state]) for S sequences, all float32: zxbcdt and the
    convolution windows N(0, 1), the SSM state 0.1 N(0, 1)."""
    d_inner = nheads * headdim
    conv_dim = d_inner + 2 * d_state
    f32 = np.float32
    zxbcdt = rng.standard_normal((S, d_inner + conv_dim + nheads), dtype=f32)
    conv_state = rng.standard_normal((S, conv_dim, MAMBA2_DCONV), dtype=f32)
    ssm_state = (0.1 * rng.standard_normal((S, nheads, headdim, d_state), dtype=f32)).astype(f32)
    return zxbcdt, conv_state, ssm_state


# The workloads: (name, list of (M, N, K, n_outliers), seed)
CONFIGS = {
    "tiny_m1_k256_n512": dict(shapes=[(1, 512, 256, 2)], seed=0),
    "out_proj_decode_m1_k4096_n2048": dict(shapes=[(1, 2048, 4096, 2)], seed=1),
    "in_proj_decode_k2048_n8512": dict(shapes=[(1, 8512, 2048, 2), (4, 8512, 2048, 2),
                                               (16, 8512, 2048, 2)], seed=2),
    # 48 layers x (in_proj K2048->N8512, out_proj K4096->N2048), fresh N(0,1) inputs
    "decode_sweep_48l": dict(shapes=[(1, 8512, 2048, 0), (1, 2048, 4096, 0)], seed=3, layers=48),
    # prefill: 1 % outlier channels (round(0.01 K)) -> 20 at K 2048, 41 at K 4096
    "prefill_m2048": dict(shapes=[(2048, 8512, 2048, 20), (2048, 2048, 4096, 41)], seed=4),
    # int8 LM head of the model: vocabulary 50280 x width 2048, decode token counts
    "lm_head_decode_v50280_d2048": dict(shapes=[(1, 50280, 2048), (4, 50280, 2048), (16, 50280, 2048)], seed=5),
    # the Mamba-2 step between the projections (conv shift register, SSM recurrence,
    # gated RMS norm): 64 heads x 64 channels, state 128, at 1 and 64 sequences
    "mamba2_decode_step": dict(sequences=[1, 64], seed=6),
}


def prefill_problems() -> list[Problem]:
    """The M = 2048 prefill workload: in_proj (K 2048 -> N 8512), then out_proj
    (K 4096 -> N 2048), drawn back to back from one stream seeded as the workload says."""
    cfg = CONFIGS["prefill_m2048"]
    rng = np.random.default_rng(cfg["seed"])
    return [draw_problem(rng, *shape) for shape in cfg["shapes"]]


@dataclass
class DecodeStack:
    """A stack of L layers' decode weights and state for one sequence (host arrays,
    stacked over layers in the layout the persistent decode entry point reads)."""
    in_P: np.ndarray       # uint8 [L, 8512, 256]
    in_s_w: np.ndarray     # float32 [L, 8512]
    in_W_A: np.ndarray     # int8 [L, 8512, 16]
    in_s_A: np.ndarray     # float32 [L, 8512]
    in_W_B: np.ndarray     # int8 [L, 16, 2048]
    in_s_B: np.ndarray     # float32 [L, 16]
    conv_w: np.ndarray     # float32 [L, 4352, 4]
    conv_b: np.ndarray     # float32 [L, 4352]
    dt_bias: np.ndarray    # float32 [L, 64]
    A_log: np.ndarray      # float32 [L, 64]
    D: np.ndarray          # float32 [L, 64]
    norm_w: np.ndarray     # float32 [L, 4096]
    out_P: np.ndarray      # uint8 [L, 2048, 512]
    out_s_w: np.ndarray    # float32 [L, 2048]
    out_W_A: np.ndarray    # int8 [L, 2048, 16]
    out_s_A: np.ndarray    # float32 [L, 2048]
    out_W_B: np.ndarray    # int8 [L, 16, 4096]
    out_s_B: np.ndarray    # float32 [L, 16]
    conv_state: np.ndarray  # float32 [L, 4352, 4]
    ssm_state: np.ndarray   # float32 [L, 64, 64, 128]
    x: np.ndarray           # float32 [2048]: the first layer's input

    @property
    def L(self):
        return self.in_P.shape[0]

    def layer(self, l):
        """Layer l's Mamba-2 parameters as a Mamba2Layer."""
        return Mamba2Layer(self.conv_w[l], self.conv_b[l], self.dt_bias[l], self.A_log[l], self.D[l], self.norm_w[l])


def draw_decode_stack(rng: np.random.Generator, L: int) -> DecodeStack:
    """Per layer, in order: the in_proj weights (draw_problem at M = 1, K 2048 -> N 8512, no
    outliers; its x is discarded), the Mamba-2 parameters (draw_mamba2_layer), the layer's
    windows and state (draw_mamba2_inputs at one sequence; its zxbcdt is discarded), the
    out_proj weights (draw_problem, K 4096 -> N 2048); then the first layer's input
    x ~ N(0, 1)."""
    ins, mls, convs, ssms, outs = [], [], [], [], []
    for _ in range(L):
        ins.append(draw_problem(rng, 1, 8512, 2048, 0))
        mls.append(draw_mamba2_layer(rng))
        _, conv, ssm = draw_mamba2_inputs(rng, 1)
        convs.append(conv[0])
        ssms.append(ssm[0])
        outs.append(draw_problem(rng, 1, 2048, 4096, 0))
    x = rng.standard_normal(2048, dtype=np.float32)
    st = lambda items, name: np.ascontiguousarray(np.stack([getattr(i, name) for i in items]))  # noqa: E731
    return DecodeStack(st(ins, "P"), st(ins, "s_w"), st(ins, "W_A"), st(ins, "s_A"), st(ins, "W_B"), st(ins, "s_B"),
                       st(mls, "conv_w"), st(mls, "conv_b"), st(mls, "dt_bias"), st(mls, "A_log"), st(mls, "D"),
                       st(mls, "norm_w"), st(outs, "P"), st(outs, "s_w"), st(outs, "W_A"), st(outs, "s_A"),
                       st(outs, "W_B"), st(outs, "s_B"), np.ascontiguousarray(np.stack(convs)),
                       np.ascontiguousarray(np.stack(ssms)), x)

