"""Device-side plumbing around the C ABI: copy projections' operands to HBM once,
preallocate the outputs, and call the entry points on a stream.

No arithmetic of the projection happens here; it only moves buffers and forwards
pointers to ``libdfssm.so`` through the ctypes binding.  A ``DeviceProjections``
holds B independent problems of one shape (B = 1 for a single projection) laid
out densely, as the strided-batched entry points expect.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np
import torch

from . import dfssm


@dataclass
class DeviceProjections:
    x: torch.Tensor         # fp32  [B, M, K]
    w_bits: torch.Tensor    # uint8 [B, N, K/8]
    s_w: torch.Tensor       # fp32  [B, N]
    w_a: torch.Tensor | None   # int8 [B, N, 16]
    s_a: torch.Tensor | None   # fp32 [B, N]
    w_b: torch.Tensor | None   # int8 [B, 16, K]
    s_b: torch.Tensor | None   # fp32 [B, 16]
    x_q: torch.Tensor       # int8  [B, M, K]   (out)
    s_x: torch.Tensor       # fp32  [B, M]      (out)
    t: torch.Tensor | None  # int32 [B, M, 16]  (out)
    y: torch.Tensor         # fp32  [B, M, N]   (out)
    acc_dbg: torch.Tensor | None

    @property
    def B(self):
        return self.x.shape[0]

    @property
    def M(self):
        return self.x.shape[1]

    @property
    def K(self):
        return self.x.shape[2]

    @property
    def N(self):
        return self.w_bits.shape[1]

    @property
    def rank(self):
        return 0 if self.w_a is None else self.w_a.shape[2]

    @classmethod
    def from_problems(cls, problems, device="cuda:0", rank: bool = True, with_acc: bool = False):
        """Stack host problems (objects with x, P, s_w, W_A, s_A, W_B, s_B) onto the device."""
        def dev(name):
            return torch.from_numpy(np.stack([getattr(p, name) for p in problems])).to(device).contiguous()
        B = len(problems)
        M, K = problems[0].x.shape
        N = problems[0].P.shape[0]
        return cls(
            x=dev("x"), w_bits=dev("P"), s_w=dev("s_w"),
            w_a=dev("W_A") if rank else None, s_a=dev("s_A") if rank else None,
            w_b=dev("W_B") if rank else None, s_b=dev("s_B") if rank else None,
            x_q=torch.empty((B, M, K), dtype=torch.int8, device=device),
            s_x=torch.empty((B, M), dtype=torch.float32, device=device),
            t=torch.empty((B, M, 16), dtype=torch.int32, device=device) if rank else None,
            y=torch.empty((B, M, N), dtype=torch.float32, device=device),
            acc_dbg=torch.empty((B, M, N), dtype=torch.int32, device=device) if with_acc else None,
        )

    # ---- the two launches of a forward step
    def quantize_lora_down(self, stream=None):
        dfssm.dfssm_quantize_lora_down_strided_batched(self.x, self.w_b, self.x_q, self.s_x, self.t, stream)

    def gemm(self, stream=None, debug: bool = True):
        """The product with t given (dfssm_scaffold_lora_gemm_given_t, after quantize_lora_down)."""
        dfssm.dfssm_scaffold_lora_gemm_given_t_strided_batched(
            self.x_q, self.s_x, self.w_bits, self.s_w, self.w_a, self.s_a, self.s_b, self.t, self.y,
            self.acc_dbg if debug else None, stream)

    def forward(self, stream=None, debug: bool = True):
        self.quantize_lora_down(stream)
        self.gemm(stream, debug)

    # ---- the specified two-call form: quantize, then the product computing t itself
    def quantize(self, stream=None):
        B, M, K = self.x.shape
        dfssm.dfssm_quantize_act(self.x.view(B * M, K), self.x_q.view(B * M, K), self.s_x.view(B * M), stream)

    def gemm_computing_t(self, stream=None, debug: bool = True):
        """dfssm_scaffold_lora_gemm: t = W_B x_q inside the kernel (written to self.t when
        debug and rank 16)."""
        dfssm.dfssm_scaffold_lora_gemm_strided_batched(
            self.x_q, self.s_x, self.w_bits, self.s_w, self.w_a, self.s_a, self.w_b, self.s_b, self.y,
            self.acc_dbg if debug else None, self.t if debug else None, stream)

    def forward_contract(self, stream=None, debug: bool = True):
        self.quantize(stream)
        self.gemm_computing_t(stream, debug)

    # ---- the one-call form (one launch at decode shapes)
    def forward_one_call(self, stream=None, debug: bool = True):
        dfssm.dfssm_scaffold_lora_forward_strided_batched(
            self.x, self.w_bits, self.s_w, self.w_a, self.s_a, self.w_b, self.s_b, self.x_q, self.s_x, self.t,
            self.y, self.acc_dbg if debug else None, stream)

    # ---- the unfused entry points, problem by problem (single-problem API)
    def forward_unfused(self, stream=None, debug: bool = True):
        for b in range(self.B):
            dfssm.dfssm_quantize_act(self.x[b], self.x_q[b], self.s_x[b], stream)
            if self.rank:
                dfssm.dfssm_lora_down(self.x_q[b], self.w_b[b], self.t[b], stream)
            dfssm.dfssm_scaffold_lora_gemm_given_t(
                self.x_q[b], self.s_x[b], self.w_bits[b], self.s_w[b],
                None if not self.rank else self.w_a[b], None if not self.rank else self.s_a[b],
                None if not self.rank else self.s_b[b], None if not self.rank else self.t[b], self.y[b],
                None if (self.acc_dbg is None or not debug) else self.acc_dbg[b], stream)

    def forward_contract_unfused(self, stream=None, debug: bool = True):
        """Problem by problem through the single-problem entry points of the specified
        form: dfssm_quantize_act, then dfssm_scaffold_lora_gemm (t computed inside)."""
        for b in range(self.B):
            dfssm.dfssm_quantize_act(self.x[b], self.x_q[b], self.s_x[b], stream)
            dfssm.dfssm_scaffold_lora_gemm(
                self.x_q[b], self.s_x[b], self.w_bits[b], self.s_w[b],
                None if not self.rank else self.w_a[b], None if not self.rank else self.s_a[b],
                None if not self.rank else self.w_b[b], None if not self.rank else self.s_b[b], self.y[b],
                None if (self.acc_dbg is None or not debug) else self.acc_dbg[b],
                None if (not self.rank or not debug) else self.t[b], stream)


@dataclass
class DeviceMamba2Layer:
    """One layer's Mamba-2 step operands on the device, for S sequences: parameters,
    the two convolution-window buffers (the step reads one and writes the other), the
    SSM state (updated in place) and the out_proj input it writes."""
    conv_w: torch.Tensor      # fp32 [conv_dim, 4]
    conv_b: torch.Tensor      # fp32 [conv_dim]
    dt_bias: torch.Tensor     # fp32 [nheads]
    A_log: torch.Tensor       # fp32 [nheads]
    D: torch.Tensor           # fp32 [nheads]
    norm_w: torch.Tensor      # fp32 [d_inner]
    windows: list             # two fp32 [S, conv_dim, 4]
    ssm_state: torch.Tensor   # fp32 [S, nheads, headdim, d_state]
    out: torch.Tensor         # fp32 [S, d_inner]
    eps: float = 1e-5

    @classmethod
    def from_host(cls, layer, conv_state, ssm_state, device="cuda:0", eps: float = 1e-5):
        """`layer` holds conv_w, conv_b, dt_bias, A_log, D, norm_w (numpy); conv_state
        [S, conv_dim, 4] and ssm_state [S, nheads, headdim, d_state] the starting state."""
        def dev(a):
            return torch.from_numpy(np.ascontiguousarray(a)).to(device)
        S, nheads, headdim, _ = ssm_state.shape
        w0 = dev(conv_state)
        return cls(conv_w=dev(layer.conv_w), conv_b=dev(layer.conv_b), dt_bias=dev(layer.dt_bias),
                   A_log=dev(layer.A_log), D=dev(layer.D), norm_w=dev(layer.norm_w),
                   windows=[w0, torch.empty_like(w0)], ssm_state=dev(ssm_state),
                   out=torch.empty((S, nheads * headdim), dtype=torch.float32, device=device), eps=eps)

    def step(self, zxbcdt, parity: int = 0, stream=None):
        """One token: windows[parity] -> windows[1 - parity], state in place, out written."""
        dfssm.dfssm_mamba2_decode_step(zxbcdt, self.windows[parity], self.windows[1 - parity], self.ssm_state,
                                       self.conv_w, self.conv_b, self.dt_bias, self.A_log, self.D, self.norm_w,
                                       self.eps, self.out, stream)


# host array name in a DecodeStack -> weight field of the persistent decode entry point
DECODE_HOST_NAMES = {
    "in_w_bits": "in_P", "in_s_w": "in_s_w", "in_w_a": "in_W_A", "in_s_a": "in_s_A", "in_w_b": "in_W_B",
    "in_s_b": "in_s_B", "conv_w": "conv_w", "conv_b": "conv_b", "dt_bias": "dt_bias", "A_log": "A_log", "D": "D",
    "norm_w": "norm_w", "out_w_bits": "out_P", "out_s_w": "out_s_w", "out_w_a": "out_W_A", "out_s_a": "out_s_A",
    "out_w_b": "out_W_B", "out_s_b": "out_s_B",
}


class DeviceDecodeStack:
    """A stack of layers on the device for dfssm_decode_layers: the stacked weights, the
    two window buffers (a token reads one and writes the other), the SSM state (updated
    in place), the exchange workspace (zeroed once here, then left to the library: it
    holds a call counter and the tagged exchange slots) and the status word."""

    def __init__(self, stack, device="cuda:0", eps: float = 1e-5):
        def dev(a):
            return torch.from_numpy(np.ascontiguousarray(a)).to(device)
        self.L = stack.L
        self.weights = {k: dev(getattr(stack, v)) for k, v in DECODE_HOST_NAMES.items()}
        w0 = dev(stack.conv_state)
        self.windows = [w0, torch.empty_like(w0)]
        self.ssm_state = dev(stack.ssm_state)
        self.eps = eps
        nbytes = dfssm.dfssm_decode_layers_workspace_bytes()
        self.workspace = torch.zeros((nbytes + 3) // 4, dtype=torch.int32, device=device)
        self.status = torch.zeros(1, dtype=torch.int32, device=device)
        self.trace_words = dfssm.dfssm_decode_layers_trace_words()

    def new_trace(self):
        return torch.zeros((self.L, self.trace_words), dtype=torch.int32, device=self.ssm_state.device)

    def step(self, x_in, x_out, parity: int = 0, trace=None, spin_limit: int = 0, flags: int = 0, stream=None):
        """One token through every layer: windows[parity] -> windows[1 - parity]."""
        dfssm.dfssm_decode_layers(self.weights, self.L, x_in, x_out, self.windows[parity], self.windows[1 - parity],
                                  self.ssm_state, self.eps, self.workspace, self.status, trace, spin_limit, flags,
                                  stream)

