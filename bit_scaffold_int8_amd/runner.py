"""Device-side plumbing around the C ABI: copy one projection's operands to HBM once,
preallocate the outputs, and call the two entry points on a stream.

No arithmetic of the projection happens here; it only moves buffers and forwards
pointers to ``libdfssm.so`` through the ctypes binding.
"""
from __future__ import annotations

from dataclasses import dataclass

import torch

from . import dfssm


@dataclass
class DeviceProjection:
    """Resident operands + outputs of one projection (M tokens, K in, N out)."""
    x: torch.Tensor        # fp32 [M, K]
    w_bits: torch.Tensor   # uint8 [N, K/8]
    s_w: torch.Tensor      # fp32 [N]
    w_a: torch.Tensor | None
    s_a: torch.Tensor | None
    w_b: torch.Tensor | None
    s_b: torch.Tensor | None
    x_q: torch.Tensor      # int8 [M, K]   (out)
    s_x: torch.Tensor      # fp32 [M]      (out)
    y: torch.Tensor        # fp32 [M, N]   (out)
    t: torch.Tensor | None  # int32 [M, 16] (out)
    acc_dbg: torch.Tensor | None

    @property
    def M(self):
        return self.x.shape[0]

    @property
    def K(self):
        return self.x.shape[1]

    @property
    def N(self):
        return self.w_bits.shape[0]

    @classmethod
    def from_host(cls, x, P, s_w, W_A=None, s_A=None, W_B=None, s_B=None, device="cuda:0",
                  with_acc: bool = False) -> "DeviceProjection":
        def dev(a):
            return None if a is None else torch.from_numpy(a).to(device).contiguous()
        M, K = x.shape
        N = P.shape[0]
        rank = 0 if W_A is None else W_B.shape[0]
        return cls(
            x=dev(x), w_bits=dev(P), s_w=dev(s_w), w_a=dev(W_A), s_a=dev(s_A), w_b=dev(W_B), s_b=dev(s_B),
            x_q=torch.empty((M, K), dtype=torch.int8, device=device),
            s_x=torch.empty((M,), dtype=torch.float32, device=device),
            y=torch.empty((M, N), dtype=torch.float32, device=device),
            t=torch.empty((M, rank), dtype=torch.int32, device=device) if rank else None,
            acc_dbg=torch.empty((M, N), dtype=torch.int32, device=device) if with_acc else None,
        )

    def quantize(self, stream=None):
        dfssm.dfssm_quantize_act(self.x, self.x_q, self.s_x, stream)

    def gemm(self, stream=None, debug: bool = True):
        dfssm.dfssm_scaffold_lora_gemm(self.x_q, self.s_x, self.w_bits, self.s_w, self.w_a, self.s_a,
                                       self.w_b, self.s_b, self.y, self.t,
                                       self.acc_dbg if debug else None, stream)

    def forward(self, stream=None, debug: bool = True):
        self.quantize(stream)
        self.gemm(stream, debug)
