"""ctypes binding of libdfssm.so (include/dfssm.h) -- argument marshalling only.

Every function here has the C entry point's name and forwards raw device pointers,
sizes and the current HIP stream; all arithmetic happens in the HIP kernels.  If
the shared library is missing the import fails loudly: there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libdfssm.so")

DFSSM_OK = 0
DFSSM_ERR_INVALID_ARG = 1
DFSSM_ERR_UNSUPPORTED = 2
DFSSM_ERR_HIP = 3

# every symbol include/dfssm.h declares
EXPORTED = ("dfssm_status_string", "dfssm_version", "dfssm_quantize_act", "dfssm_scaffold_lora_gemm")


class DfssmError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what} failed: {status_string(status)} ({status})")
        self.status = status


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python -m bit_scaffold_int8_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    P, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
    lib.dfssm_status_string.argtypes = [ctypes.c_int]
    lib.dfssm_status_string.restype = ctypes.c_char_p
    lib.dfssm_version.argtypes = []
    lib.dfssm_version.restype = i32
    lib.dfssm_quantize_act.argtypes = [P, i64, i64, P, P, P]
    lib.dfssm_quantize_act.restype = ctypes.c_int
    lib.dfssm_scaffold_lora_gemm.argtypes = [P, P, i64, i64, i64, P, P, P, P, P, P, i32, P, P, P, P]
    lib.dfssm_scaffold_lora_gemm.restype = ctypes.c_int
    return lib


lib = _load()


def status_string(status: int) -> str:
    return lib.dfssm_status_string(int(status)).decode()


def dfssm_version() -> int:
    return int(lib.dfssm_version())


def _ptr(t):
    """Device pointer of a tensor, an int address, or None (NULL)."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def raw_quantize_act(x, M, K, x_q, s_x, stream) -> int:
    """Pointer-level call; returns the status code unchanged."""
    return lib.dfssm_quantize_act(x, M, K, x_q, s_x, stream)


def raw_scaffold_lora_gemm(x_q, s_x, M, N, K, w_bits, s_w, w_a, s_a, w_b, s_b, rank, y, t, acc_dbg,
                           stream) -> int:
    """Pointer-level call; returns the status code unchanged."""
    return lib.dfssm_scaffold_lora_gemm(x_q, s_x, M, N, K, w_bits, s_w, w_a, s_a, w_b, s_b, rank,
                                        y, t, acc_dbg, stream)


def dfssm_quantize_act(x, x_q, s_x, stream=None) -> None:
    """x fp32 [M, K] -> x_q int8 [M, K], s_x fp32 [M] (device tensors)."""
    M, K = x.shape
    st = lib.dfssm_quantize_act(_ptr(x), M, K, _ptr(x_q), _ptr(s_x), _stream(stream))
    if st != DFSSM_OK:
        raise DfssmError(st, "dfssm_quantize_act")


def dfssm_scaffold_lora_gemm(x_q, s_x, w_bits, s_w, w_a, s_a, w_b, s_b, y, t=None, acc_dbg=None,
                             stream=None) -> None:
    """y = s_x (s_w (W x_q) + s_A W_A (s_B W_B x_q)); shapes are read from x_q [M, K] and
    w_bits [N, K/8]; pass w_a = None for rank 0."""
    M, K = x_q.shape
    N = w_bits.shape[0]
    rank = 0 if w_a is None else int(w_b.shape[0])
    st = lib.dfssm_scaffold_lora_gemm(_ptr(x_q), _ptr(s_x), M, N, K, _ptr(w_bits), _ptr(s_w),
                                      _ptr(w_a), _ptr(s_a), _ptr(w_b), _ptr(s_b), rank,
                                      _ptr(y), _ptr(t), _ptr(acc_dbg), _stream(stream))
    if st != DFSSM_OK:
        raise DfssmError(st, "dfssm_scaffold_lora_gemm")
