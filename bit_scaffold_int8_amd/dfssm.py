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
EXPORTED = ("dfssm_status_string", "dfssm_version", "dfssm_quantize_act", "dfssm_lora_down",
            "dfssm_lora_down_strided_batched", "dfssm_quantize_lora_down",
            "dfssm_quantize_lora_down_strided_batched", "dfssm_scaffold_lora_gemm",
            "dfssm_scaffold_lora_gemm_strided_batched", "dfssm_scaffold_lora_gemm_given_t",
            "dfssm_scaffold_lora_gemm_given_t_strided_batched", "dfssm_scaffold_lora_forward",
            "dfssm_scaffold_lora_forward_strided_batched", "dfssm_int8_rowscale_gemm",
            "dfssm_int8_rowscale_gemm_strided_batched", "dfssm_embedding_lookup", "dfssm_mamba2_decode_step",
            "dfssm_prefill_plan", "dfssm_decode_layers_workspace_bytes", "dfssm_decode_layers_trace_words",
            "dfssm_decode_layers", "dfssm_decode_layers_noalloc", "dfssm_density_field_encode",
            "dfssm_density_field_decode", "dfssm_density_field_requantize")

DFSSM_DECODE_STATUS_TIMEOUT = 1
DFSSM_DECODE_STATUS_GAVE_UP = 2
DFSSM_DECODE_UNREACHABLE_WAITS = 1

# dfssm_decode_layer_weights: the stacked per-layer weights of dfssm_decode_layers
DECODE_WEIGHT_FIELDS = ("in_w_bits", "in_s_w", "in_w_a", "in_s_a", "in_w_b", "in_s_b", "conv_w", "conv_b",
                        "dt_bias", "A_log", "D", "norm_w", "out_w_bits", "out_s_w", "out_w_a", "out_s_a",
                        "out_w_b", "out_s_b")


class DecodeLayerWeights(ctypes.Structure):
    _fields_ = [(name, ctypes.c_void_p) for name in DECODE_WEIGHT_FIELDS]


class DfssmError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what} failed: {status_string(status)} ({status})")
        self.status = status


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python -m bit_scaffold_int8_amd.build`")
    # torch ships its own HIP runtime and loads it by path.  Loaded first, the library
    # would bring in the system's copy as well, and device pointers from torch would not
    # be valid in the library's runtime; with torch loaded first, the library's
    # dependency resolves to torch's runtime (same soname).
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    lib = ctypes.CDLL(LIB_PATH)
    P, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
    lib.dfssm_status_string.argtypes = [ctypes.c_int]
    lib.dfssm_status_string.restype = ctypes.c_char_p
    lib.dfssm_version.argtypes = []
    lib.dfssm_version.restype = i32
    lib.dfssm_decode_layers_workspace_bytes.argtypes = []
    lib.dfssm_decode_layers_workspace_bytes.restype = ctypes.c_size_t
    lib.dfssm_decode_layers_trace_words.argtypes = []
    lib.dfssm_decode_layers_trace_words.restype = i64
    sigs = {
        "dfssm_quantize_act": [P, i64, i64, P, P, P],
        "dfssm_lora_down": [P, i64, i64, P, i32, P, P],
        "dfssm_lora_down_strided_batched": [P, i64, i64, P, i32, P, i64, P],
        "dfssm_quantize_lora_down": [P, i64, i64, P, i32, P, P, P, P],
        "dfssm_quantize_lora_down_strided_batched": [P, i64, i64, P, i32, P, P, P, i64, P],
        "dfssm_scaffold_lora_gemm": [P, P, i64, i64, i64, P, P, P, P, P, P, i32, P, P, P, P],
        "dfssm_scaffold_lora_gemm_strided_batched": [P, P, i64, i64, i64, P, P, P, P, P, P, i32, P, P, P, i64, P],
        "dfssm_scaffold_lora_gemm_given_t": [P, P, i64, i64, i64, P, P, P, P, P, P, i32, P, P, P],
        "dfssm_scaffold_lora_gemm_given_t_strided_batched": [P, P, i64, i64, i64, P, P, P, P, P, P, i32, P, P, i64,
                                                             P],
        "dfssm_scaffold_lora_forward": [P, i64, i64, i64, P, P, P, P, P, P, i32, P, P, P, P, P, P],
        "dfssm_scaffold_lora_forward_strided_batched": [P, i64, i64, i64, P, P, P, P, P, P, i32, P, P, P, P, P,
                                                        i64, P],
        "dfssm_int8_rowscale_gemm": [P, P, i64, i64, i64, P, P, P, P, P],
        "dfssm_int8_rowscale_gemm_strided_batched": [P, P, i64, i64, i64, P, P, P, P, i64, P],
        "dfssm_embedding_lookup": [P, i64, P, P, i64, i64, P, P],
        "dfssm_mamba2_decode_step": [P, i64, i64, i64, i64, P, P, P, P, P, P, P, P, P, ctypes.c_float, P, P],
        "dfssm_prefill_plan": [i64, i64, i64, i64, P, P, P],
        "dfssm_decode_layers": [P, i64, P, P, P, P, P, ctypes.c_float, P, ctypes.c_size_t, P, P, i64, ctypes.c_uint32,
                                P],
        "dfssm_decode_layers_noalloc": [P, i64, P, P, P, P, P, ctypes.c_float, P, P, i64, ctypes.c_uint32, P],
        "dfssm_density_field_encode": [P, i64, i64, P, P, P],
        "dfssm_density_field_decode": [P, P, i64, i64, P, P],
        "dfssm_density_field_requantize": [P, i64, i64, P, P, P],
    }
    for name, argtypes in sigs.items():
        f = getattr(lib, name)
        f.argtypes = argtypes
        f.restype = ctypes.c_int
    return lib


lib = _load()


def status_string(status: int) -> str:
    return lib.dfssm_status_string(int(status)).decode()


def dfssm_version() -> int:
    return int(lib.dfssm_version())


def dfssm_prefill_plan(M: int, N: int, K: int, batch: int = 1):
    """(main configuration, tail configuration or -1, first tail column) the MFMA
    kernel's cost model picks for this shape; host only."""
    mc, tc, ns = ctypes.c_int32(0), ctypes.c_int32(0), ctypes.c_int64(0)
    _call("dfssm_prefill_plan", M, N, K, batch, ctypes.addressof(mc), ctypes.addressof(tc), ctypes.addressof(ns))
    return mc.value, tc.value, ns.value


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


def raw(name: str, *args) -> int:
    """Pointer-level call of any entry point; returns the status code unchanged."""
    return getattr(lib, name)(*args)


def _call(name, *args):
    st = getattr(lib, name)(*args)
    if st != DFSSM_OK:
        raise DfssmError(st, name)


def dfssm_quantize_act(x, x_q, s_x, stream=None) -> None:
    """x fp32 [M, K] -> x_q int8 [M, K], s_x fp32 [M]."""
    M, K = x.shape
    _call("dfssm_quantize_act", _ptr(x), M, K, _ptr(x_q), _ptr(s_x), _stream(stream))


def dfssm_lora_down(x_q, w_b, t, stream=None) -> None:
    """t int32 [M, 16] = W_B [16, K] x_q [M, K]^T."""
    M, K = x_q.shape
    _call("dfssm_lora_down", _ptr(x_q), M, K, _ptr(w_b), int(w_b.shape[0]), _ptr(t), _stream(stream))


def dfssm_lora_down_strided_batched(x_q, w_b, t, stream=None) -> None:
    """x_q [B, M, K], w_b [B, 16, K] -> t [B, M, 16]."""
    B, M, K = x_q.shape
    _call("dfssm_lora_down_strided_batched", _ptr(x_q), M, K, _ptr(w_b), int(w_b.shape[1]), _ptr(t), B,
          _stream(stream))


def dfssm_quantize_lora_down(x, w_b, x_q, s_x, t, stream=None) -> None:
    """x fp32 [M, K] -> x_q, s_x and (w_b given) t = W_B x_q; w_b = None for rank 0."""
    M, K = x.shape
    rank = 0 if w_b is None else int(w_b.shape[0])
    _call("dfssm_quantize_lora_down", _ptr(x), M, K, _ptr(w_b), rank, _ptr(x_q), _ptr(s_x), _ptr(t),
          _stream(stream))


def dfssm_quantize_lora_down_strided_batched(x, w_b, x_q, s_x, t, stream=None) -> None:
    """x [B, M, K], w_b [B, 16, K] -> x_q [B, M, K], s_x [B, M], t [B, M, 16]."""
    B, M, K = x.shape
    rank = 0 if w_b is None else int(w_b.shape[1])
    _call("dfssm_quantize_lora_down_strided_batched", _ptr(x), M, K, _ptr(w_b), rank, _ptr(x_q), _ptr(s_x),
          _ptr(t), B, _stream(stream))


def dfssm_scaffold_lora_gemm(x_q, s_x, w_bits, s_w, w_a, s_a, w_b, s_b, y, acc_dbg=None, t_dbg=None,
                             stream=None) -> None:
    """y fp32 [M, N] from x_q [M, K], s_x [M], w_bits [N, K/8], s_w [N] and the LoRA pair
    w_a [N, 16], s_a [N], w_b [16, K], s_b [16] (all None for rank 0); t = W_B x_q is
    computed by the kernel (t_dbg [M, 16], when given, receives it)."""
    M, K = x_q.shape
    N = w_bits.shape[0]
    rank = 0 if w_a is None else int(w_a.shape[1])
    _call("dfssm_scaffold_lora_gemm", _ptr(x_q), _ptr(s_x), M, N, K, _ptr(w_bits), _ptr(s_w), _ptr(w_a),
          _ptr(s_a), _ptr(w_b), _ptr(s_b), rank, _ptr(y), _ptr(acc_dbg), _ptr(t_dbg), _stream(stream))


def dfssm_scaffold_lora_gemm_strided_batched(x_q, s_x, w_bits, s_w, w_a, s_a, w_b, s_b, y, acc_dbg=None,
                                             t_dbg=None, stream=None) -> None:
    """Batched form: x_q [B, M, K], s_x [B, M], w_bits [B, N, K/8], s_w [B, N], w_a [B, N, 16],
    s_a [B, N], w_b [B, 16, K], s_b [B, 16], y [B, M, N], t_dbg [B, M, 16]."""
    B, M, K = x_q.shape
    N = w_bits.shape[1]
    rank = 0 if w_a is None else int(w_a.shape[2])
    _call("dfssm_scaffold_lora_gemm_strided_batched", _ptr(x_q), _ptr(s_x), M, N, K, _ptr(w_bits), _ptr(s_w),
          _ptr(w_a), _ptr(s_a), _ptr(w_b), _ptr(s_b), rank, _ptr(y), _ptr(acc_dbg), _ptr(t_dbg), B,
          _stream(stream))


def dfssm_scaffold_lora_gemm_given_t(x_q, s_x, w_bits, s_w, w_a, s_a, s_b, t, y, acc_dbg=None,
                                     stream=None) -> None:
    """The product with t [M, 16] given (from dfssm_lora_down / dfssm_quantize_lora_down):
    y fp32 [M, N] from x_q, s_x, w_bits, s_w and w_a, s_a, s_b, t (all None for rank 0)."""
    M, K = x_q.shape
    N = w_bits.shape[0]
    rank = 0 if w_a is None else int(w_a.shape[1])
    _call("dfssm_scaffold_lora_gemm_given_t", _ptr(x_q), _ptr(s_x), M, N, K, _ptr(w_bits), _ptr(s_w), _ptr(w_a),
          _ptr(s_a), _ptr(s_b), _ptr(t), rank, _ptr(y), _ptr(acc_dbg), _stream(stream))


def dfssm_scaffold_lora_gemm_given_t_strided_batched(x_q, s_x, w_bits, s_w, w_a, s_a, s_b, t, y, acc_dbg=None,
                                                     stream=None) -> None:
    """Batched form of dfssm_scaffold_lora_gemm_given_t: every operand with a leading [B]."""
    B, M, K = x_q.shape
    N = w_bits.shape[1]
    rank = 0 if w_a is None else int(w_a.shape[2])
    _call("dfssm_scaffold_lora_gemm_given_t_strided_batched", _ptr(x_q), _ptr(s_x), M, N, K, _ptr(w_bits),
          _ptr(s_w), _ptr(w_a), _ptr(s_a), _ptr(s_b), _ptr(t), rank, _ptr(y), _ptr(acc_dbg), B, _stream(stream))


def dfssm_scaffold_lora_forward(x, w_bits, s_w, w_a, s_a, w_b, s_b, x_q, s_x, t, y, acc_dbg=None,
                                stream=None) -> None:
    """The whole projection in one call: x fp32 [M, K] -> x_q, s_x, t and y [M, N]
    (LoRA operands all None for rank 0)."""
    M, K = x.shape
    N = w_bits.shape[0]
    rank = 0 if w_a is None else int(w_a.shape[1])
    _call("dfssm_scaffold_lora_forward", _ptr(x), M, N, K, _ptr(w_bits), _ptr(s_w), _ptr(w_a), _ptr(s_a),
          _ptr(w_b), _ptr(s_b), rank, _ptr(x_q), _ptr(s_x), _ptr(t), _ptr(y), _ptr(acc_dbg), _stream(stream))


def dfssm_scaffold_lora_forward_strided_batched(x, w_bits, s_w, w_a, s_a, w_b, s_b, x_q, s_x, t, y,
                                                acc_dbg=None, stream=None) -> None:
    """Batched form of dfssm_scaffold_lora_forward: every operand with a leading [B]."""
    B, M, K = x.shape
    N = w_bits.shape[1]
    rank = 0 if w_a is None else int(w_a.shape[2])
    _call("dfssm_scaffold_lora_forward_strided_batched", _ptr(x), M, N, K, _ptr(w_bits), _ptr(s_w), _ptr(w_a),
          _ptr(s_a), _ptr(w_b), _ptr(s_b), rank, _ptr(x_q), _ptr(s_x), _ptr(t), _ptr(y), _ptr(acc_dbg), B,
          _stream(stream))


def dfssm_int8_rowscale_gemm(x_q, s_x, e, s_e, y, acc_dbg=None, stream=None) -> None:
    """int8 LM head: y [M, N] = s_x (s_e (E x_q)) from x_q [M, K], s_x [M], e [N, K], s_e [N]."""
    M, K = x_q.shape
    N = e.shape[0]
    _call("dfssm_int8_rowscale_gemm", _ptr(x_q), _ptr(s_x), M, N, K, _ptr(e), _ptr(s_e), _ptr(y), _ptr(acc_dbg),
          _stream(stream))


def dfssm_int8_rowscale_gemm_strided_batched(x_q, s_x, e, s_e, y, acc_dbg=None, stream=None) -> None:
    """Batched form: x_q [B, M, K], s_x [B, M], e [B, N, K], s_e [B, N], y [B, M, N]."""
    B, M, K = x_q.shape
    N = e.shape[1]
    _call("dfssm_int8_rowscale_gemm_strided_batched", _ptr(x_q), _ptr(s_x), M, N, K, _ptr(e), _ptr(s_e), _ptr(y),
          _ptr(acc_dbg), B, _stream(stream))


def dfssm_embedding_lookup(tokens, e, s_e, out, stream=None) -> None:
    """out [T, K] = s_e[id] E[id] for the int32 ids `tokens` [T] (ids outside [0, V): zeros)."""
    T = tokens.shape[0]
    V, K = e.shape
    _call("dfssm_embedding_lookup", _ptr(tokens), T, _ptr(e), _ptr(s_e), V, K, _ptr(out), _stream(stream))


def dfssm_mamba2_decode_step(zxbcdt, conv_state_in, conv_state_out, ssm_state, conv_w, conv_b, dt_bias, A_log, D,
                             norm_w, eps, out, stream=None) -> None:
    """Mamba-2 step for S sequences: zxbcdt [S, 2 d_inner + 2 d_state + nheads] (in_proj
    output) -> out [S, d_inner] (out_proj input); conv_state_in -> conv_state_out
    [S, conv_dim, 4]; ssm_state [S, nheads, headdim, d_state] updated in place."""
    S = zxbcdt.shape[0]
    _, nheads, headdim, d_state = ssm_state.shape
    _call("dfssm_mamba2_decode_step", _ptr(zxbcdt), S, nheads, headdim, d_state, _ptr(conv_state_in),
          _ptr(conv_state_out), _ptr(ssm_state), _ptr(conv_w), _ptr(conv_b), _ptr(dt_bias), _ptr(A_log), _ptr(D),
          _ptr(norm_w), float(eps), _ptr(out), _stream(stream))


def dfssm_decode_layers_workspace_bytes() -> int:
    return int(lib.dfssm_decode_layers_workspace_bytes())


def dfssm_decode_layers_trace_words() -> int:
    return int(lib.dfssm_decode_layers_trace_words())


def dfssm_decode_layers(weights: dict, n_layers, x_in, x_out, conv_state_in, conv_state_out, ssm_state, eps,
                        workspace, status, trace=None, spin_limit: int = 0, flags: int = 0, stream=None) -> None:
    """The decode step of n_layers stacked layers for one sequence, one launch.  `weights`
    maps every name of DECODE_WEIGHT_FIELDS to a device tensor (stacked over layers);
    workspace is a zeroed device buffer of dfssm_decode_layers_workspace_bytes() bytes,
    status a device int32 the kernel ORs failure bits into."""
    w = DecodeLayerWeights(*[_ptr(weights[name]) for name in DECODE_WEIGHT_FIELDS])
    nbytes = workspace.numel() * workspace.element_size()
    _call("dfssm_decode_layers", ctypes.addressof(w), int(n_layers), _ptr(x_in), _ptr(x_out), _ptr(conv_state_in),
          _ptr(conv_state_out), _ptr(ssm_state), float(eps), _ptr(workspace), nbytes, _ptr(status), _ptr(trace),
          int(spin_limit), int(flags), _stream(stream))


def dfssm_decode_layers_noalloc(weights: dict, n_layers, x_in, x_out, conv_state_in, conv_state_out, ssm_state,
                                eps, status, trace=None, spin_limit: int = 0, flags: int = 0, stream=None) -> None:
    """dfssm_decode_layers with the library's own per-GPU array as the workspace: nothing
    is allocated; calls that overlap on one GPU race."""
    w = DecodeLayerWeights(*[_ptr(weights[name]) for name in DECODE_WEIGHT_FIELDS])
    _call("dfssm_decode_layers_noalloc", ctypes.addressof(w), int(n_layers), _ptr(x_in), _ptr(x_out),
          _ptr(conv_state_in), _ptr(conv_state_out), _ptr(ssm_state), float(eps), _ptr(status), _ptr(trace),
          int(spin_limit), int(flags), _stream(stream))


def dfssm_density_field_encode(state, field, scale, stream=None) -> None:
    """state fp32 [R, d] -> field uint32 [R, d / 8], scale fp32 [R] (density-field codec)."""
    R, d = state.shape
    _call("dfssm_density_field_encode", _ptr(state), R, d, _ptr(field), _ptr(scale), _stream(stream))


def dfssm_density_field_decode(field, scale, state, stream=None) -> None:
    """field uint32 [R, d / 8], scale fp32 [R] -> state fp32 [R, d] (popcount readout)."""
    R, d = state.shape
    _call("dfssm_density_field_decode", _ptr(field), _ptr(scale), R, d, _ptr(state), _stream(stream))


def dfssm_density_field_requantize(state, field=None, scale=None, stream=None) -> None:
    """The round trip in place: state [R, d] <- its field's readout (field, scale optional)."""
    R, d = state.shape
    _call("dfssm_density_field_requantize", _ptr(state), R, d, _ptr(field), _ptr(scale), _stream(stream))

