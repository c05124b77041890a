"""CPU oracle for the DF-SSM scaffold projection -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product path (``bit_scaffold_int8_amd``)
never imports it, and it never imports the product path.

The arithmetic lives in ``dfssm_oracle.c`` (plain scalar C, fp64 epilogue,
built without FMA contraction or fast-math); this module only marshals numpy
arrays into it through ctypes.  What it computes follows the DF-SSM technical
summary (gist.science), section 2B "Frozen Scaffold with LoRA Correction"
(int8 rank-16 LoRA, W_A d_out x r, W_B r x d_in, per-channel/row scales) and
section 2C "Optimized Inference Pipeline" (1-bit packed weights expanded to
int8 for an int8 x int8 product), and the int8 embedding / LM head with per-row
scales (the summary's quantization and model-composition notes); the numeric
conventions the pages leave open
(absmax/127 scale, round half to even, LSB-first sign packing with bit 1 = +1,
per-output-channel scaffold scale, fp32 output) are written at the top of the
C file.

Parity status: every function here is pinned by ``tests/test_oracle_pins.py``
(fp64 BLAS brute force, numpy's bit unpacking, a hand-worked example under
``tests/golden/``, exhaustive K=8, and algebraic invariants).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "dfssm_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

OK, ERR_ARG, ERR_OVERFLOW = 0, 1, 2

_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc into ``oracle/liboracle.so``."""
    if not force and os.path.exists(_LIB) and os.path.getmtime(_LIB) >= os.path.getmtime(_SRC):
        return _LIB
    cmd = ["gcc", "-O1", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
           "-fno-fast-math", "-frounding-math", "-fopenmp", _SRC, "-o", _LIB + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(_LIB + ".tmp", _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        build()
    lib = ctypes.CDLL(_LIB)
    P = ctypes.c_void_p
    i64, i32 = ctypes.c_int64, ctypes.c_int32
    lib.oracle_quantize_act.argtypes = [P, i64, i64, P, P]
    lib.oracle_scaffold_acc.argtypes = [P, i64, i64, i64, P, P]
    lib.oracle_lora_down.argtypes = [P, i64, i64, P, i32, P]
    lib.oracle_scaffold_lora_gemm.argtypes = [P, P, i64, i64, i64, P, P, P, P, P, P, i32, P, P, P, i32]
    lib.oracle_scaffold_lora_at.argtypes = [P, P, i64, i64, i64, P, P, P, P, P, P, i32, P, P, i64, P, P, P]
    lib.oracle_int8_rowscale_gemm.argtypes = [P, P, i64, i64, i64, P, P, P, P, i32]
    lib.oracle_embedding_lookup.argtypes = [P, i64, P, P, i64, i64, P]
    for f in (lib.oracle_quantize_act, lib.oracle_scaffold_acc, lib.oracle_lora_down,
              lib.oracle_scaffold_lora_gemm, lib.oracle_scaffold_lora_at, lib.oracle_int8_rowscale_gemm,
              lib.oracle_embedding_lookup):
        f.restype = ctypes.c_int
    _lib = lib
    return lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def _check(status, what):
    if status != OK:
        raise RuntimeError(f"oracle {what} failed with status {status}")


def quantize_act(x):
    """Per-token absmax int8 quantization. Returns (x_q int8 [M,K], s_x float32 [M])."""
    x = _c(x, np.float32)
    M, K = x.shape
    x_q = np.empty((M, K), np.int8)
    s_x = np.empty((M,), np.float32)
    _check(_load().oracle_quantize_act(_ptr(x), M, K, _ptr(x_q), _ptr(s_x)), "quantize_act")
    return x_q, s_x


def scaffold_acc(x_q, w_bits):
    """Exact int32 scaffold accumulators acc[m, n] = sum_k w[n, k] x_q[m, k]."""
    x_q = _c(x_q, np.int8)
    w_bits = _c(w_bits, np.uint8)
    M, K = x_q.shape
    N = w_bits.shape[0]
    assert w_bits.shape == (N, K // 8)
    acc = np.empty((M, N), np.int32)
    _check(_load().oracle_scaffold_acc(_ptr(x_q), M, N, K, _ptr(w_bits), _ptr(acc)), "scaffold_acc")
    return acc


def lora_down(x_q, w_b):
    """Exact int32 LoRA down-projection t[m, r] = sum_k W_B[r, k] x_q[m, k]."""
    x_q = _c(x_q, np.int8)
    w_b = _c(w_b, np.int8)
    M, K = x_q.shape
    rank = w_b.shape[0]
    t = np.empty((M, rank), np.int32)
    _check(_load().oracle_lora_down(_ptr(x_q), M, K, _ptr(w_b), rank, _ptr(t)), "lora_down")
    return t


def scaffold_lora_gemm(x_q, s_x, w_bits, s_w, w_a, s_a, w_b, s_b, nthreads: int = 1):
    """Full projection. Returns (y float32 [M,N], acc int32 [M,N], t int32 [M,rank])."""
    x_q = _c(x_q, np.int8)
    s_x = _c(s_x, np.float32)
    w_bits = _c(w_bits, np.uint8)
    s_w = _c(s_w, np.float32)
    M, K = x_q.shape
    N = w_bits.shape[0]
    assert w_bits.shape == (N, K // 8) and s_w.shape == (N,) and s_x.shape == (M,)
    if w_a is None:
        rank = 0
        w_a = s_a = w_b = s_b = None
    else:
        w_a, s_a = _c(w_a, np.int8), _c(s_a, np.float32)
        w_b, s_b = _c(w_b, np.int8), _c(s_b, np.float32)
        rank = w_b.shape[0]
        assert w_a.shape == (N, rank) and w_b.shape == (rank, K)
        assert s_a.shape == (N,) and s_b.shape == (rank,)
    y = np.empty((M, N), np.float32)
    acc = np.empty((M, N), np.int32)
    t = np.empty((M, max(rank, 1)), np.int32)[:, :rank]
    t = np.ascontiguousarray(t)
    st = _load().oracle_scaffold_lora_gemm(
        _ptr(x_q), _ptr(s_x), M, N, K, _ptr(w_bits), _ptr(s_w), _ptr(w_a), _ptr(s_a),
        _ptr(w_b), _ptr(s_b), rank, _ptr(y), _ptr(acc), _ptr(t) if rank else None, int(nthreads))
    _check(st, "scaffold_lora_gemm")
    return y, acc, t


def scaffold_lora_at(x_q, s_x, w_bits, s_w, w_a, s_a, w_b, s_b, m_idx, n_idx):
    """The projection at sampled positions. Returns (y [c], acc [c], t [c, rank])."""
    x_q = _c(x_q, np.int8)
    s_x = _c(s_x, np.float32)
    w_bits = _c(w_bits, np.uint8)
    s_w = _c(s_w, np.float32)
    M, K = x_q.shape
    N = w_bits.shape[0]
    m_idx = _c(m_idx, np.int64)
    n_idx = _c(n_idx, np.int64)
    c = m_idx.shape[0]
    if w_a is None:
        rank = 0
        w_a = s_a = w_b = s_b = None
    else:
        w_a, s_a = _c(w_a, np.int8), _c(s_a, np.float32)
        w_b, s_b = _c(w_b, np.int8), _c(s_b, np.float32)
        rank = w_b.shape[0]
    y = np.empty((c,), np.float32)
    acc = np.empty((c,), np.int32)
    t = np.empty((c, max(rank, 1)), np.int32)
    st = _load().oracle_scaffold_lora_at(
        _ptr(x_q), _ptr(s_x), M, N, K, _ptr(w_bits), _ptr(s_w), _ptr(w_a), _ptr(s_a),
        _ptr(w_b), _ptr(s_b), rank, _ptr(m_idx), _ptr(n_idx), c, _ptr(y), _ptr(acc),
        _ptr(t) if rank else None)
    _check(st, "scaffold_lora_at")
    return y, acc, t[:, :rank]


def int8_rowscale_gemm(x_q, s_x, e, s_e, nthreads: int = 1):
    """int8 LM head: acc[m, n] = sum_k E[n, k] x_q[m, k] (exact int32) and
    y[m, n] = s_x[m] (s_e[n] acc[m, n]) (fp64, rounded once).  Returns (y, acc)."""
    x_q = _c(x_q, np.int8)
    s_x = _c(s_x, np.float32)
    e = _c(e, np.int8)
    s_e = _c(s_e, np.float32)
    M, K = x_q.shape
    N = e.shape[0]
    assert e.shape == (N, K) and s_e.shape == (N,) and s_x.shape == (M,)
    y = np.empty((M, N), np.float32)
    acc = np.empty((M, N), np.int32)
    _check(_load().oracle_int8_rowscale_gemm(_ptr(x_q), _ptr(s_x), M, N, K, _ptr(e), _ptr(s_e), _ptr(y),
                                              _ptr(acc), int(nthreads)), "int8_rowscale_gemm")
    return y, acc


def embedding_lookup(tokens, e, s_e):
    """Rows of the int8 embedding, dequantized: out[t, k] = s_e[id] E[id, k] (fp32);
    ids outside [0, V) give zeros."""
    tokens = _c(tokens, np.int32)
    e = _c(e, np.int8)
    s_e = _c(s_e, np.float32)
    V, K = e.shape
    T = tokens.shape[0]
    out = np.empty((T, K), np.float32)
    _check(_load().oracle_embedding_lookup(_ptr(tokens), T, _ptr(e), _ptr(s_e), V, K, _ptr(out)),
           "embedding_lookup")
    return out
