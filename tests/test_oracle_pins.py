"""Pins for the CPU oracle: checks against what the mathematics fixes, not against itself.

Each test would fail on a plausible slip in the oracle: wrong bit order or sign
mapping (numpy unpackbits + fp64 BLAS, exhaustive K=8, hand-worked example),
wrong rounding (half-even hand cases, nearest-integer property), a dropped or
misplaced scale, a transposed LoRA operand (dequantized fp64 brute force on
non-square shapes), or a broken epilogue (invariants).
"""
import json
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand_case(rng, M, N, K, rank=16, outliers=2):
    P = rng.integers(0, 256, (N, K // 8), dtype=np.uint8)
    s_w = rng.uniform(0.01, 0.05, N).astype(np.float32)
    x = rng.standard_normal((M, K), dtype=np.float32)
    if outliers:
        x[:, rng.choice(K, outliers, replace=False)] *= np.float32(20)
    W_A = rng.integers(-127, 128, (N, rank), dtype=np.int8)
    s_A = rng.uniform(1e-4, 1e-3, N).astype(np.float32)
    W_B = rng.integers(-127, 128, (rank, K), dtype=np.int8)
    s_B = rng.uniform(1e-4, 1e-3, rank).astype(np.float32)
    return x, P, s_w, W_A, s_A, W_B, s_B


def _signs(P, K):
    """+-1 matrix [N, K] from numpy's own little-endian bit unpacking."""
    bits = np.unpackbits(P, axis=1, bitorder="little")[:, :K]
    return 2.0 * bits.astype(np.float64) - 1.0


# ---------------------------------------------------------------- hand-worked example

def test_hand_worked_example():
    g = json.load(open(os.path.join(GOLDEN, "hand_worked_example.json")))
    x = np.array(g["x"], np.float32)
    x_q, s_x = oracle.quantize_act(x)
    assert s_x.tolist() == g["expect_s_x"]
    assert x_q.tolist() == g["expect_x_q"]
    K, N, r = g["K"], g["N"], g["rank"]
    P = np.array(g["w_bits"], np.uint8)
    W_B = np.zeros((r, K), np.int8)
    for rr, k, v in g["w_b_nonzero"]:
        W_B[rr, k] = v
    y, acc, t = oracle.scaffold_lora_gemm(
        x_q, s_x, P, np.array(g["s_w"], np.float32), np.array(g["w_a"], np.int8),
        np.array(g["s_a"], np.float32), W_B, np.array(g["s_b"], np.float32))
    assert acc.tolist() == g["expect_acc"]
    assert t[:, :2].tolist() == g["expect_t_first2"]
    assert not t[:, 2:].any()
    assert y.tolist() == g["expect_y"]


# ---------------------------------------------------------------- packing and accumulators

def test_acc_matches_numpy_unpackbits_and_fp64_blas():
    rng = np.random.default_rng(11)
    for (M, N, K) in [(3, 37, 200), (1, 5, 8), (5, 64, 1024)]:
        x, P, *_ = _rand_case(rng, M, N, K)
        x_q, _ = oracle.quantize_act(x)
        acc = oracle.scaffold_acc(x_q, P)
        # every partial sum is an integer far below 2^53: fp64 BLAS is exact in any order
        ref = x_q.astype(np.float64) @ _signs(P, K).T
        assert np.array_equal(acc.astype(np.float64), ref)


def test_k8_exhaustive_all_256_bytes():
    rng = np.random.default_rng(12)
    P = np.arange(256, dtype=np.uint8).reshape(256, 1)
    x_q = rng.integers(-127, 128, (2, 8), dtype=np.int8)
    acc = oracle.scaffold_acc(x_q, P)
    for m in range(2):
        for b in range(256):
            want = sum((1 if (b >> i) & 1 else -1) * int(x_q[m, i]) for i in range(8))
            assert acc[m, b] == want


def test_lora_down_matches_fp64_blas():
    rng = np.random.default_rng(13)
    x_q = rng.integers(-127, 128, (4, 520), dtype=np.int8)
    W_B = rng.integers(-127, 128, (16, 520), dtype=np.int8)
    t = oracle.lora_down(x_q, W_B)
    assert np.array_equal(t.astype(np.float64), x_q.astype(np.float64) @ W_B.astype(np.float64).T)


def test_extreme_accumulators_fit_int32():
    K = 4096
    x_q = np.full((1, K), 127, np.int8)
    P = np.full((2, K // 8), 0xFF, np.uint8)
    P[1] = 0
    assert oracle.scaffold_acc(x_q, P).tolist() == [[127 * K, -127 * K]]
    x_q2 = np.full((1, K), -127, np.int8)
    W_B = np.full((16, K), -127, np.int8)
    assert (oracle.lora_down(x_q2, W_B) == 127 * 127 * K).all()


# ---------------------------------------------------------------- quantizer

def test_quantizer_half_even_special_cases():
    # absmax 127 -> scale exactly 1, so x/s is x itself
    x = np.array([[127, 2.5, 3.5, -2.5, 0.5, -0.5, 1.5, -1.5, 126.5, -3.5]], np.float32)
    x_q, s_x = oracle.quantize_act(x)
    assert s_x[0] == 1.0
    assert x_q.tolist() == [[127, 2, 4, -2, 0, 0, 2, -2, 126, -4]]


def test_quantizer_properties():
    rng = np.random.default_rng(14)
    x = rng.standard_normal((16, 777), dtype=np.float32)
    x[:, :3] *= 20
    x[5] = 0.0
    x_q, s_x = oracle.quantize_act(x)
    assert s_x[5] == 0.0 and not x_q[5].any()
    live = np.arange(16) != 5
    amax = np.abs(x[live]).max(axis=1)
    assert np.array_equal(s_x[live], amax / np.float32(127))  # one IEEE fp32 division
    assert np.abs(x_q).max() <= 127
    # the absmax element lands on +-127 exactly
    arg = np.abs(x[live]).argmax(axis=1)
    assert (np.abs(x_q[live][np.arange(live.sum()), arg]) == 127).all()
    # nearest integer to the fp32 quotient, ties to even
    v = (x[live] / s_x[live, None]).astype(np.float64)
    d = np.abs(v - x_q[live])
    assert (d <= 0.5).all()
    ties = d == 0.5
    assert (x_q[live][ties] % 2 == 0).all()


def test_quantizer_power_of_two_scaling():
    rng = np.random.default_rng(15)
    x = rng.standard_normal((4, 300), dtype=np.float32)
    q0, s0 = oracle.quantize_act(x)
    for j in (-3, 1, 5):
        q, s = oracle.quantize_act(x * np.float32(2.0 ** j))
        assert np.array_equal(q, q0)
        assert np.array_equal(s, s0 * np.float32(2.0 ** j))


# ---------------------------------------------------------------- full projection

def _dequantized_fp64(x_q, s_x, P, s_w, W_A, s_A, W_B, s_B):
    """Y = (s_x . X_q)(diag(s_w) W)^T + (s_x . X_q)(diag(s_B) W_B)^T (diag(s_A) W_A)^T in fp64."""
    K = x_q.shape[1]
    X = s_x.astype(np.float64)[:, None] * x_q.astype(np.float64)
    W = s_w.astype(np.float64)[:, None] * _signs(P, K)
    B = s_B.astype(np.float64)[:, None] * W_B.astype(np.float64)
    A = s_A.astype(np.float64)[:, None] * W_A.astype(np.float64)
    scaffold = X @ W.T
    lora = (X @ B.T) @ A.T
    mag = np.abs(X) @ np.abs(W).T + (np.abs(X) @ np.abs(B).T) @ np.abs(A).T
    return scaffold + lora, mag


@pytest.mark.parametrize("M,N,K", [(1, 40, 64), (3, 24, 136), (7, 33, 512)])
def test_y_matches_dequantized_fp64_brute_force(M, N, K):
    rng = np.random.default_rng(100 + M)
    x, P, s_w, W_A, s_A, W_B, s_B = _rand_case(rng, M, N, K)
    x_q, s_x = oracle.quantize_act(x)
    y, acc, t = oracle.scaffold_lora_gemm(x_q, s_x, P, s_w, W_A, s_A, W_B, s_B)
    Y, mag = _dequantized_fp64(x_q, s_x, P, s_w, W_A, s_A, W_B, s_B)
    ulp = np.spacing(np.abs(Y).astype(np.float32)).astype(np.float64)
    assert (np.abs(y.astype(np.float64) - Y) <= ulp + 1e-12 * mag).all()


def test_invariants():
    rng = np.random.default_rng(21)
    M, N, K = 3, 48, 256
    x, P, s_w, W_A, s_A, W_B, s_B = _rand_case(rng, M, N, K)
    x_q, s_x = oracle.quantize_act(x)
    y, acc, t = oracle.scaffold_lora_gemm(x_q, s_x, P, s_w, W_A, s_A, W_B, s_B)
    # flipping every sign bit negates the scaffold accumulator exactly
    _, acc_f, _ = oracle.scaffold_lora_gemm(x_q, s_x, ~P, s_w, W_A, s_A, W_B, s_B)
    assert np.array_equal(acc_f, -acc)
    # zero W_A (or zero W_B) removes the LoRA term: y = fl32(s_x * (s_w * acc))
    scaffold_only = (s_x.astype(np.float64)[:, None]
                     * (s_w.astype(np.float64)[None, :] * acc.astype(np.float64))).astype(np.float32)
    y0, _, _ = oracle.scaffold_lora_gemm(x_q, s_x, P, s_w, np.zeros_like(W_A), s_A, W_B, s_B)
    assert np.array_equal(y0, scaffold_only)
    y0b, _, t0 = oracle.scaffold_lora_gemm(x_q, s_x, P, s_w, W_A, s_A, np.zeros_like(W_B), s_B)
    assert not t0.any() and np.array_equal(y0b, scaffold_only)
    # rank 0 is the scaffold alone
    yr0, _, _ = oracle.scaffold_lora_gemm(x_q, s_x, P, s_w, None, None, None, None)
    assert np.array_equal(yr0, scaffold_only)
    # all sign bits set: every output channel sees sum_k x_q
    _, acc1, _ = oracle.scaffold_lora_gemm(x_q, s_x, np.full_like(P, 0xFF), s_w, W_A, s_A, W_B, s_B)
    assert (acc1 == x_q.astype(np.int64).sum(axis=1, keepdims=True)).all()
    # permuting output channels (P, s_w, W_A, s_A rows) permutes y's columns
    perm = rng.permutation(N)
    yp, _, _ = oracle.scaffold_lora_gemm(x_q, s_x, P[perm], s_w[perm], W_A[perm], s_A[perm], W_B, s_B)
    assert np.array_equal(yp, y[:, perm])
    # doubling s_w doubles the scaffold-only output exactly
    y2, _, _ = oracle.scaffold_lora_gemm(x_q, s_x, P, s_w * np.float32(2), np.zeros_like(W_A), s_A, W_B, s_B)
    assert np.array_equal(y2, scaffold_only * np.float32(2))


def test_sampled_positions_agree_with_full_product():
    rng = np.random.default_rng(31)
    M, N, K = 4, 70, 328
    x, P, s_w, W_A, s_A, W_B, s_B = _rand_case(rng, M, N, K)
    x_q, s_x = oracle.quantize_act(x)
    y, acc, t = oracle.scaffold_lora_gemm(x_q, s_x, P, s_w, W_A, s_A, W_B, s_B, nthreads=3)
    mi = rng.integers(0, M, 50)
    ni = rng.integers(0, N, 50)
    ys, accs, ts = oracle.scaffold_lora_at(x_q, s_x, P, s_w, W_A, s_A, W_B, s_B, mi, ni)
    assert np.array_equal(ys, y[mi, ni])
    assert np.array_equal(accs, acc[mi, ni])
    assert np.array_equal(ts, t[mi])


def test_rejects_bad_arguments():
    # K must be a multiple of 8: the C side refuses K = 12
    with pytest.raises(RuntimeError):
        oracle.scaffold_acc(np.zeros((1, 12), np.int8), np.zeros((1, 1), np.uint8))


# ------------------------------------------------------------------ int8 embedding / LM head

def test_lm_head_hand_worked_example():
    with open(os.path.join(GOLDEN, "lm_head_hand_worked.json")) as fh:
        g = json.load(fh)
    x = np.array(g["x"], np.float32)
    e = np.array(g["e"], np.int8)
    s_e = np.array(g["s_e"], np.float32)
    x_q, s_x = oracle.quantize_act(x)
    assert np.array_equal(s_x, np.array(g["expect_s_x"], np.float32))
    assert np.array_equal(x_q, np.array(g["expect_x_q"], np.int8))
    y, acc = oracle.int8_rowscale_gemm(x_q, s_x, e, s_e)
    assert np.array_equal(acc, np.array(g["expect_acc"], np.int32))
    assert np.array_equal(y, np.array(g["expect_y"], np.float32))
    out = oracle.embedding_lookup(np.array(g["lookup_ids"], np.int32), e, s_e)
    assert np.array_equal(out, np.array(g["expect_lookup"], np.float32))


@pytest.mark.parametrize("M,N,K", [(1, 50, 64), (3, 37, 136), (16, 20, 520)])
def test_lm_head_matches_fp64_blas(M, N, K):
    # acc against numpy's int64 matrix product; y against the dequantized fp64 product
    # sum_k (s_x x_q) (s_e E), which associates the scales differently
    rng = np.random.default_rng(500 + M)
    x = rng.standard_normal((M, K), dtype=np.float32)
    e = rng.integers(-127, 128, (N, K), dtype=np.int8)
    s_e = rng.uniform(1e-3, 1e-2, N).astype(np.float32)
    x_q, s_x = oracle.quantize_act(x)
    y, acc = oracle.int8_rowscale_gemm(x_q, s_x, e, s_e, nthreads=2)
    assert np.array_equal(acc.astype(np.int64), x_q.astype(np.int64) @ e.astype(np.int64).T)
    X = s_x.astype(np.float64)[:, None] * x_q.astype(np.float64)
    E = s_e.astype(np.float64)[:, None] * e.astype(np.float64)
    Y = X @ E.T
    mag = np.abs(X) @ np.abs(E).T
    ulp = np.spacing(np.abs(Y).astype(np.float32)).astype(np.float64)
    assert (np.abs(y.astype(np.float64) - Y) <= ulp + 1e-12 * mag).all()


def test_lm_head_invariants():
    rng = np.random.default_rng(41)
    M, N, K = 2, 64, 200
    x_q = rng.integers(-127, 128, (M, K), dtype=np.int8)
    s_x = rng.uniform(0.01, 0.1, M).astype(np.float32)
    e = rng.integers(-127, 128, (N, K), dtype=np.int8)
    s_e = rng.uniform(1e-3, 1e-2, N).astype(np.float32)
    y, acc = oracle.int8_rowscale_gemm(x_q, s_x, e, s_e)
    # negating the matrix negates acc and y exactly (-128 never occurs in either operand)
    y_n, acc_n = oracle.int8_rowscale_gemm(x_q, s_x, -e, s_e)
    assert np.array_equal(acc_n, -acc) and np.array_equal(y_n, -y)
    # permuting rows (with their scales) permutes the output columns
    perm = rng.permutation(N)
    y_p, acc_p = oracle.int8_rowscale_gemm(x_q, s_x, e[perm], s_e[perm])
    assert np.array_equal(acc_p, acc[:, perm]) and np.array_equal(y_p, y[:, perm])
    # a power-of-two row scale scales y exactly
    y_2, _ = oracle.int8_rowscale_gemm(x_q, s_x, e, s_e * np.float32(4))
    assert np.array_equal(y_2, y * np.float32(4))
    # the largest accumulator: every operand at +-127
    full = np.full((1, K), 127, np.int8)
    _, acc_max = oracle.int8_rowscale_gemm(full, np.ones(1, np.float32), -full, np.ones(1, np.float32))
    assert acc_max[0, 0] == -127 * 127 * K


def test_embedding_lookup_properties():
    rng = np.random.default_rng(43)
    V, K = 30, 48
    e = rng.integers(-127, 128, (V, K), dtype=np.int8)
    ids = np.array([0, 29, 5, 5, -1, 30, 1 << 30], np.int32)
    # unit scales return the int8 rows exactly; ids outside [0, V) give zeros
    out = oracle.embedding_lookup(ids, e, np.ones(V, np.float32))
    assert np.array_equal(out[:4], e[ids[:4]].astype(np.float32))
    assert not out[4:].any()
    # a scale 2^-j is an exact binary shift of every entry
    s_e = np.float32(2.0) ** -rng.integers(0, 20, V).astype(np.float32)
    out2 = oracle.embedding_lookup(ids[:4], e, s_e)
    assert np.array_equal(out2, e[ids[:4]].astype(np.float64) * s_e[ids[:4]].astype(np.float64)[:, None])
