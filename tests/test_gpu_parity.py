"""GPU parity: the HIP path through the C ABI against the CPU oracle, element by element.

Bar: x_q, s_x, t and the scaffold accumulators bit-exact; y within 1e-5 relative to
the magnitude of its terms, D = |s_x| (|s_w acc| + |s_A| sum_r |W_A s_B t|), per
element (several fp32 evaluation orders of the epilogue are correct; D bounds all
of them).  Full-size prefill is checked on sampled positions the oracle computes
one by one, plus full x_q, s_x and t.
"""
import numpy as np
import pytest

import oracle
import synth_inputs as si

pytestmark = pytest.mark.gpu

REL_TOL = 1e-5


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


PATHS = ("fused", "contract")


def _run_hip(prob, with_acc=True, rank=16, path="fused"):
    """Run one problem through the C ABI:
    'fused'    quantize_lora_down + gemm_given_t (batched entry points, batch 1);
    'unfused'  quantize_act, lora_down, gemm_given_t (single-problem entry points);
    'contract' quantize_act + scaffold_lora_gemm, which computes t itself (batched);
    'contract_unfused' the same through the single-problem entry points;
    'one_call' scaffold_lora_forward (batched entry point, batch 1)."""
    from bit_scaffold_int8_amd.runner import DeviceProjections
    import torch
    dp = DeviceProjections.from_problems([prob], rank=bool(rank), with_acc=with_acc)
    if path == "fused":
        dp.forward()
    elif path == "unfused":
        dp.forward_unfused()
    elif path == "contract":
        dp.forward_contract()
    elif path == "contract_unfused":
        dp.forward_contract_unfused()
    elif path == "one_call":
        dp.forward_one_call()
    else:
        raise ValueError(path)
    torch.cuda.synchronize()
    out = dict(x_q=dp.x_q[0].cpu().numpy(), s_x=dp.s_x[0].cpu().numpy(), y=dp.y[0].cpu().numpy())
    if rank:
        out["t"] = dp.t[0].cpu().numpy()
    if with_acc:
        out["acc"] = dp.acc_dbg[0].cpu().numpy()
    return out


def _magnitude(s_x, s_w, acc, s_A, W_A, s_B, t):
    """D[m, n] in fp64 (with rank 0, only the scaffold term)."""
    sc = np.abs(s_w.astype(np.float64)[None, :] * acc.astype(np.float64))
    if W_A is not None:
        u = np.abs(s_B.astype(np.float64)[None, :] * t.astype(np.float64))       # [M, r]
        lo = u @ np.abs(W_A.astype(np.float64)).T                                 # [M, N]
        sc = sc + np.abs(s_A.astype(np.float64))[None, :] * lo
    return np.abs(s_x.astype(np.float64))[:, None] * sc


def _assert_y(y, y_ref, D, where=""):
    err = np.abs(y.astype(np.float64) - y_ref.astype(np.float64))
    bad = err > REL_TOL * D
    assert not bad.any(), (f"{where}: {bad.sum()} of {bad.size} outputs outside 1e-5*D; "
                           f"worst err/D = {(err / np.maximum(D, 1e-300)).max():.3e}")


def _check_full(prob, rank=16, nthreads=8, path="fused"):
    got = _run_hip(prob, rank=rank, path=path)
    xq_ref, sx_ref = oracle.quantize_act(prob.x)
    assert np.array_equal(got["s_x"].view(np.uint32), sx_ref.view(np.uint32)), "s_x not bit-exact"
    assert np.array_equal(got["x_q"], xq_ref), "x_q not bit-exact"
    if rank:
        y_ref, acc_ref, t_ref = oracle.scaffold_lora_gemm(xq_ref, sx_ref, prob.P, prob.s_w, prob.W_A, prob.s_A,
                                                          prob.W_B, prob.s_B, nthreads=nthreads)
        assert np.array_equal(got["t"], t_ref), "t not bit-exact"
        D = _magnitude(sx_ref, prob.s_w, acc_ref, prob.s_A, prob.W_A, prob.s_B, t_ref)
    else:
        y_ref, acc_ref, _ = oracle.scaffold_lora_gemm(xq_ref, sx_ref, prob.P, prob.s_w, None, None, None, None,
                                                      nthreads=nthreads)
        D = _magnitude(sx_ref, prob.s_w, acc_ref, None, None, None, None)
    assert np.array_equal(got["acc"], acc_ref), "acc not bit-exact"
    _assert_y(got["y"], y_ref, D, f"M{prob.M} N{prob.N} K{prob.K} rank{rank}")
    return got, y_ref


# ------------------------------------------------------------------ the five workloads

@pytest.mark.parametrize("path", PATHS)
def test_tiny_m1_k256_n512(torch_cuda, path):
    (M, N, K, o), = si.CONFIGS["tiny_m1_k256_n512"]["shapes"]
    _check_full(si.make_problem(M, N, K, o, seed=0), path=path)


@pytest.mark.parametrize("path", PATHS)
def test_out_proj_decode_m1_k4096_n2048(torch_cuda, path):
    (M, N, K, o), = si.CONFIGS["out_proj_decode_m1_k4096_n2048"]["shapes"]
    # several rotated copies from the same stream, as the benchmark draws them
    for prob in si.make_copies(M, N, K, o, seed=1, copies=3):
        _check_full(prob, path=path)


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("M", [1, 4, 16])
def test_in_proj_decode_k2048_n8512(torch_cuda, M, path):
    _check_full(si.make_problem(M, 8512, 2048, 2, seed=2), path=path)


def test_decode_sweep_48_layers_sampled(torch_cuda):
    # 48 x (in_proj, out_proj) weight sets drawn from one stream; check the first two
    # and last two layers in full (the rest only differ in their random draws)
    cfg = si.CONFIGS["decode_sweep_48l"]
    rng = np.random.default_rng(cfg["seed"])
    for layer in range(cfg["layers"]):
        for (M, N, K, o) in cfg["shapes"]:
            prob = si.draw_problem(rng, M, N, K, o)
            if layer in (0, 1, 46, 47):
                _check_full(prob)


@pytest.mark.parametrize("which", [0, 1])
def test_prefill_m2048_sampled(torch_cuda, which):
    prob = si.prefill_problems()[which]
    got = _run_hip(prob)
    xq_ref, sx_ref = oracle.quantize_act(prob.x)
    assert np.array_equal(got["s_x"].view(np.uint32), sx_ref.view(np.uint32))
    assert np.array_equal(got["x_q"], xq_ref)
    assert np.array_equal(got["t"], oracle.lora_down(xq_ref, prob.W_B))
    srng = np.random.default_rng(99)
    # random positions plus every tile corner and the ragged edges, and the seams of the
    # plans the cost model picks: 64-, 128- and 256-column tiles, 64- and 128-row tiles,
    # and the first column of a narrow tail (8192 of 8512)
    mi = np.concatenate([srng.integers(0, prob.M, 3000), [0, prob.M - 1, 127, 128, 0, prob.M - 1]])
    ni = np.concatenate([srng.integers(0, prob.N, 3000), [0, prob.N - 1, 0, prob.N - 1, 127, 128]])
    seam_cols = [c for c in (63, 64, 255, 256, 511, 512, 8191, 8192, 8193, prob.N - 65, prob.N - 64)
                 if 0 <= c < prob.N]
    seam_rows = [63, 64, 127, 128, 1023, 1024, prob.M - 65, prob.M - 64]
    mi = np.concatenate([mi, np.repeat(seam_rows, len(seam_cols))])
    ni = np.concatenate([ni, np.tile(seam_cols, len(seam_rows))])
    y_ref, acc_ref, t_ref = oracle.scaffold_lora_at(xq_ref, sx_ref, prob.P, prob.s_w, prob.W_A, prob.s_A,
                                                    prob.W_B, prob.s_B, mi, ni)
    assert np.array_equal(got["acc"][mi, ni], acc_ref)
    # D per sampled element
    u = np.abs(prob.s_B.astype(np.float64)[None, :] * t_ref.astype(np.float64))
    lo = (u * np.abs(prob.W_A[ni].astype(np.float64))).sum(axis=1)
    D = np.abs(sx_ref[mi].astype(np.float64)) * (
        np.abs(prob.s_w[ni].astype(np.float64) * acc_ref) + np.abs(prob.s_A[ni].astype(np.float64)) * lo)
    _assert_y(got["y"][mi, ni], y_ref, D, f"prefill {which}")
    # a property that holds at any size: with the accumulators verified exact at the
    # samples, every row's acc lies within the exact bound |acc| <= sum_k |x_q|
    bound = np.abs(xq_ref.astype(np.int64)).sum(axis=1)
    assert (np.abs(got["acc"]) <= bound[:, None]).all()
    # and acc has the parity of sum_k x_q (each term is +-x_q)
    assert ((got["acc"].astype(np.int64) - xq_ref.astype(np.int64).sum(axis=1)[:, None]) % 2 == 0).all()


# ------------------------------------------------------------------ edge shapes

@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("M", [1, 2, 3, 15, 16, 17, 127, 128, 129])
def test_token_counts(torch_cuda, M, path):
    _check_full(si.make_problem(M, 100, 2048, 2, seed=1000 + M), path=path)


@pytest.mark.parametrize("M,N,K", [
    (1, 1, 8), (1, 63, 40), (1, 64, 136), (1, 65, 1000), (3, 33, 2056), (16, 17, 4104),
    (17, 1, 8), (17, 63, 40), (33, 70, 1000), (129, 65, 520), (200, 130, 136), (64, 129, 4104),
    (1, 64, 16384), (2, 40, 16392), (1, 300, 12288),
])
@pytest.mark.parametrize("path", PATHS)
def test_ragged_shapes(torch_cuda, M, N, K, path):
    _check_full(si.make_problem(M, N, K, 2 if K >= 16 else 0, seed=M * 7 + N * 3 + K), path=path)


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("M", [1, 5, 40])
def test_rank_zero(torch_cuda, M, path):
    _check_full(si.make_problem(M, 96, 1024, 2, seed=77 + M), rank=0, path=path)


@pytest.mark.parametrize("M,N,K", [(1, 2048, 4096), (4, 300, 2048), (16, 64, 1000), (40, 90, 520),
                                   (2, 70, 72), (1, 33, 65536)])
@pytest.mark.parametrize("path", ["unfused", "contract_unfused"])
def test_unfused_entry_points(torch_cuda, M, N, K, path):
    # the single-problem entry points called one by one: quantize_act, lora_down and
    # gemm_given_t, or quantize_act and scaffold_lora_gemm (t computed inside)
    _check_full(si.make_problem(M, N, K, 2, seed=5 * M + K), path=path)


@pytest.mark.parametrize("M,K", [(1, 65536), (3, 65544), (2, 131072)])
def test_long_rows_take_the_two_kernel_fallback(torch_cuda, M, K):
    # rows too long for the fused kernel's LDS: quantize + lora_down run as two kernels
    _check_full(si.make_problem(M, 24, K, 2, seed=K + M))


@pytest.mark.parametrize("M,K", [(1, 1), (3, 7), (2, 1001), (5, 4099)])
def test_quantize_act_any_row_length(torch_cuda, M, K):
    import torch
    from bit_scaffold_int8_amd import dfssm
    rng = np.random.default_rng(M * 100 + K)
    x = rng.standard_normal((M, K), dtype=np.float32)
    x[0, 0] = 30.0
    xd = torch.from_numpy(x).cuda()
    x_q = torch.empty((M, K), dtype=torch.int8, device="cuda")
    s_x = torch.empty((M,), dtype=torch.float32, device="cuda")
    dfssm.dfssm_quantize_act(xd, x_q, s_x)
    torch.cuda.synchronize()
    q_ref, s_ref = oracle.quantize_act(x)
    assert np.array_equal(x_q.cpu().numpy(), q_ref)
    assert np.array_equal(s_x.cpu().numpy().view(np.uint32), s_ref.view(np.uint32))


@pytest.mark.parametrize("B,M,N,K", [(5, 1, 2048, 4096), (3, 4, 8512, 2048), (4, 33, 100, 1024), (7, 2, 40, 136)])
@pytest.mark.parametrize("path", PATHS)
def test_strided_batched_matches_oracle_per_problem(torch_cuda, B, M, N, K, path):
    import torch
    from bit_scaffold_int8_amd.runner import DeviceProjections
    probs = si.make_copies(M, N, K, 2, seed=B * 1000 + K, copies=B)
    dp = DeviceProjections.from_problems(probs, with_acc=True)
    dp.forward() if path == "fused" else dp.forward_contract()
    torch.cuda.synchronize()
    for b, prob in enumerate(probs):
        xq_ref, sx_ref = oracle.quantize_act(prob.x)
        y_ref, acc_ref, t_ref = oracle.scaffold_lora_gemm(xq_ref, sx_ref, prob.P, prob.s_w, prob.W_A, prob.s_A,
                                                          prob.W_B, prob.s_B, nthreads=8)
        assert np.array_equal(dp.x_q[b].cpu().numpy(), xq_ref)
        assert np.array_equal(dp.t[b].cpu().numpy(), t_ref)
        assert np.array_equal(dp.acc_dbg[b].cpu().numpy(), acc_ref)
        D = _magnitude(sx_ref, prob.s_w, acc_ref, prob.s_A, prob.W_A, prob.s_B, t_ref)
        _assert_y(dp.y[b].cpu().numpy(), y_ref, D, f"batch {b}")


@pytest.mark.parametrize("B,M,N,K", [(512, 1, 2048, 4096), (200, 3, 2000, 4096), (300, 16, 1024, 2048)])
@pytest.mark.parametrize("path", PATHS)
def test_large_batches_one_group_round(torch_cuda, B, M, N, K, path):
    # batches large enough that the decode kernel gives each group a whole problem (or
    # an even share of one) in a single resident round: the benchmark's launch (512
    # out_proj copies), ragged rows with an uneven split, and 16 tokens on 4-wave groups
    import torch
    from bit_scaffold_int8_amd.runner import DeviceProjections
    probs = si.make_copies(M, N, K, 2, seed=B + N + K, copies=B)
    dp = DeviceProjections.from_problems(probs, with_acc=True)
    dp.forward() if path == "fused" else dp.forward_contract()
    torch.cuda.synchronize()
    acc_all, y_all, t_all = dp.acc_dbg.cpu().numpy(), dp.y.cpu().numpy(), dp.t.cpu().numpy()
    for b, prob in enumerate(probs):
        xq_ref, sx_ref = oracle.quantize_act(prob.x)
        y_ref, acc_ref, t_ref = oracle.scaffold_lora_gemm(xq_ref, sx_ref, prob.P, prob.s_w, prob.W_A, prob.s_A,
                                                          prob.W_B, prob.s_B, nthreads=16)
        assert np.array_equal(t_all[b], t_ref), b
        assert np.array_equal(acc_all[b], acc_ref), b
        D = _magnitude(sx_ref, prob.s_w, acc_ref, prob.s_A, prob.W_A, prob.s_B, t_ref)
        _assert_y(y_all[b], y_ref, D, f"batch {b}")


@pytest.mark.parametrize("path", PATHS)
def test_gemm_without_debug_output_gives_same_y(torch_cuda, path):
    import torch
    from bit_scaffold_int8_amd.runner import DeviceProjections
    for (M, N, K) in [(1, 2048, 4096), (300, 200, 512)]:
        dp = DeviceProjections.from_problems([si.make_problem(M, N, K, 2, seed=3)], with_acc=True)
        fwd = dp.forward if path == "fused" else dp.forward_contract
        fwd(debug=True)
        torch.cuda.synchronize()
        y1 = dp.y.clone()
        dp.y.zero_()
        fwd(debug=False)
        torch.cuda.synchronize()
        assert torch.equal(y1, dp.y)


@pytest.mark.parametrize("M,N,K", [(1, 2048, 4096), (5, 300, 2048), (40, 200, 1024), (3, 33, 200)])
def test_contract_matches_given_t_bitwise(torch_cuda, M, N, K):
    # t computed inside the product (scaffold_lora_gemm) and t given (quantize_lora_down
    # + scaffold_lora_gemm_given_t) produce the same bytes
    a = _run_hip(si.make_problem(M, N, K, 2, seed=M + N + K), path="fused")
    b = _run_hip(si.make_problem(M, N, K, 2, seed=M + N + K), path="contract")
    for k in ("x_q", "s_x", "t", "acc", "y"):
        assert np.array_equal(a[k].view(np.uint8), b[k].view(np.uint8)), k


def test_zero_token_and_exact_ties(torch_cuda):
    prob = si.make_problem(5, 80, 512, 2, seed=5)
    prob.x[1] = 0.0                     # all-zero token: s_x = 0, y = 0
    prob.x[3] = np.round(prob.x[3] * 4) / 4
    prob.x[3, 0] = 127.0                # absmax 127 -> s_x = 1, many exact .5 ties
    prob.x[3, 1:40] = np.arange(39) - 19.5
    got, y_ref = _check_full(prob)
    assert not got["y"][1].any() and got["s_x"][1] == 0 and not got["x_q"][1].any()


def test_flipped_signs_negate_accumulators(torch_cuda):
    prob = si.make_problem(3, 48, 1024, 2, seed=8)
    a = _run_hip(prob)["acc"]
    prob.P = ~prob.P
    b = _run_hip(prob)["acc"]
    assert np.array_equal(a, -b)


def test_repeated_calls_are_deterministic(torch_cuda):
    prob = si.make_problem(16, 8512, 2048, 2, seed=2)
    a, b = _run_hip(prob), _run_hip(prob)
    for k in a:
        assert np.array_equal(a[k], b[k]), k


def _near_tie_rows(K=1024):
    """Rows whose quotients x/s land within a few ulps of half-integers, for several
    scales (including one whose reciprocal overflows fp32)."""
    rng = np.random.default_rng(4242)
    rows = []
    for amax in (100.0, 3.7, 1e-3, 5.0e4, 1e-39):
        s = np.float32(amax) / np.float32(127)
        vals = [np.float32(amax)]
        for k in range(-127, 127):
            c = np.float32((k + 0.5) * np.float64(s))
            for d in (-2, -1, 0, 1, 2):
                v = c
                for _ in range(abs(d)):
                    v = np.nextafter(v, np.float32(np.inf if d > 0 else -np.inf), dtype=np.float32)
                vals.append(v)
        vals = np.array(vals, np.float32)
        vals = vals[np.abs(vals) <= np.float32(amax)]
        row = (rng.uniform(-1, 1, K) * amax * 0.5).astype(np.float32)
        row[:len(vals)] = vals[:K]
        row[0] = np.float32(amax)
        rows.append(row)
    return np.stack(rows)


def test_quantizer_near_ties_bit_exact(torch_cuda):
    import torch
    from bit_scaffold_int8_amd import dfssm
    x = _near_tie_rows()
    M, K = x.shape
    q_ref, s_ref = oracle.quantize_act(x)
    xd = torch.from_numpy(x).cuda()
    x_q = torch.empty((M, K), dtype=torch.int8, device="cuda")
    s_x = torch.empty((M,), dtype=torch.float32, device="cuda")
    dfssm.dfssm_quantize_act(xd, x_q, s_x)
    torch.cuda.synchronize()
    assert np.array_equal(s_x.cpu().numpy().view(np.uint32), s_ref.view(np.uint32))
    assert np.array_equal(x_q.cpu().numpy(), q_ref)
    # the fused quantize + LoRA-down kernel, token counts that exercise every
    # waves-per-row split (1, 2, 4, 8 rows per group and two passes)
    for m in (1, 2, 3, 5, 9, 16):
        xs = np.concatenate([x] * 4)[:m]
        prob = si.make_problem(m, 16, K, 0, seed=m)
        prob.x = np.ascontiguousarray(xs)
        got = _run_hip(prob)
        q2, s2 = oracle.quantize_act(xs)
        assert np.array_equal(got["s_x"].view(np.uint32), s2.view(np.uint32)), m
        assert np.array_equal(got["x_q"], q2), m
        assert np.array_equal(got["t"], oracle.lora_down(q2, prob.W_B)), m


@pytest.mark.parametrize("B", [48, 96])
@pytest.mark.parametrize("N,K", [(2048, 4096), (8512, 2048)], ids=["out_proj", "in_proj"])
@pytest.mark.parametrize("form", ["one_call", "fused", "contract"])
def test_mid_batches_every_problem(torch_cuda, B, N, K, form):
    # The decode kernel's launch plan at batches that do not divide its resident group
    # count (the 48-layer sweep's batch, and twice it): every group count per problem
    # must still cover each problem's rows exactly once.  Every problem against the
    # oracle, with the accumulators; then the instances without debug outputs must
    # write the same y bytes.
    import torch
    from bit_scaffold_int8_amd.runner import DeviceProjections
    probs = si.make_copies(1, N, K, 2, seed=7 * B + N, copies=B)
    print(f"batch {B}, N {N}, K {K}, {form}", flush=True)
    dp = DeviceProjections.from_problems(probs, with_acc=True)
    run = {"one_call": dp.forward_one_call, "fused": dp.forward, "contract": dp.forward_contract}[form]
    run()
    torch.cuda.synchronize()
    xq_all, acc_all, y_all = dp.x_q.cpu().numpy(), dp.acc_dbg.cpu().numpy(), dp.y.cpu().numpy()
    for b, prob in enumerate(probs):
        xq_ref, sx_ref = oracle.quantize_act(prob.x)
        y_ref, acc_ref, t_ref = oracle.scaffold_lora_gemm(xq_ref, sx_ref, prob.P, prob.s_w, prob.W_A, prob.s_A,
                                                          prob.W_B, prob.s_B, nthreads=16)
        assert np.array_equal(xq_all[b], xq_ref), b
        assert np.array_equal(acc_all[b], acc_ref), b
        D = _magnitude(sx_ref, prob.s_w, acc_ref, prob.s_A, prob.W_A, prob.s_B, t_ref)
        _assert_y(y_all[b], y_ref, D, f"problem {b}")
    dp.y.fill_(float("nan"))
    run(debug=False)
    torch.cuda.synchronize()
    assert np.array_equal(dp.y.cpu().numpy().view(np.uint32), y_all.view(np.uint32)), "y without debug outputs"
