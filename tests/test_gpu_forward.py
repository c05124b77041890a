"""GPU parity of the one-call form (dfssm_scaffold_lora_forward): x -> x_q, s_x, t, y.

At decode shapes it is one kernel whose every workgroup quantizes the tokens and
computes t = W_B x_q itself; elsewhere two kernels: for many-token shapes with under 2^24
outputs the quantizer, then the MFMA product computing t in its K loop (which writes t
out), otherwise those of the two-call form.
Same bar as the rest: x_q, s_x, t and the accumulators bit-exact against the CPU
oracle, y within 1e-5 of the magnitude of its terms; and y bit-identical to the
two-call form's (both apply the same epilogue arithmetic to the same integers).
"""
import numpy as np
import pytest

import oracle
import synth_inputs as si
from test_gpu_parity import _assert_y, _magnitude, torch_cuda  # noqa: F401  (fixture)

pytestmark = pytest.mark.gpu


def _device(probs, rank=True):
    from bit_scaffold_int8_amd.runner import DeviceProjections
    return DeviceProjections.from_problems(probs, rank=rank, with_acc=True)


def _check(probs, rank=True, nthreads=8, compare_two_call=True):
    import torch
    dp = _device(probs, rank)
    dp.forward_one_call()
    torch.cuda.synchronize()
    got = dict(x_q=dp.x_q.cpu().numpy(), s_x=dp.s_x.cpu().numpy(), y=dp.y.cpu().numpy(),
               acc=dp.acc_dbg.cpu().numpy(), t=dp.t.cpu().numpy() if rank else None)
    for b, prob in enumerate(probs):
        xq_ref, sx_ref = oracle.quantize_act(prob.x)
        assert np.array_equal(got["s_x"][b].view(np.uint32), sx_ref.view(np.uint32)), f"s_x, problem {b}"
        assert np.array_equal(got["x_q"][b], xq_ref), f"x_q, problem {b}"
        if rank:
            y_ref, acc_ref, t_ref = oracle.scaffold_lora_gemm(xq_ref, sx_ref, prob.P, prob.s_w, prob.W_A,
                                                              prob.s_A, prob.W_B, prob.s_B, nthreads=nthreads)
            assert np.array_equal(got["t"][b], t_ref), f"t, problem {b}"
            D = _magnitude(sx_ref, prob.s_w, acc_ref, prob.s_A, prob.W_A, prob.s_B, t_ref)
        else:
            y_ref, acc_ref, _ = oracle.scaffold_lora_gemm(xq_ref, sx_ref, prob.P, prob.s_w, None, None, None, None,
                                                          nthreads=nthreads)
            D = _magnitude(sx_ref, prob.s_w, acc_ref, None, None, None, None)
        assert np.array_equal(got["acc"][b], acc_ref), f"acc, problem {b}"
        _assert_y(got["y"][b], y_ref, D, f"problem {b}")
    if compare_two_call:
        two = _device(probs, rank)
        two.forward()
        torch.cuda.synchronize()
        assert np.array_equal(two.y.cpu().numpy().view(np.uint32), got["y"].view(np.uint32)), \
            "one-call y differs from the two-call form's"
    return got


# one launch: K % 128 == 0, K <= 4096, M <= 4, M K <= 1024 x waves per group
FUSED = [(1, 512, 128), (2, 100, 256), (4, 64, 256), (1, 333, 512), (2, 130, 1024), (1, 2048, 4096),
         (2, 2048, 4096), (1, 8512, 2048), (2, 8512, 2048), (3, 1000, 1280), (1, 17, 384), (1, 1, 4096)]
# two launches
FALLBACK = [(4, 2048, 4096), (5, 300, 2048), (1, 200, 136), (1, 300, 8192), (16, 1000, 2048), (64, 700, 1024)]
# many tokens: the quantizer, then the product computing t (ragged M and N, several K
# tiles, N > K); K % 64 != 0 and 2^24 outputs or more keep the two-call form's kernels
MANY = [(17, 2048, 4096), (200, 2048, 4096), (70, 96, 1088), (256, 1024, 1024), (33, 100, 136), (40, 600, 512),
        (4100, 4096, 128), (2, 100, 20480)]  # the last: few tokens, K past the decode kernel's 16384


@pytest.mark.parametrize("M,N,K", FUSED + FALLBACK + MANY)
def test_one_call_matches_oracle(torch_cuda, M, N, K):
    _check([si.make_problem(M, N, K, max(1, K // 512), seed=7 * M + N + K)])


@pytest.mark.parametrize("M,N,K", [(1, 2048, 4096), (2, 513, 2048), (4, 100, 512)])
def test_one_call_rank_zero(torch_cuda, M, N, K):
    _check([si.make_problem(M, N, K, 2, seed=M + N + K)], rank=False)


# (64 out_proj copies: a throughput batch with several groups per problem, so two kernels)
@pytest.mark.parametrize("B,M,N,K", [(3, 1, 2048, 4096), (5, 2, 8512, 2048), (7, 1, 40, 256), (4, 6, 100, 1024),
                                     (64, 1, 2048, 4096), (3, 40, 256, 512), (2, 100, 2048, 4096)])
def test_one_call_batched(torch_cuda, B, M, N, K):
    _check(si.make_copies(M, N, K, 2, seed=B * 100 + M, copies=B))


def test_one_call_benchmark_launch_512_copies(torch_cuda):
    # the benchmark's decode step: 512 out_proj copies, one launch, every output checked
    _check(si.make_copies(1, 2048, 4096, 2, seed=1, copies=512), nthreads=16)


def test_one_call_zero_token_and_ties(torch_cuda):
    # an all-zero token (s_x = 0, codes 0) next to one whose values sit on rounding ties
    prob = si.make_problem(2, 300, 1024, 0, seed=12)
    prob.x[0] = 0.0
    prob.x[1] = (np.arange(1024) % 255 - 127).astype(np.float32) * np.float32(0.5)
    prob.x[1, 7] = 127.0  # s = 1: codes are rint(v) with ties to even
    _check([prob])


def test_one_call_outputs_only_from_first_group(torch_cuda):
    # several groups per problem each compute x_q, s_x and t; the results are written
    # once and equal the two-call form's, including on repeated calls
    import torch
    probs = [si.make_problem(1, 8512, 2048, 2, seed=21)]
    dp = _device(probs)
    outs = []
    for _ in range(3):
        dp.forward_one_call()
        torch.cuda.synchronize()
        outs.append((dp.x_q.cpu().numpy().copy(), dp.t.cpu().numpy().copy(), dp.y.cpu().numpy().copy()))
    for o in outs[1:]:
        assert all(np.array_equal(a, b) for a, b in zip(o, outs[0]))
    _check(probs)


def test_one_call_equals_two_call_form_on_random_shapes(torch_cuda):
    # the one-call form promises the two-call form's results bit for bit, whichever
    # kernels it takes: seeded random many-token shapes on both sides of the routing
    # (ragged M and N, K with and without whole 64-k slices, batches), every output byte
    # compared (x_q, s_x, t, y; no oracle needed for an identity between two paths)
    import torch
    rng = np.random.default_rng(2024)
    for case in range(24):
        M = int(rng.integers(1, 400))
        N = int(rng.integers(1, 3000))
        K = int(rng.choice([64, 136, 448, 1024, 2112, 4096]))
        B = int(rng.integers(1, 4))
        print(f"case {case}: B={B} M={M} N={N} K={K}", flush=True)
        probs = si.make_copies(M, N, K, max(1, K // 512), seed=500 + case, copies=B)
        one, two = _device(probs), _device(probs)
        one.forward_one_call()
        two.forward()
        torch.cuda.synchronize()
        for name in ("x_q", "s_x", "t", "y", "acc_dbg"):
            a = getattr(one, name).cpu().numpy()
            b = getattr(two, name).cpu().numpy()
            assert np.array_equal(a.view(np.uint8), b.view(np.uint8)), f"{name}, case {case}"
