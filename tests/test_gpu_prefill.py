"""GPU parity of the many-token kernels, each tile configuration pinned in turn.

The dispatcher picks the prefill kernel's tile configuration by a cost model, so
ordinary calls exercise only some of them; DFSSM_PREFILL_CFG pins one (0 .. n-1,
or -2 for the generic fallback kernel).  Every configuration must match the CPU
oracle on the same bar as the rest: x_q, s_x, t and the accumulators bit-exact, y
within 1e-5 of the magnitude of its terms.
"""
import numpy as np
import pytest

import synth_inputs as si
from test_gpu_parity import PATHS, _check_full, torch_cuda  # noqa: F401  (fixture)

pytestmark = pytest.mark.gpu

N_CFGS = 9                      # tile configurations of the prefill kernel
CFGS = list(range(N_CFGS)) + [-2]

SHAPES = [
    (17, 1, 64),        # one column, one 64-k slice (half a chunk)
    (33, 70, 192),      # odd chunk count and a half chunk
    (100, 513, 1024),   # ragged rows and columns
    (128, 512, 2048),   # whole tiles
    (129, 130, 4096),   # one row into the next tile, 32 chunks
    (300, 1000, 2112),  # several row tiles, ragged K
]


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("cfg", CFGS)
@pytest.mark.parametrize("M,N,K", SHAPES)
def test_prefill_config_parity(torch_cuda, monkeypatch, cfg, M, N, K, path):
    monkeypatch.setenv("DFSSM_PREFILL_CFG", str(cfg))
    _check_full(si.make_problem(M, N, K, max(1, K // 100), seed=M * 31 + N * 7 + K + 5 * cfg), path=path)


@pytest.mark.parametrize("cfg", CFGS)
@pytest.mark.parametrize("M,N,K", [(129, 130, 4096), (300, 1000, 2112)])
def test_prefill_config_one_call(torch_cuda, monkeypatch, cfg, M, N, K):
    # the one-call form at these sizes runs the quantizer, then the product computing t,
    # which writes t out from its first column tile (every configuration, and the
    # generic kernel)
    monkeypatch.setenv("DFSSM_PREFILL_CFG", str(cfg))
    _check_full(si.make_problem(M, N, K, max(1, K // 100), seed=M + N + K + 3 * cfg), path="one_call")


MAIN_TAIL = [(0, 1), (0, 2), (1, 2), (3, 5), (3, 6), (4, 5), (4, 6), (5, 6), (7, 8), (3, 4)]


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("main,tail", MAIN_TAIL)
@pytest.mark.parametrize("M,N,K", [(130, 700, 1024), (64, 1000, 256), (2048, 8512, 512)])
def test_prefill_main_plus_tail(torch_cuda, monkeypatch, main, tail, M, N, K, path):
    # whole tiles of one configuration and the remaining columns on a narrower one,
    # in one launch (the plan the cost model picks for widths like 8512); (3, 4) pins
    # a tail the main configuration has no instance for: every column then runs on
    # the main configuration
    monkeypatch.setenv("DFSSM_PREFILL_CFG", str(main))
    monkeypatch.setenv("DFSSM_PREFILL_TAIL", str(tail))
    _check_full(si.make_problem(M, N, K, 3, seed=M + N + K + 10 * main + tail), nthreads=16, path=path)


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("cfg", [(c, -1) for c in range(N_CFGS)] + MAIN_TAIL + [(-2, -1)])
def test_prefill_no_debug_instance_gives_same_y(torch_cuda, monkeypatch, cfg, path):
    # the kernels timed without acc_dbg (and t_dbg) are separate instances from the
    # ones the parity tests run with them: every plan's two instances must write the
    # same y, byte for byte (seam-crossing shape: ragged rows, a 8192-column main part)
    import torch
    from bit_scaffold_int8_amd.runner import DeviceProjections
    main, tail = cfg
    monkeypatch.setenv("DFSSM_PREFILL_CFG", str(main))
    monkeypatch.setenv("DFSSM_PREFILL_TAIL", str(tail))
    dp = DeviceProjections.from_problems([si.make_problem(200, 8512, 256, 3, seed=(main + 3) * 10 + tail + 2)],
                                         with_acc=True)
    fwd = dp.forward if path == "fused" else dp.forward_contract
    fwd(debug=True)
    torch.cuda.synchronize()
    y1 = dp.y.clone()
    dp.y.fill_(float("nan"))
    fwd(debug=False)
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int32), dp.y.view(torch.int32))


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("cfg", CFGS)
def test_prefill_config_rank_zero(torch_cuda, monkeypatch, cfg, path):
    monkeypatch.setenv("DFSSM_PREFILL_CFG", str(cfg))
    _check_full(si.make_problem(70, 200, 1024, 10, seed=11 + cfg), rank=0, path=path)


@pytest.mark.parametrize("cfg", CFGS)
def test_prefill_config_extreme_accumulators(torch_cuda, monkeypatch, cfg):
    # every code at +-127 and every sign +1 (or all -1): |acc| = 127 K, the largest
    # the contraction can produce
    monkeypatch.setenv("DFSSM_PREFILL_CFG", str(cfg))
    prob = si.make_problem(40, 96, 2048, 0, seed=3)
    prob.x = np.where(np.arange(2048)[None, :] % 2 == 0, 1.0, -1.0).astype(np.float32) * np.ones((40, 1), np.float32)
    prob.x[1::2] = 1.0
    prob.P[:48] = 0xFF
    prob.P[48:] = 0x00
    got, _ = _check_full(prob)
    assert got["acc"][1, 0] == 127 * 2048 and got["acc"][1, 50] == -127 * 2048


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("cfg", CFGS)
def test_prefill_config_batched(torch_cuda, monkeypatch, cfg, path):
    import torch
    from bit_scaffold_int8_amd.runner import DeviceProjections
    import oracle
    from test_gpu_parity import _magnitude, _assert_y
    monkeypatch.setenv("DFSSM_PREFILL_CFG", str(cfg))
    probs = si.make_copies(65, 300, 512, 5, seed=90 + cfg, copies=3)
    dp = DeviceProjections.from_problems(probs, with_acc=True)
    dp.forward() if path == "fused" else dp.forward_contract()
    torch.cuda.synchronize()
    for b, prob in enumerate(probs):
        xq_ref, sx_ref = oracle.quantize_act(prob.x)
        y_ref, acc_ref, t_ref = oracle.scaffold_lora_gemm(xq_ref, sx_ref, prob.P, prob.s_w, prob.W_A, prob.s_A,
                                                          prob.W_B, prob.s_B, nthreads=8)
        assert np.array_equal(dp.acc_dbg[b].cpu().numpy(), acc_ref), b
        assert np.array_equal(dp.t[b].cpu().numpy(), t_ref), b
        D = _magnitude(sx_ref, prob.s_w, acc_ref, prob.s_A, prob.W_A, prob.s_B, t_ref)
        _assert_y(dp.y[b].cpu().numpy(), y_ref, D, f"batch {b}")
