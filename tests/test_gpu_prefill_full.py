"""Full-size prefill parity: every output of both M = 2048 projections, through the
exact calls and kernel instances the benchmark times.

The benchmark times dfssm_quantize_act followed by dfssm_scaffold_lora_gemm with
acc_dbg = t_dbg = NULL (the kernel computes t = W_B x_q inside its K loop), and the
split form dfssm_quantize_lora_down + dfssm_scaffold_lora_gemm_given_t beside it.  The
debug outputs select separate kernel instances, so the timed instances are checked
here without them: x_q and s_x bit-exact, every y within 1e-5 of the magnitude of its
terms against the oracle run over the whole product (host threads, a few seconds);
then the debug instance's accumulators and t bit-exact, and its y, and the split
form's y, byte-identical to the timed instance's.
"""
import os

import numpy as np
import pytest

import oracle
import synth_inputs as si
from test_gpu_parity import _assert_y, _magnitude, torch_cuda  # noqa: F401  (fixture)

pytestmark = pytest.mark.gpu

_REF = {}


def _threads():
    return max(1, min(len(os.sched_getaffinity(0)), 16))


def _reference(which):
    if which not in _REF:
        prob = si.prefill_problems()[which]
        xq, sx = oracle.quantize_act(prob.x)
        y, acc, t = oracle.scaffold_lora_gemm(xq, sx, prob.P, prob.s_w, prob.W_A, prob.s_A, prob.W_B, prob.s_B,
                                              nthreads=_threads())
        D = _magnitude(sx, prob.s_w, acc, prob.s_A, prob.W_A, prob.s_B, t)
        _REF[which] = (prob, xq, sx, y, acc, t, D)
    return _REF[which]


@pytest.mark.parametrize("which", [0, 1], ids=["in_proj_k2048_n8512", "out_proj_k4096_n2048"])
def test_prefill_m2048_full_as_timed(torch_cuda, which):
    import torch
    from bit_scaffold_int8_amd.runner import DeviceProjections
    prob, xq, sx, y_ref, acc_ref, t_ref, D = _reference(which)
    name = ["in_proj", "out_proj"][which]
    print(f"prefill {name}: M{prob.M} K{prob.K} N{prob.N}, timed instance (no debug outputs)", flush=True)
    dp = DeviceProjections.from_problems([prob])
    dp.forward_contract(debug=False)
    torch.cuda.synchronize()
    assert np.array_equal(dp.s_x[0].cpu().numpy().view(np.uint32), sx.view(np.uint32)), "s_x"
    assert np.array_equal(dp.x_q[0].cpu().numpy(), xq), "x_q"
    y_timed = dp.y[0].cpu().numpy()
    _assert_y(y_timed, y_ref, D, f"{name} timed instance")

    # the debug instance: exact integers, and the same y bytes
    dd = DeviceProjections.from_problems([prob], with_acc=True)
    dd.forward_contract(debug=True)
    torch.cuda.synchronize()
    assert np.array_equal(dd.acc_dbg[0].cpu().numpy(), acc_ref), "acc"
    assert np.array_equal(dd.t[0].cpu().numpy(), t_ref), "t"
    assert np.array_equal(dd.y[0].cpu().numpy().view(np.uint32), y_timed.view(np.uint32)), "debug y"

    # the split form (t from quantize_lora_down, product given t), no debug outputs
    dp.y.fill_(float("nan"))
    dp.forward(debug=False)
    torch.cuda.synchronize()
    assert np.array_equal(dp.t[0].cpu().numpy(), t_ref), "t (split form)"
    assert np.array_equal(dp.y[0].cpu().numpy().view(np.uint32), y_timed.view(np.uint32)), "split-form y"
