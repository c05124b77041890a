"""GPU parity of the one-launch multi-layer decode (dfssm_decode_layers) against the
chain of CPU oracles, stage by stage.

The kernel runs each layer's in_proj, Mamba-2 step and out_proj in one persistent
launch and, with a trace buffer, records every layer's intermediates.  Each stage is
checked against its oracle fed with the GPU's own input to that stage, on the bar of
that stage:
  * quantizer: x_q and s_x bit-exact (of the layer's input and of the step's output);
  * projections: accumulators and t bit-exact, outputs within 1e-5 of the magnitude of
    their terms (the projection tests' bar);
  * Mamba-2 step: windows bit-exact, state and output within the step tests' bar.
The last layer's output must equal x_out byte for byte, and a second token (the
windows swapped, the state carried) must pass the same checks: what the first call
left in the workspace (the done count cleared, the call counter advanced, its tagged
values) does not disturb the second.
"""
import numpy as np
import pytest

import oracle
import synth_inputs as si
from oracle import decode_chain as dc
from test_gpu_mamba2 import TOL as M2_TOL, _oracle_step_with_magnitudes
from test_gpu_parity import _assert_y, _magnitude, torch_cuda  # noqa: F401  (fixture)

pytestmark = pytest.mark.gpu

EPS = 1e-5
DONE_WORD, GEN_WORD = 0, 16     # the workspace's done count and call counter (then the exchange slots)
TW = dict(zx=(0, 8512), out=(8512, 4096), xn=(12608, 2048), acc_in=(14656, 8512), acc_out=(23168, 2048),
          xq_in=(25216, 512), xq_out=(25728, 1024), t_in=(26752, 16), t_out=(26768, 16), sx=(26784, 2))


def _field(tr, l, name, dtype):
    o, n = TW[name]
    return np.ascontiguousarray(tr[l, o:o + n]).view(dtype)


def _check_token(stack, tr, x_in, conv_in, ssm_in, conv_out, ssm_out, x_out, layers):
    """Stage-wise checks of one token, for the given layers."""
    for l in layers:
        x = x_in if l == 0 else _field(tr, l - 1, "xn", np.float32)
        # in_proj
        xq, sx = oracle.quantize_act(x[None])
        assert np.array_equal(_field(tr, l, "xq_in", np.int8), xq[0]), f"layer {l}: x_q"
        assert _field(tr, l, "sx", np.float32)[0].view(np.uint32) == sx[0].view(np.uint32), f"layer {l}: s_x"
        y, acc, t = oracle.scaffold_lora_gemm(xq, sx, stack.in_P[l], stack.in_s_w[l], stack.in_W_A[l],
                                              stack.in_s_A[l], stack.in_W_B[l], stack.in_s_B[l], nthreads=8)
        assert np.array_equal(_field(tr, l, "acc_in", np.int32), acc[0]), f"layer {l}: in_proj acc"
        assert np.array_equal(_field(tr, l, "t_in", np.int32), t[0]), f"layer {l}: in_proj t"
        zx = _field(tr, l, "zx", np.float32)
        _assert_y(zx[None], y, _magnitude(sx, stack.in_s_w[l], acc, stack.in_s_A[l], stack.in_W_A[l],
                                          stack.in_s_B[l], t), f"layer {l}: in_proj y")
        # Mamba-2 step on the GPU's in_proj output
        out_r, win_r, st_r, st_mag, out_mag = _oracle_step_with_magnitudes(
            stack.layer(l), zx[None], conv_in[l][None], ssm_in[l][None].astype(np.float64), 64, 64, 128, EPS)
        assert np.array_equal(conv_out[l], win_r[0].astype(np.float32)), f"layer {l}: windows"
        err = np.abs(ssm_out[l].astype(np.float64) - st_r[0])
        assert (err <= M2_TOL * st_mag[0] + 1e-30).all(), f"layer {l}: state"
        out = _field(tr, l, "out", np.float32)
        err = np.abs(out.astype(np.float64) - out_r[0])
        assert (err <= M2_TOL * out_mag[0] + 1e-30).all(), f"layer {l}: out, worst {(err / out_mag[0]).max():.2e}"
        # out_proj on the GPU's step output
        xq2, sx2 = oracle.quantize_act(out[None])
        assert np.array_equal(_field(tr, l, "xq_out", np.int8), xq2[0]), f"layer {l}: x_q of out"
        assert _field(tr, l, "sx", np.float32)[1].view(np.uint32) == sx2[0].view(np.uint32), f"layer {l}: s_x"
        y2, acc2, t2 = oracle.scaffold_lora_gemm(xq2, sx2, stack.out_P[l], stack.out_s_w[l], stack.out_W_A[l],
                                                 stack.out_s_A[l], stack.out_W_B[l], stack.out_s_B[l], nthreads=8)
        assert np.array_equal(_field(tr, l, "acc_out", np.int32), acc2[0]), f"layer {l}: out_proj acc"
        assert np.array_equal(_field(tr, l, "t_out", np.int32), t2[0]), f"layer {l}: out_proj t"
        _assert_y(_field(tr, l, "xn", np.float32)[None], y2,
                  _magnitude(sx2, stack.out_s_w[l], acc2, stack.out_s_A[l], stack.out_W_A[l], stack.out_s_B[l], t2),
                  f"layer {l}: out_proj y")
    last = stack.L - 1
    assert np.array_equal(x_out.view(np.uint32), _field(tr, last, "xn", np.float32).view(np.uint32)), "x_out"


def _run(stack, tokens=1, layers=None):
    import torch
    from bit_scaffold_int8_amd.runner import DeviceDecodeStack
    dev = DeviceDecodeStack(stack)
    x = torch.from_numpy(stack.x).cuda()
    x_out = torch.empty_like(x)
    conv, ssm = stack.conv_state, stack.ssm_state
    for tok in range(tokens):
        print(f"decode_layers: L={stack.L} token {tok}", flush=True)
        tr = dev.new_trace()
        dev.step(x, x_out, parity=tok % 2, trace=tr)
        torch.cuda.synchronize()
        assert int(dev.status.item()) == 0, f"status {int(dev.status.item())}"
        conv_out = dev.windows[1 - tok % 2].cpu().numpy()
        ssm_out = dev.ssm_state.cpu().numpy()
        _check_token(stack, tr.cpu().numpy(), x.cpu().numpy(), conv, ssm, conv_out, ssm_out, x_out.cpu().numpy(),
                     range(stack.L) if layers is None else layers)
        conv, ssm = conv_out, ssm_out
        x = x_out.clone()
    assert int(dev.workspace[DONE_WORD]) == 0, "the done count is left zeroed"
    assert int(dev.workspace[GEN_WORD]) == tokens, "the call counter advances once per call"
    return dev


def test_decode_layers_three_layers_two_tokens(torch_cuda):
    _run(si.draw_decode_stack(np.random.default_rng(11), 3), tokens=2)


def test_decode_layers_one_layer(torch_cuda):
    _run(si.draw_decode_stack(np.random.default_rng(12), 1), tokens=2)


def test_decode_layers_48_layers(torch_cuda):
    # the model's depth: every layer checked stage by stage
    _run(si.draw_decode_stack(np.random.default_rng(13), 48), tokens=1)


def test_decode_layers_end_to_end_against_chain_oracle(torch_cuda):
    # the whole chain in the oracle (fp64 step, rounded where a device holds fp32):
    # GPU and oracle only drift by the step's fp32 rounding and rare quantizer ties
    import torch
    from bit_scaffold_int8_amd.runner import DeviceDecodeStack
    st = si.draw_decode_stack(np.random.default_rng(14), 4)
    x_ref, _ = dc.decode_token(st, st.x, st.conv_state, st.ssm_state, nthreads=8)
    dev = DeviceDecodeStack(st)
    x = torch.from_numpy(st.x).cuda()
    x_out = torch.empty_like(x)
    dev.step(x, x_out)
    torch.cuda.synchronize()
    assert int(dev.status.item()) == 0
    got = x_out.cpu().numpy().astype(np.float64)
    assert np.abs(got - x_ref).max() <= 1e-3 * np.abs(x_ref).max()


def test_decode_layers_bounded_waits_end_the_kernel(torch_cuda):
    # every wait made unreachable from the host: each gives up after its poll limit,
    # the status says so, the kernel still ends, and the next normal call is correct
    import torch
    from bit_scaffold_int8_amd import dfssm
    from bit_scaffold_int8_amd.runner import DeviceDecodeStack
    st = si.draw_decode_stack(np.random.default_rng(15), 2)
    dev = DeviceDecodeStack(st)
    x = torch.from_numpy(st.x).cuda()
    x_out = torch.empty_like(x)
    # a copy of the state for the normal call after
    ssm0 = dev.ssm_state.clone()
    dev.step(x, x_out, spin_limit=64, flags=dfssm.DFSSM_DECODE_UNREACHABLE_WAITS)
    torch.cuda.synchronize()
    status = int(dev.status.item())
    assert status & dfssm.DFSSM_DECODE_STATUS_TIMEOUT, status
    assert int(dev.workspace[DONE_WORD]) == 0, "the done count is reset even after a failed call"
    assert int(dev.workspace[GEN_WORD]) == 1, "the failed call still advanced the call counter"
    dev.status.zero_()
    dev.ssm_state.copy_(ssm0)
    tr = dev.new_trace()
    dev.step(x, x_out, trace=tr)
    torch.cuda.synchronize()
    assert int(dev.status.item()) == 0
    _check_token(st, tr.cpu().numpy(), st.x, st.conv_state, st.ssm_state, dev.windows[1].cpu().numpy(),
                 dev.ssm_state.cpu().numpy(), x_out.cpu().numpy(), range(2))
