"""The no-allocation decode entry point (dfssm_decode_layers_noalloc) against the
workspace form (dfssm_decode_layers), through the C ABI.

Both run the same kernel; the only difference is where the done count, the call
counter and the tagged exchange slots live (the library's own per-GPU array instead of
the caller's workspace).  Two calls in a row on the library's array, the second with a
smaller stack (4 layers, then 2), must each reproduce the workspace form's outputs
byte for byte: the last layer's output, every layer's trace, the advanced windows and
the updated state, with a clear status word.  The second call also shows that what
the first left in the shared array (its done count cleared, its call counter
advanced, its tagged values) does not disturb the next.
"""
import numpy as np
import pytest

import synth_inputs as si
from test_gpu_parity import torch_cuda  # noqa: F401  (fixture)

pytestmark = pytest.mark.gpu


def _run_both(stack):
    import torch
    from bit_scaffold_int8_amd import dfssm
    from bit_scaffold_int8_amd.runner import DeviceDecodeStack
    outs = []
    for form in ("workspace", "noalloc"):
        d = DeviceDecodeStack(stack)       # fresh copies of the same weights and state
        x = torch.from_numpy(stack.x).cuda()
        x_out = torch.full_like(x, float("nan"))
        tr = d.new_trace()
        print(f"no-alloc: L={stack.L} form={form}", flush=True)
        if form == "workspace":
            d.step(x, x_out, parity=0, trace=tr)
        else:
            dfssm.dfssm_decode_layers_noalloc(d.weights, d.L, x, x_out, d.windows[0], d.windows[1], d.ssm_state,
                                              d.eps, d.status, tr)
        torch.cuda.synchronize()
        assert int(d.status.item()) == 0, (form, int(d.status.item()))
        outs.append({"x_out": x_out.cpu().numpy(), "trace": tr.cpu().numpy(), "conv": d.windows[1].cpu().numpy(),
                     "ssm": d.ssm_state.cpu().numpy()})
        del d
    return outs


def test_noalloc_matches_workspace_form_on_two_calls(torch_cuda):
    big = si.draw_decode_stack(np.random.default_rng(31), 4)
    small = si.draw_decode_stack(np.random.default_rng(32), 2)
    for stack in (big, small):
        a, b = _run_both(stack)
        for k in a:
            assert np.array_equal(a[k].view(np.uint8), b[k].view(np.uint8)), (stack.L, k)
        assert np.isfinite(a["x_out"]).all()


def test_noalloc_rejects_what_the_workspace_form_rejects(torch_cuda):
    from bit_scaffold_int8_amd import dfssm
    import ctypes
    w = dfssm.DecodeLayerWeights(*([0x10000] * len(dfssm.DECODE_WEIGHT_FIELDS)))
    A = 0x10000
    # more layers than the array covers, and no layers
    for n in (65, 0):
        assert dfssm.raw("dfssm_decode_layers_noalloc", ctypes.addressof(w), n, A, A, A, A + 0x1000000, A, 1e-5, A,
                         None, 0, 0, None) == dfssm.DFSSM_ERR_INVALID_ARG
