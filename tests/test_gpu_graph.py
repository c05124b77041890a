"""The entry points inside captured HIP graphs, replayed several times, and on two
streams at once.

The library's calls are asynchronous on the caller's stream and allocate nothing, so
a caller can capture them; decode runs them that way (the whole per-token sequence in
one graph).  Each test captures a sequence once, then replays it several times with
the program's own eager work and synchronizations between the replays (outputs
overwritten, other calls on other buffers), and checks every replay bit for bit
against the same calls made eagerly.  Graph and eager runs use the same kernels on
the same inputs, so the results must be identical, not merely close.
"""
import numpy as np
import pytest

import synth_inputs as si
from test_gpu_parity import torch_cuda  # noqa: F401  (fixture)

pytestmark = pytest.mark.gpu

REPLAYS = 4


def _capture(torch, fn):
    """Warm up fn on a side stream, then capture it into a graph on that stream."""
    cs = torch.cuda.Stream()
    with torch.cuda.stream(cs):
        fn(cs)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=cs):
        fn(torch.cuda.current_stream())
    torch.cuda.synchronize()
    return g


def _projection_outputs(dp):
    return [dp.x_q.clone(), dp.s_x.clone(), dp.t.clone(), dp.y.clone()]


def _scribble(dp):
    # overwrite every output between replays, eagerly, so a replay that skipped or
    # half-did its work cannot pass on the previous replay's values
    dp.x_q.fill_(77)
    dp.s_x.fill_(float("nan"))
    dp.t.fill_(-5)
    dp.y.fill_(float("nan"))


@pytest.mark.parametrize("form", ["one_call", "two_call"])
@pytest.mark.parametrize("M,N,K,B", [(1, 2048, 4096, 3), (1, 8512, 2048, 2), (4, 333, 512, 2), (130, 700, 1024, 1)])
def test_projection_graph_replays_match_eager(torch_cuda, form, M, N, K, B):
    import torch
    from bit_scaffold_int8_amd.runner import DeviceProjections
    probs = [si.make_problem(M, N, K, 2, seed=300 + 7 * b + M) for b in range(B)]
    dp = DeviceProjections.from_problems(probs, device="cuda")
    other = DeviceProjections.from_problems([si.make_problem(M, N, K, 2, seed=999)], device="cuda")
    run = (lambda s: dp.forward_one_call(s, debug=False)) if form == "one_call" else \
        (lambda s: dp.forward(s, debug=False))
    run(torch.cuda.current_stream())
    torch.cuda.synchronize()
    want = _projection_outputs(dp)
    g = _capture(torch, run)
    for r in range(REPLAYS):
        _scribble(dp)
        other.forward_one_call(debug=False)   # the program's own eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, got, ref in zip(("x_q", "s_x", "t", "y"), _projection_outputs(dp), want):
            assert torch.equal(got.view(torch.int8) if got.dtype == torch.int8 else got.view(torch.int32),
                               ref.view(torch.int8) if ref.dtype == torch.int8 else ref.view(torch.int32)), \
                f"replay {r}: {name} differs from the eager result"


def test_prefill_gemm_graph_replays_match_eager(torch_cuda):
    import torch
    from bit_scaffold_int8_amd.runner import DeviceProjections
    dp = DeviceProjections.from_problems([si.make_problem(300, 1000, 2112, 3, seed=41)], device="cuda",
                                         with_acc=True)
    dp.quantize_lora_down()
    torch.cuda.synchronize()
    dp.gemm(debug=True)
    torch.cuda.synchronize()
    want_y, want_acc = dp.y.clone(), dp.acc_dbg.clone()
    g = _capture(torch, lambda s: dp.gemm(s, debug=True))
    for r in range(REPLAYS):
        dp.y.fill_(float("nan"))
        dp.acc_dbg.fill_(12345)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(dp.acc_dbg, want_acc), f"replay {r}: acc"
        assert torch.equal(dp.y.view(torch.int32), want_y.view(torch.int32)), f"replay {r}: y"


def test_mamba2_step_graph_replays_match_eager(torch_cuda):
    # two steps per replay (the windows ping-pong, the state is updated in place): the
    # graph's state after each replay must equal an eager run of as many steps
    import torch
    from bit_scaffold_int8_amd.runner import DeviceMamba2Layer
    rng = np.random.default_rng(77)
    layer = si.draw_mamba2_layer(rng, nheads=6)
    zx, conv, ssm = si.draw_mamba2_inputs(rng, 3, nheads=6)
    zxd = torch.from_numpy(zx).cuda()
    graph_side = DeviceMamba2Layer.from_host(layer, conv, ssm, device="cuda")
    eager_side = DeviceMamba2Layer.from_host(layer, conv, ssm, device="cuda")

    def two_steps(m, s):
        m.step(zxd, 0, s)
        m.step(zxd, 1, s)

    g = _capture(torch, lambda s: two_steps(graph_side, s))   # the warm-up ran two steps
    two_steps(eager_side, torch.cuda.current_stream())         # keep the eager side level
    torch.cuda.synchronize()
    for r in range(REPLAYS):
        graph_side.out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        two_steps(eager_side, torch.cuda.current_stream())
        torch.cuda.synchronize()
        assert torch.equal(graph_side.ssm_state.view(torch.int32), eager_side.ssm_state.view(torch.int32)), \
            f"replay {r}: state"
        assert torch.equal(graph_side.windows[0].view(torch.int32), eager_side.windows[0].view(torch.int32)), \
            f"replay {r}: window"
        assert torch.equal(graph_side.out.view(torch.int32), eager_side.out.view(torch.int32)), f"replay {r}: out"


def test_calls_on_two_streams_at_once_match_sequential(torch_cuda):
    # the library keeps no per-call state on the device: calls on two streams (default
    # priority) may run at the same time, each on its own buffers, and give what the
    # same calls give one after another
    import torch
    from bit_scaffold_int8_amd.runner import DeviceProjections
    a = DeviceProjections.from_problems([si.make_problem(1, 2048, 4096, 2, seed=500 + b) for b in range(4)],
                                        device="cuda")
    b = DeviceProjections.from_problems([si.make_problem(2, 8512, 2048, 2, seed=600 + j) for j in range(2)],
                                        device="cuda")
    c = DeviceProjections.from_problems([si.make_problem(200, 700, 1024, 3, seed=700)], device="cuda")
    for p in (a, b, c):
        p.forward_one_call(debug=False)
    torch.cuda.synchronize()
    want = [p.y.clone() for p in (a, b, c)]
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    for r in range(3):
        for p in (a, b, c):
            p.y.fill_(float("nan"))
        torch.cuda.synchronize()
        for _ in range(2):   # interleaved launches on both streams
            a.forward_one_call(s1, debug=False)
            b.forward_one_call(s2, debug=False)
            c.forward(s1, debug=False)
        torch.cuda.synchronize()
        for name, p, w in zip("abc", (a, b, c), want):
            assert torch.equal(p.y.view(torch.int32), w.view(torch.int32)), f"round {r}: {name} differs"
