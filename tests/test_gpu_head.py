"""GPU parity of the int8 embedding / LM head against the CPU oracle.

The head takes the tokens' codes from the HIP quantizer (checked bit-exact against the
oracle's first), then: the int32 accumulators bit-exact, y within 1e-5 of the
magnitude D = |s_x s_e acc| of its one term (the kernel rounds twice in fp32 where the
oracle rounds once from fp64).  The lookup is one fp32 product per element: bit-exact.
"""
import numpy as np
import pytest

import oracle
import synth_inputs as si
from test_gpu_parity import torch_cuda  # noqa: F401  (fixture)

pytestmark = pytest.mark.gpu

REL_TOL = 1e-5


def _head_on_gpu(probs):
    import torch
    from bit_scaffold_int8_amd import dfssm
    B = len(probs)
    M, K = probs[0].x.shape
    N = probs[0].E.shape[0]
    x = torch.from_numpy(np.stack([p.x for p in probs])).cuda()
    e = torch.from_numpy(np.stack([p.E for p in probs])).cuda()
    s_e = torch.from_numpy(np.stack([p.s_e for p in probs])).cuda()
    x_q = torch.empty((B, M, K), dtype=torch.int8, device="cuda")
    s_x = torch.empty((B, M), dtype=torch.float32, device="cuda")
    y = torch.empty((B, M, N), dtype=torch.float32, device="cuda")
    acc = torch.empty((B, M, N), dtype=torch.int32, device="cuda")
    dfssm.dfssm_quantize_act(x.view(B * M, K), x_q.view(B * M, K), s_x.view(B * M))
    if B == 1:
        dfssm.dfssm_int8_rowscale_gemm(x_q[0], s_x[0], e[0], s_e[0], y[0], acc[0])
    else:
        dfssm.dfssm_int8_rowscale_gemm_strided_batched(x_q, s_x, e, s_e, y, acc)
    torch.cuda.synchronize()
    return x_q.cpu().numpy(), s_x.cpu().numpy(), y.cpu().numpy(), acc.cpu().numpy()


def _check(probs, nthreads=8):
    x_q, s_x, y, acc = _head_on_gpu(probs)
    for b, p in enumerate(probs):
        xq_ref, sx_ref = oracle.quantize_act(p.x)
        assert np.array_equal(x_q[b], xq_ref) and np.array_equal(s_x[b].view(np.uint32), sx_ref.view(np.uint32))
        y_ref, acc_ref = oracle.int8_rowscale_gemm(xq_ref, sx_ref, p.E, p.s_e, nthreads=nthreads)
        assert np.array_equal(acc[b], acc_ref), f"acc, problem {b}"
        D = np.abs(sx_ref.astype(np.float64)[:, None] * p.s_e.astype(np.float64)[None, :] * acc_ref.astype(np.float64))
        err = np.abs(y[b].astype(np.float64) - y_ref.astype(np.float64))
        bad = err > REL_TOL * D
        assert not bad.any(), f"problem {b}: {bad.sum()} outputs outside 1e-5 D, worst {(err / np.maximum(D, 1e-300)).max():.2e}"


@pytest.mark.parametrize("M", [1, 4, 16])
def test_lm_head_full_vocabulary(torch_cuda, M):
    # the model's head: 50280 rows of width 2048
    cfg = si.CONFIGS["lm_head_decode_v50280_d2048"]
    _check([si.make_head(M, 50280, 2048, seed=cfg["seed"] + M)], nthreads=16)


@pytest.mark.parametrize("M,N,K", [
    (1, 1, 16), (3, 17, 48), (2, 1000, 528), (5, 333, 1040), (16, 64, 4096), (1, 100, 4096), (7, 129, 256),
    (1, 4097, 512), (2, 61, 1024), (9, 200, 2064), (1, 300, 3072),
])
def test_lm_head_ragged_shapes(torch_cuda, M, N, K):
    _check([si.make_head(M, N, K, seed=M * 13 + N + K)])


def test_lm_head_batched(torch_cuda):
    rng = np.random.default_rng(9)
    _check([si.draw_head(rng, 2, 700, 2048) for _ in range(3)])


def test_lm_head_extreme_accumulators(torch_cuda):
    # every code +-127 against every weight +-127: |acc| = 127 * 127 * K
    p = si.make_head(2, 40, 4096, seed=3)
    p.x[:] = 1.0
    p.x[1] = -1.0
    p.E[:20] = 127
    p.E[20:] = -127
    _check([p])
    _, _, _, acc = _head_on_gpu([p])
    assert acc[0, 0, 0] == 127 * 127 * 4096 and acc[0, 1, 0] == -127 * 127 * 4096


def test_embedding_lookup_matches_oracle(torch_cuda):
    import torch
    from bit_scaffold_int8_amd import dfssm
    p = si.make_head(1, 5000, 2048, seed=17)
    ids = np.array([0, 4999, 123, 123, -1, 5000, 77, 1 << 30], np.int32)
    out = torch.empty((len(ids), 2048), dtype=torch.float32, device="cuda")
    dfssm.dfssm_embedding_lookup(torch.from_numpy(ids).cuda(), torch.from_numpy(p.E).cuda(),
                                 torch.from_numpy(p.s_e).cuda(), out)
    torch.cuda.synchronize()
    ref = oracle.embedding_lookup(ids, p.E, p.s_e)
    assert np.array_equal(out.cpu().numpy().view(np.uint32), ref.view(np.uint32))
