"""GPU parity of the density-field codec (dfssm_density_field_*) against the CPU oracle.

The codec decides integers (cells) in fp32, and both sides take every decision in the
same fp32 arithmetic (one IEEE division, an add and an exact halving per value, then
the modulator's add, compare and exact subtraction per cell): the field and the scale
must be bit-exact, and so must the readout (a product of the scale with -1, -1/2, 0,
1/2 or 1).
"""
import numpy as np
import pytest

from oracle import density_field as dfc
from test_gpu_parity import torch_cuda  # noqa: F401  (fixture)

pytestmark = pytest.mark.gpu


def _rows(R, d, seed):
    rng = np.random.default_rng(seed)
    x = (0.1 * rng.standard_normal((R, d))).astype(np.float32)
    x *= rng.uniform(1e-3, 1e2, (R, 1)).astype(np.float32)
    if R > 4:
        x[0] = 0.0                                   # all-zero row
        x[1] = 2.5                                   # constant row
        x[2] = np.where(np.arange(d) % 3 == 0, -1.0, 0.25).astype(np.float32)
        k = rng.integers(0, 65, d)                   # dyadic densities: many exact 1/2 ties
        x[3] = ((2 * k - 64) / 64.0).astype(np.float32)
        x[3, 0] = 1.0
    return x


def _gpu(x, mode):
    import torch
    from bit_scaffold_int8_amd import dfssm
    R, d = x.shape
    xs = torch.from_numpy(x).cuda()
    field = torch.full((R, d // 8), 0xAB, dtype=torch.int32, device="cuda")
    scale = torch.full((R,), float("nan"), dtype=torch.float32, device="cuda")
    out = torch.full_like(xs, float("nan"))
    if mode == "encode_decode":
        dfssm.dfssm_density_field_encode(xs, field, scale)
        dfssm.dfssm_density_field_decode(field, scale, out)
    else:
        out.copy_(xs)
        dfssm.dfssm_density_field_requantize(out, field, scale)
    torch.cuda.synchronize()
    return field.cpu().numpy().view(np.uint32), scale.cpu().numpy(), out.cpu().numpy()


@pytest.mark.parametrize("mode", ["encode_decode", "requantize"])
@pytest.mark.parametrize("R,d", [(1, 128), (63, 128), (64, 128), (65, 128), (1000, 128), (257, 64), (130, 256),
                                 (4096, 128)])
def test_density_field_matches_oracle(torch_cuda, mode, R, d):
    x = _rows(R, d, R * 7 + d)
    f_ref, s_ref = dfc.encode(x)
    v_ref = dfc.decode(f_ref, s_ref, d)
    f, s, v = _gpu(x, mode)
    assert np.array_equal(s.view(np.uint32), s_ref.view(np.uint32)), "scale"
    assert np.array_equal(f, f_ref), f"field: {(f != f_ref).sum()} words differ"
    assert np.array_equal(v.view(np.uint32), v_ref.view(np.uint32)), "readout"


def test_density_field_requantize_without_field_outputs(torch_cuda):
    import torch
    from bit_scaffold_int8_amd import dfssm
    x = _rows(300, 128, 5)
    v_ref, _, _ = dfc.requantize(x)
    xs = torch.from_numpy(x).cuda()
    dfssm.dfssm_density_field_requantize(xs)
    torch.cuda.synchronize()
    assert np.array_equal(xs.cpu().numpy().view(np.uint32), v_ref.view(np.uint32))


def test_density_field_full_decode_batch(torch_cuda):
    # one layer's SSM state for 64 sequences: 64 x 64 heads x 64 channels rows of 128
    # (the bench's size); checked on 2000 rows drawn over the whole range
    import torch
    from bit_scaffold_int8_amd import dfssm
    R, d = 64 * 64 * 64, 128
    rng = np.random.default_rng(77)
    x = (0.1 * rng.standard_normal((R, d))).astype(np.float32)
    xs = torch.from_numpy(x).cuda()
    field = torch.empty((R, d // 8), dtype=torch.int32, device="cuda")
    scale = torch.empty((R,), dtype=torch.float32, device="cuda")
    out = torch.empty_like(xs)
    dfssm.dfssm_density_field_encode(xs, field, scale)
    dfssm.dfssm_density_field_decode(field, scale, out)
    torch.cuda.synchronize()
    idx = np.unique(np.concatenate([rng.integers(0, R, 2000), [0, R - 1, 63, 64]]))
    f_ref, s_ref = dfc.encode(x[idx])
    assert np.array_equal(field.cpu().numpy().view(np.uint32)[idx], f_ref)
    assert np.array_equal(scale.cpu().numpy()[idx].view(np.uint32), s_ref.view(np.uint32))
    assert np.array_equal(out.cpu().numpy()[idx].view(np.uint32), dfc.decode(f_ref, s_ref, d).view(np.uint32))


def test_density_field_scales_across_the_fp32_range(torch_cuda):
    # Row scales over the whole fp32 range: subnormal, tiny, normal, huge (up to the
    # largest finite value) and infinite.  Within a row: the scale itself, values just
    # below it, all-ones significands, values far below it (quotients that underflow)
    # and exact dyadic ratios.  The encode forms v / s through a power-of-two scaling
    # and a correction step; field, scale and readout must still be bit-exact.
    rng = np.random.default_rng(11)
    d = 128
    rows = []
    for e in list(range(-149, 128, 2)) + [127]:
        m = np.float32(1) + rng.random(dtype=np.float32)
        if e == 127:
            m = np.float32(np.nextafter(np.float32(2), np.float32(0)))  # the largest finite scale
        s = np.ldexp(m, e).astype(np.float32)
        if not np.isfinite(s) or s == 0:
            continue
        frac = rng.uniform(-1, 1, d).astype(np.float32)
        v = (s * frac).astype(np.float32)
        v[0] = s
        v[1] = -np.nextafter(s, np.float32(0))
        v[2] = np.float32(np.uint32((s.view(np.uint32) & 0xFF800000) | 0x7FFFFF).view(np.float32))
        v[3:11] = np.ldexp(np.float32(1) + rng.random(8, dtype=np.float32), e - rng.integers(20, 160, 8)).astype(np.float32)
        v[11:19] = (s * (rng.integers(-64, 65, 8) / np.float32(64))).astype(np.float32)
        v = np.clip(v, -s, s).astype(np.float32)
        rows.append(v)
    inf_row = rng.uniform(-1e3, 1e3, d).astype(np.float32)
    inf_row[5] = np.inf
    ninf_row = inf_row.copy()
    ninf_row[5] = -np.inf
    x = np.stack(rows + [inf_row, ninf_row, np.zeros(d, np.float32)]).astype(np.float32)
    f_ref, s_ref = dfc.encode(x)
    with np.errstate(invalid="ignore"):  # the infinite rows read out inf * 0 = NaN
        v_ref = dfc.decode(f_ref, s_ref, d)
    for mode in ("encode_decode", "requantize"):
        f, s, v = _gpu(x, mode)
        assert np.array_equal(s.view(np.uint32), s_ref.view(np.uint32)), f"{mode}: scale"
        bad = np.nonzero((f != f_ref).any(axis=1))[0]
        assert bad.size == 0, f"{mode}: field differs in rows {bad[:8]} (scales {s_ref[bad[:8]]})"
        assert np.array_equal(v.view(np.uint32), v_ref.view(np.uint32)), f"{mode}: readout"
