"""C ABI checks that need no GPU: the library loads, exports every declared symbol,
and rejects bad arguments on the host before anything is launched."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dfssm.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dfssm_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = _declared_functions()
    assert "dfssm_quantize_act" in names and "dfssm_scaffold_lora_gemm" in names


def test_library_exports_every_declared_symbol():
    from bit_scaffold_int8_amd import dfssm
    lib = ctypes.CDLL(dfssm.LIB_PATH)
    for name in _declared_functions():
        assert hasattr(lib, name), name
    assert set(_declared_functions()) == set(dfssm.EXPORTED)


def test_status_strings_and_version():
    from bit_scaffold_int8_amd import dfssm
    assert dfssm.status_string(0) == "DFSSM_OK"
    assert dfssm.status_string(1) == "DFSSM_ERR_INVALID_ARG"
    assert dfssm.status_string(2) == "DFSSM_ERR_UNSUPPORTED"
    assert dfssm.status_string(3) == "DFSSM_ERR_HIP"
    assert dfssm.dfssm_version() >= 100


# Fake, 16-byte aligned "device" addresses: validation must reject before any launch,
# so they are never dereferenced.
A = 0x10000


def _raw(name, *args):
    from bit_scaffold_int8_amd import dfssm
    return dfssm.raw(name, *args)


@pytest.mark.parametrize("args,want", [
    ((None, 1, 8, A, A), 1),           # NULL x
    ((A, 1, 8, None, A), 1),           # NULL x_q
    ((A, 1, 8, A, None), 1),           # NULL s_x
    ((A, 0, 8, A, A), 1),              # M = 0
    ((A, 1, 0, A, A), 1),              # K = 0
    ((A, -3, 8, A, A), 1),             # M < 0
    ((A + 2, 1, 8, A, A), 1),          # x not float-aligned
    ((A, 1, 8, A, A + 1), 1),          # s_x not float-aligned
])
def test_quantize_rejects(args, want):
    x, M, K, x_q, s_x = args
    assert _raw("dfssm_quantize_act", x, M, K, x_q, s_x, None) == want


@pytest.mark.parametrize("kw,want", [
    (dict(x_q=None), 1), (dict(w_b=None), 1), (dict(t=None), 1), (dict(M=0), 1), (dict(K=0), 1),
    (dict(x_q=A + 4), 1), (dict(w_b=A + 8), 1), (dict(t=A + 2), 1),
    (dict(rank=0), 2), (dict(rank=8), 2), (dict(K=131072 + 16), 2), (dict(batch=0), 1), (dict(batch=70000), 2),
])
def test_lora_down_rejects(kw, want):
    a = dict(x_q=A, M=1, K=64, w_b=A, rank=16, t=A, batch=1)
    a.update(kw)
    assert _raw("dfssm_lora_down_strided_batched", a["x_q"], a["M"], a["K"], a["w_b"], a["rank"], a["t"],
                a["batch"], None) == want


@pytest.mark.parametrize("kw,want", [
    (dict(x=None), 1), (dict(x_q=None), 1), (dict(s_x=None), 1), (dict(M=0), 1), (dict(K=0), 1),
    (dict(x=A + 4), 1), (dict(x_q=A + 4), 1), (dict(s_x=A + 2), 1),
    (dict(w_b=None), 1), (dict(t=None), 1), (dict(w_b=A + 8), 1), (dict(t=A + 1), 1),
    (dict(rank=4), 2), (dict(batch=0), 1), (dict(batch=65536), 2),
])
def test_quantize_lora_down_rejects(kw, want):
    a = dict(x=A, M=1, K=64, w_b=A, rank=16, x_q=A, s_x=A, t=A, batch=1)
    a.update(kw)
    assert _raw("dfssm_quantize_lora_down_strided_batched", a["x"], a["M"], a["K"], a["w_b"], a["rank"],
                a["x_q"], a["s_x"], a["t"], a["batch"], None) == want


def _gemm(**kw):
    """dfssm_scaffold_lora_gemm_strided_batched, the specified form (t computed inside)."""
    a = dict(x_q=A, s_x=A, M=1, N=16, K=64, w_bits=A, s_w=A, w_a=A, s_a=A, w_b=A, s_b=A, rank=16,
             y=A, acc_dbg=None, t_dbg=None, batch=1)
    a.update(kw)
    return _raw("dfssm_scaffold_lora_gemm_strided_batched", a["x_q"], a["s_x"], a["M"], a["N"], a["K"],
                a["w_bits"], a["s_w"], a["w_a"], a["s_a"], a["w_b"], a["s_b"], a["rank"], a["y"], a["acc_dbg"],
                a["t_dbg"], a["batch"], None)


def _gemm_given_t(**kw):
    a = dict(x_q=A, s_x=A, M=1, N=16, K=64, w_bits=A, s_w=A, w_a=A, s_a=A, s_b=A, t=A, rank=16,
             y=A, acc_dbg=None, batch=1)
    a.update(kw)
    return _raw("dfssm_scaffold_lora_gemm_given_t_strided_batched", a["x_q"], a["s_x"], a["M"], a["N"], a["K"],
                a["w_bits"], a["s_w"], a["w_a"], a["s_a"], a["s_b"], a["t"], a["rank"], a["y"], a["acc_dbg"],
                a["batch"], None)


_GEMM_COMMON_REJECTS = [
    (dict(x_q=None), 1), (dict(s_x=None), 1), (dict(w_bits=None), 1), (dict(s_w=None), 1),
    (dict(y=None), 1),
    (dict(M=0), 1), (dict(N=0), 1), (dict(K=0), 1), (dict(K=12), 1), (dict(K=-8), 1), (dict(batch=0), 1),
    (dict(w_a=None), 1), (dict(s_a=None), 1), (dict(s_b=None), 1),
    (dict(w_bits=A + 8), 1), (dict(x_q=A + 4), 1), (dict(w_a=A + 4), 1), (dict(y=A + 2), 1),
    (dict(acc_dbg=A + 2), 1), (dict(s_w=A + 1), 1),
    (dict(rank=8), 2), (dict(rank=32), 2), (dict(rank=-1), 2),
    (dict(K=131072 + 8), 2), (dict(batch=65536), 2),
]


@pytest.mark.parametrize("kw,want", _GEMM_COMMON_REJECTS + [
    (dict(w_b=None), 1), (dict(w_b=A + 8), 1), (dict(t_dbg=A + 2), 1),
])
def test_gemm_rejects(kw, want):
    assert _gemm(**kw) == want


@pytest.mark.parametrize("kw,want", _GEMM_COMMON_REJECTS + [(dict(t=None), 1), (dict(t=A + 1), 1)])
def test_gemm_given_t_rejects(kw, want):
    assert _gemm_given_t(**kw) == want


def test_gemm_rank_zero_needs_no_lora_operands():
    # rank 0: every LoRA pointer may be NULL; validation passes, so only a launch could
    # fail -- checked here on the host path by a size error after the LoRA checks
    assert _gemm(rank=0, w_a=None, s_a=None, w_b=None, s_b=None, K=12) == 1
    assert _gemm_given_t(rank=0, w_a=None, s_a=None, s_b=None, t=None, K=12) == 1


def test_single_problem_gemm_rejects_like_batched():
    # dfssm_scaffold_lora_gemm(x_q, s_x, M, N, K, w_bits, s_w, w_a, s_a, w_b, s_b, rank, y, acc_dbg, t_dbg, stream)
    assert _raw("dfssm_scaffold_lora_gemm", A, A, 1, 16, 12, A, A, A, A, A, A, 16, A, None, None, None) == 1
    assert _raw("dfssm_scaffold_lora_gemm", A, A, 1, 16, 64, A, A, A, A, A, A, 8, A, None, None, None) == 2
    assert _raw("dfssm_scaffold_lora_gemm", A, A, 1, 16, 64, A, A, A, A, None, A, 16, A, None, None, None) == 1
    assert _raw("dfssm_scaffold_lora_gemm", A, A, 1, 16, 64, A, A, A, A, A, A, 16, A, None, A + 2, None) == 1
    assert _raw("dfssm_scaffold_lora_gemm_given_t", A, A, 1, 16, 12, A, A, A, A, A, A, 16, A, None, None) == 1
    assert _raw("dfssm_scaffold_lora_gemm_given_t", A, A, 1, 16, 64, A, A, A, A, A, None, 16, A, None, None) == 1
    assert _raw("dfssm_lora_down", A, 1, 64, A, 0, A, None) == 2
    assert _raw("dfssm_quantize_lora_down", A, 1, 64, None, 16, A, A, A, None) == 1


def _forward(**kw):
    a = dict(x=A, M=1, N=16, K=128, w_bits=A, s_w=A, w_a=A, s_a=A, w_b=A, s_b=A, rank=16, x_q=A, s_x=A, t=A,
             y=A, acc_dbg=None, batch=1)
    a.update(kw)
    return _raw("dfssm_scaffold_lora_forward_strided_batched", a["x"], a["M"], a["N"], a["K"], a["w_bits"],
                a["s_w"], a["w_a"], a["s_a"], a["w_b"], a["s_b"], a["rank"], a["x_q"], a["s_x"], a["t"], a["y"],
                a["acc_dbg"], a["batch"], None)


@pytest.mark.parametrize("kw,want", [
    (dict(x=None), 1), (dict(x_q=None), 1), (dict(s_x=None), 1), (dict(w_bits=None), 1), (dict(s_w=None), 1),
    (dict(y=None), 1), (dict(w_a=None), 1), (dict(s_a=None), 1), (dict(w_b=None), 1), (dict(s_b=None), 1),
    (dict(t=None), 1),
    (dict(M=0), 1), (dict(N=0), 1), (dict(K=0), 1), (dict(K=12), 1), (dict(batch=0), 1),
    (dict(x=A + 4), 1), (dict(x_q=A + 4), 1), (dict(w_bits=A + 8), 1), (dict(w_a=A + 4), 1),
    (dict(w_b=A + 8), 1), (dict(s_x=A + 2), 1), (dict(t=A + 1), 1), (dict(y=A + 2), 1), (dict(acc_dbg=A + 2), 1),
    (dict(rank=8), 2), (dict(K=131072 + 8), 2), (dict(batch=65536), 2),
])
def test_forward_rejects(kw, want):
    # the one-call form checks everything both calls of the two-call form check
    assert _forward(**kw) == want


def test_single_problem_forward_rejects_like_batched():
    assert _raw("dfssm_scaffold_lora_forward", A, 1, 16, 12, A, A, A, A, A, A, 16, A, A, A, A, None, None) == 1
    assert _raw("dfssm_scaffold_lora_forward", A, 1, 16, 128, A, A, A, A, A, A, 8, A, A, A, A, None, None) == 2


def _head(**kw):
    a = dict(x_q=A, s_x=A, M=1, N=16, K=64, e=A, s_e=A, y=A, acc_dbg=None, batch=1)
    a.update(kw)
    return _raw("dfssm_int8_rowscale_gemm_strided_batched", a["x_q"], a["s_x"], a["M"], a["N"], a["K"], a["e"],
                a["s_e"], a["y"], a["acc_dbg"], a["batch"], None)


@pytest.mark.parametrize("kw,want", [
    (dict(x_q=None), 1), (dict(s_x=None), 1), (dict(e=None), 1), (dict(s_e=None), 1), (dict(y=None), 1),
    (dict(M=0), 1), (dict(N=0), 1), (dict(K=0), 1), (dict(K=24), 1), (dict(batch=0), 1),
    (dict(x_q=A + 8), 1), (dict(e=A + 4), 1), (dict(s_x=A + 2), 1), (dict(s_e=A + 1), 1), (dict(y=A + 2), 1),
    (dict(acc_dbg=A + 2), 1),
    (dict(M=17), 2), (dict(K=4096 + 16), 2), (dict(N=1 << 20, K=4096), 2), (dict(batch=65536), 2),
])
def test_int8_head_rejects(kw, want):
    assert _head(**kw) == want


@pytest.mark.parametrize("args,want", [
    ((None, 1, A, A, 10, 8, A), 1), ((A, 1, None, A, 10, 8, A), 1), ((A, 1, A, None, 10, 8, A), 1),
    ((A, 1, A, A, 10, 8, None), 1), ((A, 0, A, A, 10, 8, A), 1), ((A, 1, A, A, 0, 8, A), 1),
    ((A, 1, A, A, 10, 0, A), 1), ((A + 2, 1, A, A, 10, 8, A), 1), ((A, 1, A, A + 2, 10, 8, A), 1),
    ((A, 1, A, A, 10, 8, A + 1), 1),
])
def test_embedding_lookup_rejects(args, want):
    assert _raw("dfssm_embedding_lookup", *args, None) == want


def _mamba2(**kw):
    far = 0x10000000  # distinct fake buffers far apart, so only the cases below overlap
    a = dict(zxbcdt=A + 3 * far, S=1, nheads=64, headdim=64, d_state=128, conv_in=A, conv_out=A + far,
             ssm=A, conv_w=A, conv_b=A, dt_bias=A, A_log=A, D=A, norm_w=A, eps=1e-5, out=A + 2 * far)
    a.update(kw)
    return _raw("dfssm_mamba2_decode_step", a["zxbcdt"], a["S"], a["nheads"], a["headdim"], a["d_state"],
                a["conv_in"], a["conv_out"], a["ssm"], a["conv_w"], a["conv_b"], a["dt_bias"], a["A_log"], a["D"],
                a["norm_w"], a["eps"], a["out"], None)


@pytest.mark.parametrize("kw,want", [
    (dict(zxbcdt=None), 1), (dict(conv_in=None), 1), (dict(conv_out=None), 1), (dict(ssm=None), 1),
    (dict(conv_w=None), 1), (dict(conv_b=None), 1), (dict(dt_bias=None), 1), (dict(A_log=None), 1),
    (dict(D=None), 1), (dict(norm_w=None), 1), (dict(out=None), 1),
    (dict(S=0), 1), (dict(S=65536), 1), (dict(nheads=0), 1), (dict(headdim=0), 1), (dict(d_state=-1), 1),
    (dict(eps=-1.0), 1), (dict(eps=float("nan")), 1), (dict(eps=float("inf")), 1),
    (dict(conv_in=A + 4), 1), (dict(conv_out=A + 0x10000000 + 8), 1), (dict(ssm=A + 4), 1), (dict(conv_w=A + 4), 1),
    (dict(norm_w=A + 8), 1), (dict(out=A + 0x20000000 + 4), 1), (dict(zxbcdt=A + 2), 1), (dict(conv_b=A + 1), 1),
    (dict(dt_bias=A + 2), 1), (dict(A_log=A + 2), 1), (dict(D=A + 2), 1),
    (dict(conv_out=A), 1),                      # windows in and out overlap
    (dict(conv_out=A + 4352 * 16 - 16), 1),     # ... by one window
    (dict(out=A + 3 * 0x10000000 + 64), 1),     # out overlaps the in_proj output
    (dict(headdim=32), 2), (dict(d_state=64), 2), (dict(nheads=1025), 2),
])
def test_mamba2_step_rejects(kw, want):
    assert _mamba2(**kw) == want


# ---- the prefill planner (host only)

def test_prefill_plan_keeps_the_measured_choices():
    from bit_scaffold_int8_amd import dfssm
    # plans chosen by timing them against each other on an MI355X: in_proj M2048 on
    # 128x256 tiles at two groups per CU with a 64x64 split-K tail (43.4 us against 46.5
    # for one 8-wave group per CU plus a tail round); out_proj on 128x128 split-K; at
    # M4096 and at batch 4 one 8-wave group per CU with a 64x128 split-K tail (88.2 and
    # 187.0 us, against 93.3 and 189.6 for two groups per CU)
    assert dfssm.dfssm_prefill_plan(2048, 8512, 2048) == (7, 8, 8192)
    assert dfssm.dfssm_prefill_plan(2048, 2048, 4096) == (4, -1, 2048)
    assert dfssm.dfssm_prefill_plan(4096, 8512, 2048) == (3, 5, 8192)
    assert dfssm.dfssm_prefill_plan(2048, 8512, 2048, 4) == (3, 5, 8192)


# column width of each configuration and the tails it is built with (the header's list)
_PF_BN = {0: 512, 1: 128, 2: 64, 3: 512, 4: 128, 5: 128, 6: 64, 7: 256, 8: 64}
_PF_TAILS = {0: (1, 2), 1: (2,), 2: (), 3: (5, 6), 4: (5, 6), 5: (6,), 6: (), 7: (8,), 8: ()}


@pytest.mark.parametrize("M", [17, 100, 128, 300, 512, 2048, 4096])
@pytest.mark.parametrize("N,K", [(1, 64), (70, 192), (513, 1024), (2048, 4096), (8512, 2048), (8704, 2048)])
@pytest.mark.parametrize("batch", [1, 3])
def test_prefill_plan_is_consistent(M, N, K, batch):
    from bit_scaffold_int8_amd import dfssm
    mc, tc, ns = dfssm.dfssm_prefill_plan(M, N, K, batch)
    assert mc in _PF_BN
    if tc < 0:
        assert ns == N
    else:
        assert tc in _PF_TAILS[mc]              # a tail the main configuration is built with
        assert 0 < ns < N and ns % _PF_BN[mc] == 0
        assert _PF_BN[tc] < _PF_BN[mc]


def test_prefill_plan_rejects():
    from bit_scaffold_int8_amd import dfssm
    U, I = dfssm.DFSSM_ERR_UNSUPPORTED, dfssm.DFSSM_ERR_INVALID_ARG
    for args, want in [((16, 512, 2048, 1), U),      # the decode kernel's shape
                       ((2048, 512, 808, 1), U),     # K % 64 != 0: the generic kernel
                       ((2048, 512, 804, 1), I),     # K % 8 != 0
                       ((0, 512, 2048, 1), I), ((2048, 0, 2048, 1), I), ((2048, 512, 2048, 0), I)]:
        with pytest.raises(dfssm.DfssmError) as e:
            dfssm.dfssm_prefill_plan(*args)
        assert e.value.status == want, args
    assert dfssm.lib.dfssm_prefill_plan(2048, 512, 2048, 1, None, None, None) == I


# ---- the density-field codec and the one-launch decode (host-side checks only)

@pytest.mark.parametrize("args,want", [
    ((None, 10, 128, A, A), 1), ((A, 10, 128, None, A), 1), ((A, 10, 128, A, None), 1),
    ((A, 0, 128, A, A), 1), ((A, 10, 0, A, A), 1), ((A, 10, 100, A, A), 2), ((A, 10, 512, A, A), 2),
    ((A + 4, 10, 128, A, A), 1), ((A, 10, 128, A + 8, A), 1), ((A, 10, 128, A, A + 2), 1),
    ((A, 1 << 34, 128, A, A), 1),
])
def test_density_encode_rejects(args, want):
    assert _raw("dfssm_density_field_encode", *args, None) == want


def test_density_decode_and_requantize_reject():
    assert _raw("dfssm_density_field_decode", None, A, 10, 128, A, None) == 1
    assert _raw("dfssm_density_field_decode", A, A, 10, 96, A, None) == 2
    assert _raw("dfssm_density_field_decode", A, A, 10, 128, A + 4, None) == 1
    assert _raw("dfssm_density_field_requantize", None, 10, 128, None, None, None) == 1
    assert _raw("dfssm_density_field_requantize", A, 10, 32, None, None, None) == 2
    assert _raw("dfssm_density_field_requantize", A + 8, 10, 128, None, None, None) == 1


def _decode_layers(**kw):
    import ctypes
    from bit_scaffold_int8_amd import dfssm
    far = 0x10000000
    fields = {name: A for name in dfssm.DECODE_WEIGHT_FIELDS}
    fields.update(kw.pop("weights", {}))
    w = dfssm.DecodeLayerWeights(*[fields[n] for n in dfssm.DECODE_WEIGHT_FIELDS])
    a = dict(L=2, x_in=A, x_out=A, conv_in=A, conv_out=A + far, ssm=A, eps=1e-5, ws=A,
             ws_bytes=dfssm.dfssm_decode_layers_workspace_bytes(), status=A, trace=None, spin=0, flags=0)
    a.update(kw)
    return dfssm.raw("dfssm_decode_layers", None if a.get("null_w") else ctypes.addressof(w), a["L"], a["x_in"],
                     a["x_out"], a["conv_in"], a["conv_out"], a["ssm"], a["eps"], a["ws"], a["ws_bytes"], a["status"],
                     a["trace"], a["spin"], a["flags"], None)


@pytest.mark.parametrize("kw,want", [
    (dict(null_w=True), 1), (dict(weights={"in_w_bits": None}), 1), (dict(weights={"norm_w": A + 4}), 1),
    (dict(weights={"out_s_b": A + 2}), 1), (dict(L=0), 1), (dict(L=65), 1), (dict(x_in=None), 1),
    (dict(x_in=A + 4), 1), (dict(ssm=None), 1), (dict(ssm=A + 8), 1), (dict(ws=None), 1), (dict(ws=A + 8), 1),
    (dict(ws_bytes=64), 1), (dict(status=None), 1), (dict(status=A + 1), 1), (dict(trace=A + 2), 1),
    (dict(eps=-1.0), 1), (dict(eps=float("nan")), 1), (dict(flags=2), 1),
    (dict(conv_out=A), 1), (dict(conv_out=A + 4352 * 16), 1),       # the windows overlap (2 layers)
])
def test_decode_layers_rejects(kw, want):
    assert _decode_layers(**kw) == want


def test_binding_shares_torchs_hip_runtime():
    # importing the binding before torch must leave one HIP runtime in the process (two
    # would make torch's device pointers invalid in the library's launches)
    import subprocess
    import sys
    code = ("import bit_scaffold_int8_amd.dfssm, torch; "
            "paths = {l.split()[-1] for l in open('/proc/self/maps') if 'libamdhip64' in l}; print(len(paths))")
    out = subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True, timeout=600)
    assert out.returncode == 0, out.stderr[-2000:]
    assert out.stdout.strip() == "1", out.stdout
