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


@pytest.mark.parametrize("args,want", [
    ((None, 1, 8, A, A), 1),           # NULL x
    ((A, 1, 8, None, A), 1),           # NULL x_q
    ((A, 1, 8, A, None), 1),           # NULL s_x
    ((A, 0, 8, A, A), 1),              # M = 0
    ((A, 1, 0, A, A), 1),              # K = 0
    ((A, -3, 8, A, A), 1),             # M < 0
    ((A + 4, 1, 8, A, A), 1),          # misaligned x
    ((A, 1, 8, A + 1, A), 1),          # misaligned x_q
])
def test_quantize_rejects(args, want):
    from bit_scaffold_int8_amd import dfssm
    x, M, K, x_q, s_x = args
    assert dfssm.raw_quantize_act(x, M, K, x_q, s_x, None) == want


def _gemm(**kw):
    from bit_scaffold_int8_amd import dfssm
    a = dict(x_q=A, s_x=A, M=1, N=16, K=64, w_bits=A, s_w=A, w_a=A, s_a=A, w_b=A, s_b=A, rank=16,
             y=A, t=A, acc_dbg=None, stream=None)
    a.update(kw)
    return dfssm.raw_scaffold_lora_gemm(**a)


@pytest.mark.parametrize("kw,want", [
    (dict(x_q=None), 1), (dict(s_x=None), 1), (dict(w_bits=None), 1), (dict(s_w=None), 1),
    (dict(y=None), 1),
    (dict(M=0), 1), (dict(N=0), 1), (dict(K=0), 1), (dict(K=12), 1), (dict(K=-8), 1),
    (dict(w_a=None), 1), (dict(s_a=None), 1), (dict(w_b=None), 1), (dict(s_b=None), 1), (dict(t=None), 1),
    (dict(w_bits=A + 8), 1), (dict(y=A + 4), 1), (dict(acc_dbg=A + 2), 1), (dict(t=A + 4), 1),
    (dict(rank=8), 2), (dict(rank=32), 2), (dict(rank=-1), 2),
    (dict(K=131072 + 8), 2),
])
def test_gemm_rejects(kw, want):
    assert _gemm(**kw) == want
