"""Compile the HIP sources under csrc/ into the in-tree shared library libdfssm.so (gfx950),
and the int8 MFMA rate probe (csrc/probe_mfma.hip) into libdfssm_probe.so, which only the
benchmark loads."""
from __future__ import annotations

import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libdfssm.so")
PROBE_LIB = os.path.join(PKG, "libdfssm_probe.so")
PROBE_SOURCES = ["probe_mfma.hip"]
SOURCES = ["api.hip", "quantize.hip", "lora_down.hip", "gemv.hip", "gemm_mfma.hip", "gemm_prefill.hip",
           "int8_head.hip", "mamba2_step.hip", "decode_layers.hip",
           "density_field.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # IEEE fp32 division (the quantizer's scale and codes depend on it); no fast-math
    "-fhip-fp32-correctly-rounded-divide-sqrt", "-fno-fast-math",
    # keep the compiler from forming packed fp32 ops
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
]


def build(verbose: bool = False) -> str:
    """Compile every source to an object in parallel, then link libdfssm.so."""
    from concurrent.futures import ThreadPoolExecutor
    objdir = os.path.join(PKG, "_build")
    os.makedirs(objdir, exist_ok=True)
    inc = ["-I", os.path.join(ROOT, "include"), "-I", CSRC]

    def compile_one(src):
        obj = os.path.join(objdir, src.replace(".hip", ".o"))
        cmd = [HIPCC, *FLAGS, "-c", *inc, os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
        return obj

    jobs = min(len(SOURCES) + len(PROBE_SOURCES), max(1, (os.cpu_count() or 1)))
    with ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(compile_one, SOURCES + PROBE_SOURCES))
    for lib, lib_objs in ((LIB, objs[:len(SOURCES)]), (PROBE_LIB, objs[len(SOURCES):])):
        link = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *lib_objs, "-o", lib + ".tmp"]
        subprocess.run(link, check=True)
        os.replace(lib + ".tmp", lib)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
