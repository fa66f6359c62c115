"""Compile the HIP sources of libtq for gfx950 into an in-tree shared library.

Run as ``python bit_quantized_matvec_amd/build.py`` (it does not import the
package, whose import loads the library).  Always recompiles.
Every HIP translation unit is built with packed FP32 instructions disabled and
without fast-math (the q8_K quantizer relies on IEEE division and rounding).
"""
from __future__ import annotations

import os
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libtq.so")
# measurement kernels of the benchmark (HBM read ceiling, shader clock), kept
# out of the product library
PROBE_LIB = os.path.join(HERE, "libtq_probe.so")
PROBE_SOURCES = ["hbm_probe.hip"]
ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SOURCES = ["tq_api.cpp", "k_workspace.hip", "scratch.hip", "k_quant.hip", "k_repack.hip", "k_gemv_pq2.hip", "k_gemm_pq2.hip", "k_gemv_ptq1.hip", "k_gemm_ptq1.hip"]
FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fno-fast-math", "-ffp-contract=off",
    "-Wall", "-Wno-unused-function",
]
# Per-source extras: the MFMA kernels keep their accumulators in ordinary
# VGPRs, so the epilogues read them without v_accvgpr_read copies.
EXTRA = {"k_gemm_pq2.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
         "k_gemm_ptq1.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def _compile(src: str, out: str, extra=()) -> None:
    cmd = [HIPCC, *FLAGS, *extra, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-fp32 feature and says so: harmless.
    err = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{err}")
    if err.strip():
        sys.stderr.write(err + "\n")


def build(verbose: bool = False) -> str:
    with tempfile.TemporaryDirectory() as tmp:
        objs = [os.path.join(tmp, s + ".o") for s in SOURCES]
        with ThreadPoolExecutor(min(len(SOURCES), os.cpu_count() or 4)) as ex:
            list(ex.map(lambda a: _compile(a[0], a[1], EXTRA.get(a[0], ())), zip(SOURCES, objs)))
        tmp_lib = LIB + ".tmp"
        subprocess.check_call([HIPCC, "-shared", f"--offload-arch={ARCH}", *objs, "-o", tmp_lib])
        os.replace(tmp_lib, LIB)
        pobjs = [os.path.join(tmp, s + ".o") for s in PROBE_SOURCES]
        for src, obj in zip(PROBE_SOURCES, pobjs):
            _compile(src, obj)
        tmp_lib = PROBE_LIB + ".tmp"
        subprocess.check_call([HIPCC, "-shared", f"--offload-arch={ARCH}", *pobjs, "-o", tmp_lib])
        os.replace(tmp_lib, PROBE_LIB)
    if verbose:
        print("built", LIB, "and", PROBE_LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
