"""Builds libm2rnn.so (the HIP kernels + C ABI) for gfx950 with hipcc, in-tree.

Each translation unit is compiled in its own hipcc process (in parallel), then linked into
``matrix_state_nonlinear_m2rnn_amd/libm2rnn.so``.
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libm2rnn.so")
BUILD_DIR = os.path.join(os.path.dirname(PKG), "_build")
ARCH = os.environ.get("M2RNN_OFFLOAD_ARCH", "gfx950")

SOURCES = [
    "m2rnn_api.hip",
    "m2rnn_fwd_f32.hip",
    "m2rnn_fwd_f16x3.hip",
    "m2rnn_fwd_bf16x3.hip",
    "m2rnn_fwd_bf16.hip",
    "m2rnn_decode.hip",
    "m2rnn_block.hip",
]

# Packed fp32 VALU ops stay off: hipcc -O3 would otherwise form v_pk_{add,mul,fma}_f32.
# MFMA results stay in ordinary VGPRs (no accumulation-register copies in the step loop).
# -Wno-pass-failed: the step loops ask to be unrolled whole; in the four-row-block kernels (never
# planned automatically) the unrolled body exceeds the compiler's limit and the loop runs rolled,
# which is correct, only slower, so the warning that reports it is not printed.
FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang",
         "-packed-fp32-ops", "-mllvm", "-amdgpu-mfma-vgpr-form", "-Wno-unused-command-line-argument",
         "-Wno-pass-failed"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libm2rnn.so)")


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc()] + FLAGS + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(line for line in r.stderr.splitlines() if noise not in line)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{err}")
    if err.strip():
        sys.stderr.write(err + "\n")
    return obj


def build(jobs: int = 0) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    jobs = jobs or min(len(SOURCES), max(1, (os.cpu_count() or 2)))
    with concurrent.futures.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
