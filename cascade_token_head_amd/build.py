"""Build libspatten.so for gfx950 in-tree (next to this file).

    python -m cascade_token_head_amd.build

Every HIP source is compiled with hipcc for gfx950 only; the HIP-free
argument validator is compiled as plain C++ into the same library.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libspatten.so")

HIP_SOURCES = ["api.hip", "gemm.hip", "attn.hip", "decode.hip", "topk.hip", "compact.hip",
               "quant.hip", "ada.hip", "timing.hip"]
CXX_SOURCES = ["validate.cpp"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
HIP_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # no packed fp32 instructions in generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # IEEE fp32 division (the int8 quantizer's codes depend on it)
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-Wno-unused-result",
]
CXX_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall", "-Wextra"]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("command failed: %s\n%s%s" % (" ".join(cmd), r.stdout, r.stderr))
    return r


# Per-source extra flags. Attention never sees NaN inputs, so its max
# reductions skip IEEE-mode NaN quieting (one v_max per element instead of
# two); infinities (masked scores) keep their meaning. Its MFMA results are
# consumed by VALU code at once, so they are kept in VGPRs rather than
# accumulation registers that would need a copy per element.
EXTRA_FLAGS = {"attn.hip": ["-fno-honor-nans", "-mno-amdgpu-ieee",
                            "-mllvm", "-amdgpu-mfma-vgpr-form"]}


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    jobs = []
    for src in HIP_SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        jobs.append([HIPCC] + HIP_FLAGS + EXTRA_FLAGS.get(src, []) +
                    ["-c", os.path.join(CSRC, src), "-o", obj])
    for src in CXX_SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        jobs.append(["g++"] + CXX_FLAGS + ["-c", os.path.join(CSRC, src), "-o", obj])
    workers = min(len(jobs), max(1, (os.cpu_count() or 2)))
    with ThreadPoolExecutor(max_workers=workers) as ex:
        for r in ex.map(_run, jobs):
            if verbose and (r.stdout or r.stderr):
                print(r.stdout, r.stderr, file=sys.stderr)
    objs = [os.path.join(BUILD, s + ".o") for s in HIP_SOURCES + CXX_SOURCES]
    tmp = LIB + ".tmp"
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
