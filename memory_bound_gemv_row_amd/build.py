"""Build the gfx950 HIP library in-tree with hipcc.

``python -m memory_bound_gemv_row_amd.build`` compiles
``csrc/gemv_api.hip`` (GEMV, which includes its kernels) and
``csrc/quant_api.hip`` (the weight quantiser) and ``csrc/softmax_api.hip``
(the row softmax) into one library,
``memory_bound_gemv_row_amd/libgemv_amd.so``.
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SRC_DIR = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libgemv_amd.so")
SOURCES = [os.path.join(SRC_DIR, f) for f in ("gemv_api.hip", "quant_api.hip", "softmax_api.hip")]
DEPENDS = SOURCES + [os.path.join(SRC_DIR, f) for f in ("gemv_kernels.hpp", "quant_kernels.hpp", "softmax_kernels.hpp",
                                                    "device_info.hpp")] \
    + [os.path.join(INCLUDE, f) for f in ("gemv.h", "gemv_quant.h", "gemv_softmax.h")]
ARCH = "gfx950"

HIPCC_FLAGS = [
    "-O3",
    "-std=c++17",
    f"--offload-arch={ARCH}",
    "-fPIC",
    "-shared",
    "-Wall",
    "-Wextra",
    "-Werror",          # host and device warnings fail the build
    # no packed FP32 instructions in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    cand = os.path.join(rocm, "bin", "hipcc")
    return cand if os.path.exists(cand) else "hipcc"


def stale() -> bool:
    if not os.path.exists(LIB):
        return True
    t = os.path.getmtime(LIB)
    return any(os.path.getmtime(p) > t for p in DEPENDS)


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [hipcc(), *HIPCC_FLAGS, "-I", INCLUDE, "-I", SRC_DIR, *SOURCES, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    proc = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass reports the device-only feature flag as unknown; that
    # line is expected and harmless, anything else is shown.
    noise = "is not a recognized feature for this target"
    msgs = [l for l in (proc.stdout + proc.stderr).splitlines() if l.strip() and noise not in l]
    if proc.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if msgs and verbose:
        print("\n".join(msgs), file=sys.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
