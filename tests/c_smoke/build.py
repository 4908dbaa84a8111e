"""Compile the C-only ABI smoke program (test infrastructure) with gcc,
against the in-tree HIP library and the CPU oracle library.  Called by
__graft_entry__.build(); the binary stays in-tree (git-ignored)."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
SRC = os.path.join(HERE, "c_abi_smoke.c")
BIN = os.path.join(HERE, "c_abi_smoke")


def build() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    cmd = [
        "gcc", "-O2", "-std=c11", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
        "-I", os.path.join(ROOT, "include"), "-I", os.path.join(rocm, "include"),
        SRC, "-o", BIN,
        "-L", os.path.join(ROOT, "memory_bound_gemv_row_amd"), "-lgemv_amd",
        "-L", os.path.join(ROOT, "oracle"), "-loracle",
        "-L", os.path.join(rocm, "lib"), "-lamdhip64", "-lm",
        "-Wl,-rpath,$ORIGIN/../../memory_bound_gemv_row_amd", "-Wl,-rpath,$ORIGIN/../../oracle",
        "-Wl,-rpath," + os.path.join(rocm, "lib"),
    ]
    subprocess.run(cmd, check=True)
    return BIN


if __name__ == "__main__":
    print(build())
