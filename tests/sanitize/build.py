"""Build the host-sanitizer self-tests (test infrastructure; CPU only).

* oracle_selftest: the C oracle (oracle/*.c) and tests/sanitize/oracle_selftest.c
  with gcc -fsanitize=address,undefined.
* host_selftest: the GEMV library's host code built with hipcc, the
  sanitizers on the host pass only (-Xarch_host before each -fsanitize=;
  device code is built as always), and tests/sanitize/host_selftest.c with
  the same clang, so that one sanitizer runtime serves both.

Outputs go to a build directory given by the caller (tests use a temporary
directory); nothing is written in-tree.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]


def build_oracle_selftest(out_dir: str) -> str:
    exe = os.path.join(out_dir, "oracle_selftest")
    srcs = [os.path.join(HERE, "oracle_selftest.c")] + [
        os.path.join(ROOT, "oracle", f) for f in ("gemv_oracle.c", "quant_oracle.c", "softmax_oracle.c")]
    subprocess.run(["gcc", "-O1", "-g", "-std=c11", "-Wall", "-Wextra", "-Werror", "-fopenmp", *SAN, *srcs,
                    "-o", exe, "-lm"], check=True)
    return exe


def build_host_selftest(out_dir: str) -> str:
    lib = os.path.join(out_dir, "libgemv_san.so")
    csrc = os.path.join(ROOT, "memory_bound_gemv_row_amd", "csrc")
    host_san = []
    for flag in ("-fsanitize=address", "-fsanitize=undefined", "-fno-omit-frame-pointer"):
        host_san += ["-Xarch_host", flag]
    subprocess.run([os.path.join(ROCM, "bin", "hipcc"), "-O1", "-g", "-std=c++17", "--offload-arch=gfx950", "-fPIC",
                    "-shared", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", *host_san,
                    "-I", os.path.join(ROOT, "include"), "-I", csrc,
                    *(os.path.join(csrc, f) for f in ("gemv_api.hip", "quant_api.hip", "softmax_api.hip")),
                    "-o", lib], check=True, capture_output=True, text=True)
    exe = os.path.join(out_dir, "host_selftest")
    subprocess.run([os.path.join(ROCM, "llvm", "bin", "clang"), "-O1", "-g", "-std=c11", "-Wall", "-Wextra",
                    "-Werror", *SAN, "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"),
                    "-I", os.path.join(ROCM, "include"), os.path.join(HERE, "host_selftest.c"), "-o", exe,
                    "-L", out_dir, "-lgemv_san", "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
                    "-Wl,-rpath," + out_dir, "-Wl,-rpath," + os.path.join(ROCM, "lib")], check=True)
    return exe
