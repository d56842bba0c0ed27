"""Build of libgdn.so for gfx950 with hipcc (in-tree, no JIT cache)."""
from __future__ import annotations

import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIBRARY = os.path.join(CSRC, "libgdn.so")
SOURCES = [os.path.join(CSRC, f) for f in
           ("gdn_api.cpp", "gdn_step.hip", "gdn_seq.hip", "gdn_tail.hip")]
# Measurement aids (a copy of known size and an in-place read-modify-write with
# the step kernel's access pattern), built as their own library.
PROBE_LIBRARY = os.path.join(CSRC, "libgdn_probe.so")
PROBE_SOURCES = [os.path.join(CSRC, "probes.hip")]
ARCH = "gfx950"

# Packed FP32 instructions are switched off for the device code; hipcc's host
# pass does not know the feature and only warns.
HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Wall", "-Wno-unused-command-line-argument",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # arithmetic exactly as written (explicit fmaf where a fused multiply-add
    # is wanted), so kernels that share a formula give the same bits
    "-ffp-contract=off",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


# A plain-C program that calls the library through its C ABI only (a test).
C_CHECK_SOURCE = os.path.join(ROOT, "tests", "c", "gdn_c_check.c")
C_CHECK_BINARY = os.path.join(ROOT, "tests", "c", "gdn_c_check")


def build_c_check(verbose: bool = False) -> str:
    """Compile tests/c/gdn_c_check.c as plain C (gcc, HIP's C runtime API)
    against libgdn.so."""
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    cmd = ["gcc", "-std=c11", "-O2", "-Wall", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(rocm, "include"), "-I", os.path.join(ROOT, "include"),
           C_CHECK_SOURCE, "-o", C_CHECK_BINARY, "-L", CSRC, "-lgdn", f"-Wl,-rpath,{CSRC}",
           "-L", os.path.join(rocm, "lib"), "-lamdhip64", f"-Wl,-rpath,{os.path.join(rocm, 'lib')}",
           "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"gcc failed ({r.returncode}):\n{r.stdout}\n{r.stderr}")
    return C_CHECK_BINARY


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def build(output: str = LIBRARY, extra=(), verbose: bool = False, sources=None) -> str:
    """Compile the decode-path HIP sources into one shared library (and, for
    the default output, the copy probe into its own); returns the path."""
    if sources is None and output == LIBRARY:
        build(PROBE_LIBRARY, extra, verbose, PROBE_SOURCES)
    tmp = output + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, *extra, *(sources or SOURCES), "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, output)
    return output


if __name__ == "__main__":
    print(build(verbose=True))
