"""Build libecho.so (HIP kernels + C ABI) in-tree for gfx950 with hipcc.

Usage: ``python -m error_compensated_bit_echo_amd.build`` (or call
:func:`build_library`).  The library lands next to this file.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libecho.so")
SOURCES = ["echo_kernels.hip"] + [f"echo_owner_p{lo}_{lo + 1}.hip" for lo in range(1, 17, 2)] + \
    ["echo_gemm.hip", "echo_scratch.hip", "echo_api.hip"]
HEADERS = ["echo_internal.h", "echo_div7.h", "echo_quant.h", "echo_device.h", "echo_owner.h"]
ARCH = "gfx950"

# -ffp-contract=off: every multiply and add is its own IEEE operation (the
#   kernels must reproduce a fixed sequence of binary32 roundings).
# -packed-fp32-ops off: no v_pk_*_f32 instructions are emitted.
# Denormals are kept (HIP's default; no fast-math, no flush-to-zero).
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-ffp-contract=off", "-fno-fast-math",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libecho)")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{res.stdout}\n{res.stderr}")


def build_library(verbose: bool = False, jobs: int = 0) -> str:
    """Compile every HIP source (in parallel, one object each) and link
    ``libecho.so``; returns its path."""
    from concurrent.futures import ThreadPoolExecutor

    cc = hipcc()
    tmpdir = tempfile.mkdtemp(prefix="echo_build_")
    tmp = LIB + f".tmp{os.getpid()}"
    try:
        objs = [os.path.join(tmpdir, s + ".o") for s in SOURCES]
        cmds = [[cc, *FLAGS, f"-I{INCLUDE}", f"-I{CSRC}", "-c", os.path.join(CSRC, s), "-o", o]
                for s, o in zip(SOURCES, objs)]
        jobs = jobs or min(len(cmds), os.cpu_count() or 1, 16)
        with ThreadPoolExecutor(max_workers=jobs) as ex:
            for f in [ex.submit(_run, c, verbose) for c in cmds]:
                f.result()
        # the host pass does not know the gfx feature flag; that warning is expected
        _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp], verbose)
        os.replace(tmp, LIB)
    finally:
        if os.path.exists(tmp):
            os.unlink(tmp)
        shutil.rmtree(tmpdir, ignore_errors=True)
    return LIB


C_CLIENT_SRC = os.path.join(ROOT, "tests", "c_client", "echo_c_client.c")
C_CLIENT = os.path.join(ROOT, "tests", "c_client", "echo_c_client")
C_LATENCY_SRC = os.path.join(ROOT, "tests", "c_client", "echo_c_latency.c")
C_LATENCY = os.path.join(ROOT, "tests", "c_client", "echo_c_latency")


def _build_c(src: str, exe: str, verbose: bool) -> str:
    rocm = os.path.dirname(os.path.dirname(os.path.realpath(hipcc())))
    cmd = [shutil.which("gcc") or "gcc", "-std=c11", "-O2", "-Wall", "-Wextra", "-Werror", "-pedantic",
           "-D__HIP_PLATFORM_AMD__", "-D_POSIX_C_SOURCE=199309L", f"-I{INCLUDE}", "-isystem",
           os.path.join(rocm, "include"), src, f"-L{PKG}", "-lecho", f"-L{os.path.join(rocm, 'lib')}",
           "-lamdhip64", "-Wl,-rpath,$ORIGIN/../../error_compensated_bit_echo_amd",
           f"-Wl,-rpath,{os.path.join(rocm, 'lib')}", "-o", exe]
    _run(cmd, verbose)
    return exe


def build_c_client(verbose: bool = False) -> str:
    """Compile the plain C clients of the C ABI (gcc, strict C11) against the
    built libecho.so and the HIP runtime: the test client and the per-call
    latency program that `bench.py --config decode` runs; returns the test
    client's path."""
    _build_c(C_LATENCY_SRC, C_LATENCY, verbose)
    return _build_c(C_CLIENT_SRC, C_CLIENT, verbose)


if __name__ == "__main__":
    path = build_library(verbose="-v" in sys.argv)
    print(path)
    print(build_c_client(verbose="-v" in sys.argv))
