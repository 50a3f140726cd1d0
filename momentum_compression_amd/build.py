"""Build libonebit.so (gfx950) in-tree with hipcc.

    python -m momentum_compression_amd.build          # compile and link

Floating-point flags are part of the contract: no FMA contraction,
correctly rounded binary32 division and square root, subnormals kept, and
packed-fp32 instruction selection disabled.
"""

from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libonebit.so")

SOURCES = ["api.hip", "compress.hip", "finalize.hip", "server.hip", "scale.hip", "step.hip",
           "int8.hip", "warmup.hip"]

ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-ffp-contract=off",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-fno-gpu-flush-denormals-to-zero",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
    "-Wextra",
    "-Wno-unused-function",
    f"-I{INCLUDE}",
    f"-I{CSRC}",
]


def hipcc() -> str:
    p = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(p):
        raise RuntimeError("hipcc not found: the ROCm toolchain is required to build libonebit")
    return p


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{res.stderr}")
    # the host pass does not know the GPU feature switched off above; every
    # other diagnostic is shown
    notes = [ln for ln in res.stderr.splitlines()
             if ln.strip() and "packed-fp32-ops" not in ln and "warnings generated" not in ln
             and "warning generated" not in ln]
    if notes:
        print(f"{src}:\n" + "\n".join(notes), file=sys.stderr)
    return obj


# the memory-pattern probes of the benchmark, in a library of their own
PROBE_SRC = "stream_probe.hip"
PROBE_LIB = os.path.join(HERE, "libonebit_probe.so")


def build_probe() -> str:
    obj = _compile(PROBE_SRC)
    tmp = PROBE_LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", obj, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"probe link failed:\n{res.stderr}")
    os.replace(tmp, PROBE_LIB)
    return PROBE_LIB


CAPI_SRC = os.path.join(ROOT, "tests", "capi", "capi_roundtrip.c")
CAPI_BIN = os.path.join(BUILD, "capi_roundtrip")


def _rocm() -> str:
    return os.path.dirname(os.path.dirname(os.path.realpath(hipcc())))


def build_capi() -> str:
    """The plain C consumer of the ABI (host code only: gcc, the HIP runtime
    and libonebit.so, found next to the binary's parent directory)."""
    rocm = _rocm()
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        raise RuntimeError("no C compiler for the C ABI test program")
    cmd = [cc, "-std=c99", "-O2", "-Wall", "-Wextra", "-D__HIP_PLATFORM_AMD__",
           f"-I{rocm}/include", f"-I{INCLUDE}", CAPI_SRC, f"-L{HERE}", "-lonebit",
           f"-L{rocm}/lib", "-lamdhip64", "-lm", "-Wl,-rpath,$ORIGIN/..",
           f"-Wl,-rpath,{rocm}/lib", "-o", CAPI_BIN]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"C ABI test program failed to build:\n{res.stderr}")
    return CAPI_BIN


def build(verbose: bool = False) -> str:
    """Compile every kernel source for gfx950, link libonebit.so, build the
    plain C test program against it, and build the benchmark's probe
    library."""
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
        probe = ex.submit(build_probe)
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stderr}")
    os.replace(tmp, LIB)
    build_capi()
    probe.result()
    if verbose:
        print(f"built {LIB}, {CAPI_BIN} and {PROBE_LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
