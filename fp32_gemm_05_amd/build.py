"""Build step of libsgemm: compile the HIP sources for gfx950 into libsgemm.so (in-tree)."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libsgemm.so")
SOURCES = [os.path.join(CSRC, "sgemm.hip")]
KERNEL_HEADERS = ("kernel_common.hpp", "kernel_mfma.hpp", "kernel_pipe.hpp", "kernel_deep.hpp", "kernel_splitk.hpp",
                  "kernel_direct.hpp", "kernel_dl.hpp", "kernel_valu.hpp")
DEPENDS = SOURCES + [os.path.join(CSRC, f) for f in ("sgemm_kernels.hpp", "sgemm_launch.hpp", "tuned_table.inc")
                     + KERNEL_HEADERS] + [
    os.path.join(os.path.dirname(HERE), "include", "sgemm.h")]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-fvisibility=hidden",
    # no packed-fp32 instructions in any kernel (scalar fp32 VALU and MFMA only)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


# The read-bandwidth reference of the profiling summaries (not part of libsgemm).
HBM_READ_LIB = os.path.join(HERE, "libhbm_read.so")
HBM_READ_SOURCES = [os.path.join(CSRC, "hbm_read.hip")]


# The profiling build of libsgemm: the same sources with the kernels' phase stamps compiled in
# (read by `python -m fp32_gemm_05_amd.profiling phases`; never loaded by the product path).
STAMPS_LIB = os.path.join(HERE, "libsgemm_stamps.so")


# The launch-floor and engine-clock reference kernels of the bench (not part of libsgemm).
LAUNCH_REFS_LIB = os.path.join(HERE, "liblaunch_refs.so")
LAUNCH_REFS_SOURCES = [os.path.join(CSRC, "launch_refs.hip")]


def build(verbose: bool = False, extra_flags=None, out: str | None = None) -> str:
    """Compile libsgemm's HIP sources into one shared library; returns its path."""
    return _compile(SOURCES, out or LIB, verbose, extra_flags)


def build_stamps(verbose: bool = False) -> str:
    """Compile the phase-stamp profiling build of libsgemm (libsgemm_stamps.so); returns its path."""
    return _compile(SOURCES, STAMPS_LIB, verbose, ["-DSGEMM_PHASE_STAMPS"])


def build_hbm_read(verbose: bool = False) -> str:
    """Compile the streaming-read reference kernel (libhbm_read.so); returns its path."""
    return _compile(HBM_READ_SOURCES, HBM_READ_LIB, verbose, None)


def build_launch_refs(verbose: bool = False) -> str:
    """Compile the launch-floor and clock-probe reference kernels (liblaunch_refs.so)."""
    return _compile(LAUNCH_REFS_SOURCES, LAUNCH_REFS_LIB, verbose, None)


def _compile(sources, out: str, verbose: bool, extra_flags) -> str:
    cmd = [HIPCC, *FLAGS, *(extra_flags or []), *sources, "-o", out + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass reports the device-only target feature as unknown; drop that line only
    noise = "is not a recognized feature for this target"
    msg = "\n".join(l for l in (res.stdout + res.stderr).splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{msg}")
    if verbose and msg.strip():
        print(msg, file=sys.stderr)
    os.replace(out + ".tmp", out)
    return out


def is_stale(lib: str = LIB) -> bool:
    if not os.path.exists(lib):
        return True
    t = os.path.getmtime(lib)
    return any(os.path.getmtime(d) > t for d in DEPENDS if os.path.exists(d))


if __name__ == "__main__":
    print(build(verbose=True))
