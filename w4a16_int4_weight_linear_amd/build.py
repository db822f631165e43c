"""Build the gfx950 C-ABI library libw4a16.so in-tree with hipcc.

Every HIP source is compiled for gfx950 only; the host-only sources are
compiled by the same driver.  Objects go to _build/ at the repository root and
the shared library next to this file, where the binding loads it.

A second, profiling-only library is built from the same sources with
-DW4A16_WAVE_STAMPS into stamps/libw4a16.so: its weight-streaming kernels also
record per-wave timeline stamps (csrc/wave_stamps.hpp), read back through the
extern "C" accessors w4a16_wave_stamps_gemv / _gemv_mfma / _probe, which only
that library exports.  The binding never loads it; bench.py --wave-timeline does.
"""

from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libw4a16.so")
STAMPS_LIB = os.path.join(PKG, "stamps", "libw4a16.so")
ARCH = "gfx950"

HIP_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # no packed-fp32 VALU forms in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the W4A16 library)")


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith((".hip", ".cpp")))


def _compile(hipcc: str, src: str, build_dir: str = BUILD, extra=()) -> str:
    obj = os.path.join(build_dir, os.path.basename(src) + ".o")
    cmd = [hipcc, *HIP_FLAGS, *extra, "-c", src, "-o", obj]
    if src.endswith(".cpp"):
        cmd = [hipcc, "-O3", "-std=c++17", "-fPIC", "-Wall", "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def _check_resolves(path: str) -> None:
    """Load the freshly linked library in a child process: a symbol of its own
    that a source failed to define (for instance a kernel whose host stub
    was not emitted) is an error here rather than at the first import."""
    probe = f"import ctypes; ctypes.CDLL({path!r})"
    r = subprocess.run([sys.executable, "-c", probe], capture_output=True, text=True)
    if r.returncode != 0:
        os.remove(path)
        raise RuntimeError(f"linked library does not load: {r.stderr.strip().splitlines()[-1] if r.stderr else ''}")


def _build_one(hipcc: str, lib: str, build_dir: str, extra, verbose: bool) -> str:
    os.makedirs(build_dir, exist_ok=True)
    os.makedirs(os.path.dirname(lib), exist_ok=True)
    srcs = sources()
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(hipcc, s, build_dir, extra), srcs))
    tmp = lib + ".tmp"
    cmd = [hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    _check_resolves(tmp)
    os.replace(tmp, lib)
    if verbose:
        print(f"built {lib} from {len(srcs)} sources", file=sys.stderr)
    return lib


def build(verbose: bool = False, wave_stamps: bool = True) -> str:
    """Compile every source and link libw4a16.so (and, unless wave_stamps is
    False, the profiling library stamps/libw4a16.so); returns the product
    library's path."""
    hipcc = _hipcc()
    lib = _build_one(hipcc, LIB, BUILD, (), verbose)
    if wave_stamps:
        _build_one(hipcc, STAMPS_LIB, os.path.join(BUILD, "stamps"), ("-DW4A16_WAVE_STAMPS",), verbose)
    return lib


if __name__ == "__main__":
    build(verbose=True)
