"""Build libcsa.so (the HIP/gfx950 kernels and their C ABI) in-tree.

    python -m long_context_compressed_csa_amd.build [--jobs N] [--verbose]

Every .hip file under csrc/ is compiled for gfx950 by hipcc into an object
file under _build/, then linked into long_context_compressed_csa_amd/libcsa.so.
Packed-fp32 instruction forms are disabled for all device code; attend.hip
also selects the VGPR form of MFMA results (see EXTRA_FLAGS).
"""

from __future__ import annotations

import argparse
import concurrent.futures as cf
import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libcsa.so")
# the bounds-checked debug library: attend.hip and abi.hip built with
# CSA_DEBUG=1, every other object shared with the release build
DEBUG_LIB = os.path.join(PKG, "libcsa_debug.so")
DEBUG_SOURCES = ("attend.hip", "abi.hip")

ARCH = "gfx950"
CXXFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17", "-Wall",
    "-Wno-unused-function", "-Wno-unused-variable",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]
# Per-source extra flags.  attend.hip: MFMA results go to VGPRs by default
# (its S^T accumulators feed VALU code; its O accumulator is pinned to AGPRs
# explicitly in the source), and the scheduler tracks register pressure with
# the AMDGPU trackers, without which its main loop spills.
EXTRA_FLAGS = {
    "attend.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form", "-mllvm", "-amdgpu-use-amdgpu-trackers=1"],
    # outproj.hip: 128 accumulators + operands fit 256 VGPRs; in AGPRs the
    # compiler moves them back and forth around the K loop
    "outproj.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
}


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the ROCm toolchain is required to build libcsa.so")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    p = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the packed-fp32 feature; that warning is noise
    err = "\n".join(x for x in p.stderr.splitlines() if "packed-fp32-ops" not in x)
    if p.returncode != 0:
        raise RuntimeError(f"command failed ({p.returncode}): {' '.join(cmd)}\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)


def build(jobs: int = 8, verbose: bool = False) -> str:
    hipcc = _hipcc()
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    if not srcs:
        raise RuntimeError(f"no HIP sources under {CSRC}")
    objs = []
    cmds = []
    for s in srcs:
        o = os.path.join(BUILD, os.path.basename(s) + ".o")
        objs.append(o)
        cmds.append([hipcc, *CXXFLAGS, *EXTRA_FLAGS.get(os.path.basename(s), []), "-c", s, "-o", o])
    with cf.ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        list(ex.map(lambda c: _run(c, verbose), cmds))
    tmp = LIB + ".tmp"
    _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs], verbose)
    os.replace(tmp, LIB)
    build_debug(verbose)
    return LIB


def build_debug(verbose: bool = False) -> str:
    """Build DEBUG_LIB; the release objects must exist (build() does both)."""
    hipcc = _hipcc()
    out = os.path.join(BUILD, "debug")
    os.makedirs(out, exist_ok=True)
    objs, cmds = [], []
    for s in sorted(glob.glob(os.path.join(CSRC, "*.hip"))):
        name = os.path.basename(s)
        if name in DEBUG_SOURCES:
            o = os.path.join(out, name + ".o")
            cmds.append([hipcc, *CXXFLAGS, *EXTRA_FLAGS.get(name, []), "-DCSA_DEBUG=1", "-c", s, "-o", o])
        else:
            o = os.path.join(BUILD, name + ".o")
        objs.append(o)
    with cf.ThreadPoolExecutor(max_workers=len(cmds)) as ex:
        list(ex.map(lambda c: _run(c, verbose), cmds))
    tmp = DEBUG_LIB + ".tmp"
    _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs], verbose)
    os.replace(tmp, DEBUG_LIB)
    return DEBUG_LIB


# Host-side sanitizer build: the files whose host code validates arguments
# and keeps host state (abi.hip, blockpool.hip) are compiled with
# AddressSanitizer and UndefinedBehaviorSanitizer on their host pass only
# (device code is unchanged); every other object comes from the regular
# build.  The result needs the sanitizer runtime preloaded (see
# sanitizer_runtime()); the CPU tests load it through CSA_LIBRARY.
HOSTSAN_SOURCES = ("abi.hip", "blockpool.hip")
HOSTSAN_FLAGS = ["-O1", "-g", "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                 "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]
HOSTSAN_LIB = os.path.join(BUILD, "hostsan", "libcsa_hostsan.so")


def sanitizer_runtime() -> str | None:
    """The clang AddressSanitizer runtime of the ROCm toolchain, if present."""
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


def build_host_sanitized(verbose: bool = False) -> str:
    """Build HOSTSAN_LIB; the regular objects must exist (build() first)."""
    hipcc = _hipcc()
    out = os.path.dirname(HOSTSAN_LIB)
    os.makedirs(out, exist_ok=True)
    objs = []
    for s in sorted(glob.glob(os.path.join(CSRC, "*.hip"))):
        name = os.path.basename(s)
        if name in HOSTSAN_SOURCES:
            o = os.path.join(out, name + ".o")
            flags = [f for f in CXXFLAGS if f != "-O3"]
            _run([hipcc, *flags, *HOSTSAN_FLAGS, "-c", s, "-o", o], verbose)
        else:
            o = os.path.join(BUILD, name + ".o")
            if not os.path.exists(o):
                raise RuntimeError(f"{o} is missing: run the regular build first")
        objs.append(o)
    _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", HOSTSAN_LIB, *objs], verbose)
    return HOSTSAN_LIB


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--jobs", type=int, default=8)
    ap.add_argument("--verbose", action="store_true")
    ap.add_argument("--host-sanitize", action="store_true",
                    help="also build the host-sanitizer variant of the library")
    a = ap.parse_args(argv)
    print(build(a.jobs, a.verbose))
    if a.host_sanitize:
        print(build_host_sanitized(a.verbose))


if __name__ == "__main__":
    main()
