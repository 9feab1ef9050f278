"""Build ``libpagedkv.so`` in-tree with hipcc for gfx950.

Usage: ``python paged_kv_cache_360_amd/build.py`` (or ``__graft_entry__.build()``); the
script does not import the package, so a stale library never blocks a rebuild.
Objects go to ``_build/`` at the repository root; the shared library is written
next to this file, where the binding loads it.  Always recompiles.
"""

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT = os.path.join(PKG, "libpagedkv.so")
BUILD_DIR = os.path.join(ROOT, "_build")

ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
HIPCC = os.path.join(ROCM, "bin", "hipcc")
ARCH = "gfx950"

# Device code: gfx950 only; packed-fp32 instruction selection is switched off
# (ordinary scalar fp32 code is generated instead).
HIP_FLAGS = [
    "-O3", "-fPIC", "-std=c++17", f"--offload-arch={ARCH}", "-mcode-object-version=5",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # Work tickets are taken with one lane's atomic add whose result is only
    # needed at the end of the current item.  The atomic optimizer rewrites such
    # an add into a wave-wide form that reads the result at once, which stalls
    # the wave for the round trip and, as vector memory operations complete in
    # order, for every block load issued before it.
    "-Xarch_device", "-mllvm=-amdgpu-atomic-optimizer-strategy=None",
    "-Wall", "-Wno-unused-function", "-Wno-unused-command-line-argument",
]
HOST_FLAGS = ["-O2", "-fPIC", "-std=c++17", "-Wall", "-D__HIP_PLATFORM_AMD__",
              f"-I{ROCM}/include"]

HIP_SOURCES = ["kernels/cache_ops.hip", "kernels/plan.hip", "kernels/decode.hip", "kernels/decode_mfma.hip",
               "kernels/prefill_mfma.hip", "kernels/static_workspace.hip"]
HOST_SOURCES = ["api.cpp", "allocator.cpp"]
# Measurement only: read-bandwidth probes the bench compares the decode kernel
# with (a library of its own; the attention library does not contain them).
PROBE_SOURCES = ["probes/read_probe.hip", "probes/lds_probe.hip"]
PROBE_OUT = os.path.join(PKG, "libpkvprobe.so")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"build step failed: {' '.join(cmd[:3])} ... ({r.returncode})")
    return r


def build(verbose=False, jobs=8):
    """Compile every source and link ``libpagedkv.so``.  Returns the library path."""
    if not os.path.exists(HIPCC):
        raise RuntimeError(f"hipcc not found at {HIPCC}")
    os.makedirs(BUILD_DIR, exist_ok=True)
    cmds, objs = [], []
    for src in HIP_SOURCES:
        obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
        cmds.append([HIPCC, *HIP_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    for src in HOST_SOURCES:
        obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
        cmds.append([HIPCC, *HOST_FLAGS, "-x", "c++", "-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    probe_objs = []
    for src in PROBE_SOURCES:
        obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
        cmds.append([HIPCC, *HIP_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj])
        probe_objs.append(obj)
    with ThreadPoolExecutor(max_workers=max(1, min(jobs, len(cmds)))) as ex:
        list(ex.map(lambda c: _run(c, verbose), cmds))
    for out, names, soname in ((OUT, objs, "libpagedkv.so"), (PROBE_OUT, probe_objs, "libpkvprobe.so")):
        tmp = out + ".tmp"
        _run([HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp, *names,
              f"-Wl,-soname,{soname}", f"-Wl,-rpath,{ROCM}/lib"], verbose)
        shutil.move(tmp, out)
    return OUT


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
