"""Builds the HIP libraries in-tree for gfx950.

* ``learned_kv_cache_dms_amd/libdms_hip.so`` - the DMS decode path (C ABI of
  ``include/dms.h``).
* ``synth/libdms_synth.so`` - device twin of the synthetic input generator.

Run ``python -m learned_kv_cache_dms_amd.build`` (or ``__graft_entry__.build()``).
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "learned_kv_cache_dms_amd")
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libdms_hip.so")
SYNTH_LIB = os.path.join(ROOT, "synth", "libdms_synth.so")
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the DMS library)")


COMMON = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
    # packed-FP32 VALU forms are kept out of every code object
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
    # only the C ABI is exported; internal C++ symbols stay private
    "-fvisibility=hidden",
]

# Device code only: the atomic optimizer rewrites a one-lane atomicAdd into a
# wave-wide one whose result is read at once, which makes the wave wait for
# every load it has in flight; the attention takes its next work item that
# way while its prefetched blocks are loading.
DMS_DEVICE = ["-Xarch_device", "-mllvm=-amdgpu-atomic-optimizer-strategy=None",
              # MFMA accumulators in ordinary VGPRs: the attention kernels rescale and
              # normalise them with VALU code, which cannot read AGPRs; with the
              # accumulators in AGPRs every pair step copied them back and forth
              # (prompt attention 328 -> 292 ms, relaxed forward 1.83 -> 1.60 ms)
              "-Xarch_device", "-mllvm=-amdgpu-mfma-vgpr-form=1"]


def _run(cmd):
    print("+", " ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if out.strip():
        print(out, flush=True)
    if r.returncode != 0:
        raise RuntimeError(f"build failed ({r.returncode}): {' '.join(cmd)}")


# the kernels by subsystem, and the host runtime behind the C ABI
DMS_SOURCES = ("dms_decode.hip", "dms_prompt.hip", "dms_soft.hip", "dms_runtime.cpp")


def build_dms(out: str = LIB, extra=()):
    tmp = out + ".tmp"
    _run([hipcc(), *COMMON, *DMS_DEVICE, *extra, "-I", os.path.join(ROOT, "include"), "-I", CSRC,
          *[os.path.join(CSRC, f) for f in DMS_SOURCES], "-o", tmp])
    os.replace(tmp, out)
    return out


def build_synth(out: str = SYNTH_LIB):
    tmp = out + ".tmp"
    _run([hipcc(), *COMMON, os.path.join(ROOT, "synth", "synth.hip"), "-o", tmp])
    os.replace(tmp, out)
    return out


def build_all():
    build_dms()
    build_synth()


if __name__ == "__main__":
    build_all()
    sys.exit(0)
