"""Build libsta.so (the STA C-ABI library) for gfx950 with hipcc, in-tree.

Usage: ``python -m block_sparse_sliding_amd.build`` (or call ``build()``).
Objects go to ``_build/`` at the repository root; the shared library is
written next to this file as ``libsta.so``.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libsta.so")
SOURCES = ["sta_api.hip", "sta_layout.hip", "sta_schedule.hip", "sta_attention.hip",
           "sta_backward.hip"]
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-result",
    # packed fp32 VALU forms are kept out of the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{os.path.join(ROOT, 'include')}",
]


# The attention kernel never creates a NaN (keys that must not contribute are
# masked to -inf and read from a zero row), so its max reductions need no NaN
# quieting; its MFMAs are selected in the VGPR form (the configuration it was
# measured in).
EXTRA_FLAGS = {"sta_attention.hip": ["-fno-honor-nans", "-mllvm", "-amdgpu-mfma-vgpr-form=1"]}


def _hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found; ROCm is required to build libsta.so")
    return path


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # hipcc's host pass warns about the device-only target feature: harmless
    lines = [ln for ln in r.stdout.splitlines() if "packed-fp32-ops" not in ln]
    if r.returncode != 0:
        raise RuntimeError("build failed:\n" + " ".join(cmd) + "\n" + "\n".join(lines))
    return "\n".join(lines)


def build(verbose: bool = False, jobs: int = 4) -> str:
    """Compile every HIP source and link libsta.so. Always recompiles."""
    os.makedirs(BUILD, exist_ok=True)
    hipcc = _hipcc()
    objs = []
    cmds = []
    for src in SOURCES:
        obj = os.path.join(BUILD, src.replace(".hip", ".o"))
        objs.append(obj)
        cmds.append([hipcc, *HIPCC_FLAGS, *EXTRA_FLAGS.get(src, []), "-c", os.path.join(CSRC, src),
                     "-o", obj])
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        logs = list(ex.map(_run, cmds))
    tmp = LIB + ".tmp"
    logs.append(_run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]))
    os.replace(tmp, LIB)
    if verbose:
        for log in logs:
            if log.strip():
                print(log)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
