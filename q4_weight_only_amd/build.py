"""Build libq4amd.so in-tree for gfx950 with hipcc.

    python -m q4_weight_only_amd.build

Each .hip source is compiled to an object in parallel, then linked into
q4_weight_only_amd/libq4amd.so (written to a temporary name and renamed, so a
concurrent reader never sees a half-written library).
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
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libq4amd.so")

SOURCES = ("q4_0_format.hip", "q4_1_format.hip", "q4_0_linear.hip", "q4_0_measure.hip", "q4_0_abi.hip")
ARCH = "gfx950"

COMMON_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    # Packed fp32 VALU ops stay off: every fp32 op is issued one lane value
    # at a time.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA results in VGPRs: the per-block fp32 rescale reads them directly
    # instead of copying each one out of an AGPR first.
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    # Up to 12 leading scalar kernel arguments arrive preloaded in SGPRs, so a
    # decode launch's first loads do not wait on a fetch of its arguments.
    "-mllvm", "-amdgpu-kernarg-preload-count=12",
    "-Wall",
    "-Wextra",
    "-Wno-unused-command-line-argument",
    f"-I{INCLUDE}",
    f"-I{CSRC}",
]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (expected /opt/rocm/bin/hipcc)")


def _run(cmd):
    proc = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # the host pass of hipcc does not know the packed-fp32 target feature and
    # says so; that note is harmless and filtered out
    out = "\n".join(l for l in proc.stdout.splitlines() if "packed-fp32-ops" not in l)
    if proc.returncode != 0:
        raise RuntimeError(f"command failed ({proc.returncode}): {' '.join(cmd)}\n{out}")
    return out


BUILD_INFO = os.path.join(BUILD_DIR, "build_info.json")


def _write_build_info() -> None:
    """Record the source revision the library was built from (reports read
    it where no git checkout exists)."""
    import json

    def git(*args):
        try:
            return subprocess.run(["git", *args], cwd=ROOT, stdout=subprocess.PIPE, stderr=subprocess.DEVNULL,
                                  text=True, timeout=30).stdout.strip()
        except (OSError, subprocess.SubprocessError):
            return ""
    info = {"git_rev": git("rev-parse", "HEAD") or None,
            "dirty": bool(git("status", "--porcelain", "--untracked-files=no"))}
    with open(BUILD_INFO, "w") as f:
        json.dump(info, f)


def build(verbose: bool = False) -> str:
    """Compile every HIP source for gfx950 and link libq4amd.so; return its path."""
    hipcc = _hipcc()
    os.makedirs(BUILD_DIR, exist_ok=True)
    objs = []
    cmds = []
    for src in SOURCES:
        obj = os.path.join(BUILD_DIR, src.replace(".hip", ".o"))
        objs.append(obj)
        cmds.append([hipcc, *COMMON_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj])
    with ThreadPoolExecutor(max_workers=len(cmds)) as ex:
        outs = list(ex.map(_run, cmds))
    for o in outs:
        # compiler warnings are always shown; other output only when asked
        shown = o if verbose else "\n".join(l for l in o.splitlines() if "warning:" in l)
        if shown.strip():
            print(shown)
    _write_build_info()
    tmp = LIB + f".tmp{os.getpid()}"
    _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    path = build(verbose="-v" in sys.argv)
    print(path)
