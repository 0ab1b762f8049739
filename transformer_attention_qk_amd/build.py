"""Build step: compile the HIP sources under csrc/ into libattn.so for gfx950 with hipcc.

Run ``python -m transformer_attention_qk_amd.build`` (or ``__graft_entry__.build()``). The
library is written next to this file, so it travels with the source tree.
"""

from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys
import tempfile

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
REPO_DIR = os.path.dirname(PKG_DIR)
LIB_NAME = "libattn.so"
LIB_PATH = os.path.join(PKG_DIR, LIB_NAME)
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-Wall",
    # No packed fp32 instructions: the compiler would otherwise form them from float code.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # Inputs are finite by contract and the kernels use only +-inf as sentinels: with NaNs out
    # of the picture, max needs no operand canonicalisation.
    "-fno-honor-nans",
]


def sources() -> list[str]:
    return sorted(glob.glob(os.path.join(PKG_DIR, "csrc", "*.hip")))


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found; the HIP toolchain (ROCm) is required to build libattn")


def build_library(verbose: bool = False) -> str:
    """Compile every csrc/*.hip file into libattn.so. Raises on a compiler error."""
    srcs = sources()
    if not srcs:
        raise RuntimeError("no HIP sources found under csrc/")
    fd, tmp = tempfile.mkstemp(prefix=".libattn.", suffix=".so.tmp", dir=PKG_DIR)
    os.close(fd)
    cmd = [hipcc(), *HIPCC_FLAGS, "-I", os.path.join(REPO_DIR, "include"), "-o", tmp, *srcs]
    if verbose:
        print(" ".join(cmd), flush=True)
    proc = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-fp32 feature and says so; that line is harmless.
    noise = "packed-fp32-ops"
    err = "\n".join(l for l in proc.stderr.splitlines() if noise not in l).strip()
    if proc.returncode != 0:
        os.unlink(tmp)
        raise RuntimeError(f"hipcc failed ({proc.returncode}):\n{err}")
    if verbose and err:
        print(err, file=sys.stderr)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


DIAG_NAME = "libattn_diag.so"
DIAG_PATH = os.path.join(PKG_DIR, DIAG_NAME)


def build_diag_library(verbose: bool = False) -> str:
    """Compile the issue-rate probe (diag/issue_rates.hip) into libattn_diag.so. It is a
    measurement tool that bench.py --issue-rates loads; the attention library does not use it."""
    src = os.path.join(PKG_DIR, "diag", "issue_rates.hip")
    fd, tmp = tempfile.mkstemp(prefix=".libattn_diag.", suffix=".so.tmp", dir=PKG_DIR)
    os.close(fd)
    cmd = [hipcc(), *HIPCC_FLAGS, "-o", tmp, src]
    if verbose:
        print(" ".join(cmd), flush=True)
    proc = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in proc.stderr.splitlines() if "packed-fp32-ops" not in l).strip()
    if proc.returncode != 0:
        os.unlink(tmp)
        raise RuntimeError(f"hipcc failed ({proc.returncode}):\n{err}")
    os.replace(tmp, DIAG_PATH)
    return DIAG_PATH


if __name__ == "__main__":
    print(build_library(verbose=True))
    print(build_diag_library(verbose=True))
