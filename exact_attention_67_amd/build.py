"""Build the HIP library in-tree: exact_attention_67_amd/libfa_mi355x.so.

Compiles the HIP sources in csrc/ (forward and backward kernels, host entry
points) into one shared library, for gfx950 only, with hipcc.  Packed-fp32 code
generation is switched off for device code (the host pass warns that it does
not know the feature; that warning is harmless).

Usage:  python -m exact_attention_67_amd.build [--verbose] [--save-temps DIR]
"""

from __future__ import annotations

import argparse
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
SOURCES = [os.path.join(CSRC, "fa_fwd.hip"), os.path.join(CSRC, "fa_bwd.hip")]
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libfa_mi355x.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the library)")


def compile_flags() -> list:
    return [
        f"--offload-arch={ARCH}",
        "-O3",
        "-std=c++17",
        "-fPIC",
        "-Wall",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", INCLUDE,
        "-I", CSRC,
    ]


def build(verbose: bool = False, save_temps: str | None = None) -> str:
    """Compile the library; always recompiles.  Returns the .so path."""
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc(), *compile_flags(), "-shared", *[src for src in SOURCES if os.path.exists(src)],
           "-o", tmp]
    if save_temps:
        os.makedirs(save_temps, exist_ok=True)
        cmd.insert(1, "-save-temps=cwd")
        cmd.insert(1, "-Rpass-analysis=kernel-resource-usage")
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True,
                         cwd=save_temps if save_temps else PKG)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed with exit code {res.returncode}")
    if verbose and (res.stdout or res.stderr):
        sys.stderr.write(res.stdout + res.stderr)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


def main() -> None:
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--verbose", action="store_true")
    ap.add_argument("--save-temps", default=None,
                    help="directory to keep intermediate files (ISA) and resource usage")
    a = ap.parse_args()
    print(build(verbose=a.verbose, save_temps=a.save_temps))


if __name__ == "__main__":
    main()
