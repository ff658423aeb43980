"""Build the HIP library in-tree: exact_attention_67_amd/libfa_mi355x.so.

Compiles the HIP sources in csrc/ (forward and backward kernels, host entry
points) into one shared library, for gfx950 only, with hipcc, and the same
sources with the bf16 forward's tile pipeline in its study modes into
libfa_mi355x_pipe_<name>.so (in parallel).  Packed-fp32 code
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


def _compile(out_path: str, defines: list, verbose: bool, save_temps: str | None):
    tmp = out_path + ".tmp"
    cmd = [hipcc(), *compile_flags(), *defines, "-shared",
           *[src for src in SOURCES if os.path.exists(src)], "-o", tmp]
    if save_temps:
        os.makedirs(save_temps, exist_ok=True)
        cmd.insert(1, "-save-temps=cwd")
        cmd.insert(1, "-Rpass-analysis=kernel-resource-usage")
    if verbose:
        print(" ".join(cmd), flush=True)
    proc = subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True,
                            cwd=save_temps if save_temps else PKG)
    return proc, tmp, out_path


def build(verbose: bool = False, save_temps: str | None = None, variants: bool = True) -> str:
    """Compile the library (and, unless variants=False, the pipeline-study
    builds of it) for gfx950; always recompiles.  Returns the library path."""
    from ._lib import PIPE_VARIANTS, variant_path

    jobs = [_compile(LIB_PATH, [], verbose, save_temps)]
    if variants and not save_temps:
        for name, mode in PIPE_VARIANTS.items():
            jobs.append(_compile(variant_path(name), [f"-DFA_PIPE={mode}"], verbose, None))
    failed = []
    for proc, tmp, out_path in jobs:
        out, _ = proc.communicate()
        if proc.returncode != 0:
            sys.stderr.write(out)
            failed.append((out_path, proc.returncode))
            continue
        if verbose and out:
            sys.stderr.write(out)
        os.replace(tmp, out_path)
    if failed:
        raise RuntimeError(f"hipcc failed: {failed}")
    return LIB_PATH


def main() -> None:
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--verbose", action="store_true")
    ap.add_argument("--save-temps", default=None,
                    help="directory to keep intermediate files (ISA) and resource usage")
    ap.add_argument("--no-variants", action="store_true",
                    help="build only the library, not its pipeline-study builds")
    a = ap.parse_args()
    print(build(verbose=a.verbose, save_temps=a.save_temps, variants=not a.no_variants))


if __name__ == "__main__":
    main()
