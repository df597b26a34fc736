"""Builds the HIP library ``libsft.so`` in-tree with hipcc for gfx950."""
from __future__ import annotations

import glob
import os
import subprocess
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
LIB = os.path.join(PKG, "libsft.so")

# -ffp-contract=off: the update kernels round every product and sum on its own.
# -packed-fp32-ops off: no packed fp32 instructions are emitted.
HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-ffp-contract=off",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
]
HIPCC_LINK = ["--offload-arch=gfx950", "-shared", "-fPIC"]


# Host-only sources (plain C++, no device code) go through the host compiler,
# so that host attributes such as per-ISA clones are available to them.
CXX_FLAGS = ["-O3", "-std=c++17", "-fPIC", "-ffp-contract=off", "-Wall"]


def sources() -> list[str]:
    csrc = os.path.join(PKG, "csrc")
    return sorted(glob.glob(os.path.join(csrc, "*.hip")) + glob.glob(os.path.join(csrc, "*.cpp")))


def _run(cmd: list[str], verbose: bool) -> None:
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    msgs = [ln for ln in (res.stdout + res.stderr).splitlines() if noise not in ln]
    if res.returncode != 0:
        raise RuntimeError(f"{cmd[0]} failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs))


def build(verbose: bool = False) -> str:
    """Compile every source into ``libsft.so`` (always recompiles): each
    source to an object (HIP sources with hipcc, host-only C++ with the host
    compiler, all at once), then one link."""
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    cxx = os.environ.get("SFT_CXX", "/opt/rocm/llvm/bin/clang++")
    inc = ["-I", os.path.join(ROOT, "include")]
    tmp = LIB + ".tmp"
    with tempfile.TemporaryDirectory() as objdir:
        jobs = []
        for src in sources():
            obj = os.path.join(objdir, os.path.basename(src) + ".o")
            if src.endswith(".cpp"):
                cmd = [cxx, *CXX_FLAGS, *inc, "-c", src, "-o", obj]
            else:
                cmd = [hipcc, *HIPCC_FLAGS, *inc, "-c", src, "-o", obj]
            if verbose:
                print(" ".join(cmd), flush=True)
            jobs.append((cmd, obj, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)))
        noise = "is not a recognized feature for this target"
        failed = []
        for cmd, _, proc in jobs:
            out = proc.communicate()[0]
            msgs = [ln for ln in out.splitlines() if noise not in ln]
            if proc.returncode != 0:
                failed.append(f"{cmd[0]} {cmd[-3]} failed:\n" + "\n".join(msgs))
            elif verbose and msgs:
                print("\n".join(msgs))
        if failed:
            raise RuntimeError("\n".join(failed))
        _run([hipcc, *HIPCC_LINK, "-o", tmp, *[obj for _, obj, _ in jobs]], verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
