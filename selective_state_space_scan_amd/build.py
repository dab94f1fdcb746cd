"""Compiles the HIP library (``libssmscan.so``) for gfx950 in-tree.

The build is one hipcc invocation over the forward and backward sources, and
one for the benchmark's peak-rate microbenchmarks (``libssmpeaks.so``); it
always recompiles when called.
Packed fp32 VALU instructions are disabled for every HIP source
(``-target-feature -packed-fp32-ops``).
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
REPO_DIR = os.path.dirname(PKG_DIR)
SRCS = [os.path.join(PKG_DIR, "csrc", f) for f in ("ssm_scan.hip", "ssm_scan_bwd.hip")]
INCLUDE_DIR = os.path.join(REPO_DIR, "include")
LIB_PATH = os.path.join(PKG_DIR, "libssmscan.so")
# The peak-rate microbenchmarks the benchmark measures the roofline with: a
# library of their own, not part of the scan.
PEAKS_SRC = os.path.join(PKG_DIR, "csrc", "ssm_peaks.hip")
PEAKS_LIB_PATH = os.path.join(PKG_DIR, "libssmpeaks.so")
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise FileNotFoundError("hipcc not found (ROCm toolchain required to build the HIP library)")


def compile_command(out: str = LIB_PATH, srcs: list[str] | None = None) -> list[str]:
    srcs = SRCS if srcs is None else srcs
    return [
        hipcc(), "-O3", "-std=c++20", f"--offload-arch={ARCH}",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-fPIC", "-shared", "-Wall", f"-I{INCLUDE_DIR}",
        "-o", out, *[s for s in srcs if os.path.exists(s)],
    ]


def _compile(out: str, srcs: list[str], verbose: bool) -> str:
    tmp = out + f".tmp{os.getpid()}"
    cmd = compile_command(tmp, srcs)
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass warns that it does not know the packed-fp32 feature; that is harmless.
    noise = "is not a recognized feature for this target"
    msgs = "\n".join(l for l in (res.stdout + res.stderr).splitlines() if noise not in l)
    if res.returncode != 0:
        if os.path.exists(tmp):
            os.remove(tmp)
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{msgs}")
    if verbose and msgs.strip():
        print(msgs, file=sys.stderr)
    os.replace(tmp, out)
    return out


def build(verbose: bool = False) -> str:
    """Compile ``libssmscan.so`` (and the benchmark's ``libssmpeaks.so``) next
    to this file and return the scan library's path."""
    _compile(PEAKS_LIB_PATH, [PEAKS_SRC], verbose)
    return _compile(LIB_PATH, SRCS, verbose)


if __name__ == "__main__":
    print(build(verbose=True))
