"""Compiles the HIP library (``libssmscan.so``) for gfx950 in-tree.

Each source is compiled to an object with its own flags and the objects are
linked into one shared library; the benchmark's peak-rate microbenchmarks
(``libssmpeaks.so``) are a second library.  Every call recompiles.
Packed fp32 VALU instructions are disabled for every HIP source
(``-target-feature -packed-fp32-ops``).
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys
import tempfile

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


# Flags of one source beyond the common ones.  The forward is scheduled with
# the AMDGPU backend's memory-clause strategy, which keeps a tile's loads
# together: 1-4 % faster on every forward workload (same-GPU comparison);
# the backward keeps the default, which was 0.7 % faster for it.
SRC_FLAGS = {"ssm_scan.hip": ["-mllvm", "-amdgpu-sched-strategy=max-memory-clause"]}


def _common() -> list[str]:
    return [hipcc(), "-O3", "-std=c++20", f"--offload-arch={ARCH}",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-fPIC", "-Wall", f"-I{INCLUDE_DIR}"]


def object_command(obj: str, src: str) -> list[str]:
    return [*_common(), *SRC_FLAGS.get(os.path.basename(src), []), "-c", src, "-o", obj]


def link_command(out: str, objs: list[str]) -> list[str]:
    return [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", out, *objs]


def _run(cmd: list[str], verbose: bool) -> None:
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass warns that it does not know the packed-fp32 feature; that is harmless.
    noise = "is not a recognized feature for this target"
    msgs = "\n".join(l for l in (res.stdout + res.stderr).splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{msgs}")
    if verbose and msgs.strip():
        print(msgs, file=sys.stderr)


def _compile(out: str, srcs: list[str], verbose: bool) -> str:
    """Objects of `srcs`, linked into the shared library `out` (replaced only
    once the link succeeded)."""
    tmp = out + f".tmp{os.getpid()}"
    with tempfile.TemporaryDirectory(prefix="ssmbuild") as d:
        objs = [os.path.join(d, os.path.splitext(os.path.basename(src))[0] + ".o") for src in srcs]
        # one hipcc per source, side by side
        with concurrent.futures.ThreadPoolExecutor(max_workers=len(srcs)) as pool:
            for f in [pool.submit(_run, object_command(o, src), verbose) for o, src in zip(objs, srcs)]:
                f.result()
        try:
            _run(link_command(tmp, objs), verbose)
        except RuntimeError:
            if os.path.exists(tmp):
                os.remove(tmp)
            raise
    os.replace(tmp, out)
    return out


def build(verbose: bool = False) -> str:
    """Compile ``libssmscan.so`` (and the benchmark's ``libssmpeaks.so``) next
    to this file and return the scan library's path."""
    _compile(PEAKS_LIB_PATH, [PEAKS_SRC], verbose)
    return _compile(LIB_PATH, SRCS, verbose)


if __name__ == "__main__":
    print(build(verbose=True))
