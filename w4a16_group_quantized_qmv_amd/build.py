"""Build step: compile the HIP sources into the in-tree shared library ``libw4a16.so``.

``python -m w4a16_group_quantized_qmv_amd.build [--resource-usage]`` (also called by
``__graft_entry__.build()``).  Targets gfx950 only.  Packed fp32 instructions are disabled
(``-packed-fp32-ops``); hipcc's host pass reports that it does not know that feature, which is
harmless.
"""

from __future__ import annotations

import os
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libw4a16.so"
LIB_PATH = os.path.join(PKG_DIR, LIB_NAME)
SOURCES = ["abi.hip", "qmv.hip", "qmv_bits.hip", "qmv_burst.hip", "qmm.hip", "w4a8.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    return "hipcc"


def command(out_path: str = LIB_PATH, resource_usage: bool = False) -> list[str]:
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-Wall", "-Wno-unused-command-line-argument",
           "-I", INCLUDE, "-I", CSRC, "-o", out_path]
    if resource_usage:
        cmd += ["-Rpass-analysis=kernel-resource-usage"]
    cmd += [os.path.join(CSRC, s) for s in SOURCES]
    return cmd


PROBE_LIB_PATH = os.path.join(PKG_DIR, "libw4a16_probe.so")
PROBE_SOURCES = ["probe.hip"]


def _compile(cmd: list[str], tmp: str, out: str, verbose: bool, show: bool) -> None:
    if verbose:
        print(" ".join(cmd), flush=True)
    proc = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    log = "\n".join(line for line in (proc.stdout + proc.stderr).splitlines() if noise not in line)
    if proc.returncode != 0:
        raise RuntimeError(f"hipcc failed ({proc.returncode}):\n{log}")
    os.replace(tmp, out)
    if verbose or show:
        print(log)


def build(resource_usage: bool = False, verbose: bool = False) -> str:
    """Compile every HIP source into ``libw4a16.so`` next to this file, and the benchmark's
    streaming-read probe into ``libw4a16_probe.so``; returns the library's path."""
    tmp = LIB_PATH + ".tmp"
    _compile(command(tmp, resource_usage), tmp, LIB_PATH, verbose, resource_usage)
    ptmp = PROBE_LIB_PATH + ".tmp"
    pcmd = command(ptmp)
    pcmd = pcmd[:pcmd.index(os.path.join(CSRC, SOURCES[0]))] + [os.path.join(CSRC, s) for s in PROBE_SOURCES]
    _compile(pcmd, ptmp, PROBE_LIB_PATH, verbose, False)
    return LIB_PATH


if __name__ == "__main__":
    build(resource_usage="--resource-usage" in sys.argv, verbose=True)
