"""Builds libw4a16.so (gfx950 only) in-tree with hipcc.

    python -m weight_only_int4_02_amd.build
"""
from __future__ import annotations

import os
import re
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_PATH = os.path.join(PKG, "libw4a16.so")

SOURCES = ["w4a16_host.cpp", "w4a16_api.hip", "w4a16_kernels.hip", "w4a16_gemm.hip",
           "w4a16_small_jpg1.hip", "w4a16_small_jpg2.hip", "w4a16_small_jpg4.hip",
           "w4a16_small_jpg1_bf16.hip", "w4a16_small_jpg2_bf16.hip", "w4a16_small_jpg4_bf16.hip",
           "w4a16_large.hip", "w4a16_large_bf16.hip", "w4a16_quantize.hip",
           "w4a16_stream.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
# One target only.  Packed fp32 instructions are switched off for the device
# code (the kernels do their fp32 work in MFMA accumulators and plain VALU).
COMMON = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall",
          "-I" + INCLUDE, "-I" + CSRC,
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


_FUNC = re.compile(r"Function Name: (\S+)")
_SPILL = re.compile(r"(ScratchSize \[bytes/lane\]|VGPRs Spill): (\d+)")


def spilled_kernels(remarks: str) -> list:
    """(kernel, what, amount) for every kernel whose resource-usage remarks
    report scratch or spilled vector registers (scalar registers spill into
    lanes of a reserved vector register, which no load writes)."""
    out, name = [], None
    for line in remarks.splitlines():
        m = _FUNC.search(line)
        if m:
            name = m.group(1)
            continue
        m = _SPILL.search(line)
        if m and name and int(m.group(2)) > 0:
            out.append((name, m.group(1), int(m.group(2))))
    return out


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    lang = ["-x", "hip", "-Rpass-analysis=kernel-resource-usage"] if src.endswith(".hip") else []
    cmd = [HIPCC] + COMMON + lang + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    # The kernels wait for their loads explicitly (the compiler does not see
    # them in flight): a register spilled or reloaded between a load and its
    # wait would hold stale data, so any kernel that spills is a build error.
    bad = spilled_kernels(r.stderr)
    if bad:
        lines = "\n".join(f"  {k}: {what} {n}" for k, what, n in bad)
        raise RuntimeError(f"{src}: kernels spill registers:\n{lines}")
    if src.endswith(".hip"):
        _check_inflight(src)
    return obj


def _check_inflight(src: str) -> None:
    """A copy or reuse of a register whose load is still in flight is not a
    spill, so the remarks above miss it (the compiler has split such live
    ranges into AGPRs under register pressure): the device assembly of the
    same compile is checked against a model of the load counter
    (vmcheck.py), and any kernel that names such a register fails the build."""
    from . import vmcheck

    asm = os.path.join(BUILD_DIR, os.path.basename(src) + ".s")
    cmd = [HIPCC] + COMMON + ["-x", "hip", "--offload-device-only", "-S",
                              os.path.join(CSRC, src), "-o", asm]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    with open(asm) as f:
        found = vmcheck.check_asm(f.read())
    if found:
        lines = "\n".join(f"  {vmcheck.demangle(k)}: line {v[0][0]} {v[0][1]!r}"
                          for k, v in found.items())
        raise RuntimeError(f"{src}: kernels name registers of loads still in flight "
                           f"({asm}):\n{lines}")


def build_library(verbose: bool = False) -> str:
    """Compiles every source and links libw4a16.so; always rebuilds."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB_PATH + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB_PATH)
    if verbose:
        print("built", LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    build_library(verbose=True)
    sys.exit(0)
