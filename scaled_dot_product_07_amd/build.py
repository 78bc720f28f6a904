"""Build libsdpa07.so (HIP kernels for gfx950 + the C ABI) in-tree with hipcc.

Usage: python -m scaled_dot_product_07_amd.build   (or build() from Python)
"""

from __future__ import annotations

import concurrent.futures as cf
import os
import re
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT = os.path.join(PKG, "libsdpa07.so")
BUILD_DIR = os.path.join(ROOT, "_build")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-I", os.path.join(ROOT, "include"),
    # keep the compiler from emitting packed fp32 VALU ops (v_pk_fma_f32 and friends)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]
SOURCES = ["abi.cpp", "fwd.hip", "fwd_fp8.hip", "bwd.hip"]


_REMARK = re.compile(r"remark:\s+(Function Name|ScratchSize \[bytes/lane\]|VGPRs|AGPRs):\s*(\S+)")


def kernel_resources(remarks: str):
    """(kernel, VGPRs, AGPRs, scratch bytes per lane) from the compiler's
    kernel-resource-usage remarks."""
    out, cur = [], None
    for key, val in _REMARK.findall(remarks):
        if key == "Function Name":
            cur = {"name": val}
            out.append(cur)
        elif cur is not None:
            cur[key.split()[0]] = int(val)
    return [(k["name"], k.get("VGPRs", 0), k.get("AGPRs", 0), k.get("ScratchSize", 0))
            for k in out]


def _compile(src: str, extra) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    remarks = ["-Rpass-analysis=kernel-resource-usage"] if src.endswith(".hip") else []
    cmd = [HIPCC, *FLAGS, *remarks, *extra, *lang, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    if remarks:
        res = kernel_resources(r.stderr)
        with open(os.path.join(BUILD_DIR, os.path.basename(src) + ".resources.txt"), "w") as f:
            for name, vg, ag, sc in res:
                f.write(f"{name} vgpr={vg} agpr={ag} scratch={sc}\n")
        # The kernels count their own vmcnt waits around the direct-to-LDS loads
        # and rely on the register budget they were written for: a spill would
        # add scratch loads and stores to those counts (LDS reads could then run
        # ahead of the loads they wait for) and slow every step. Refuse it.
        spilled = [(n, sc) for n, _, _, sc in res if sc > 0]
        if spilled:
            raise RuntimeError(f"{src}: kernels use scratch (register spills): {spilled}")
    return obj


def build(extra=(), verbose: bool = False) -> str:
    """Compile every source for gfx950 and link libsdpa07.so next to this file."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(lambda s: _compile(s, list(extra)), SOURCES))
    tmp = OUT + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, OUT)
    if verbose:
        print(f"built {OUT}")
    return OUT


if __name__ == "__main__":
    build(extra=sys.argv[1:], verbose=True)
