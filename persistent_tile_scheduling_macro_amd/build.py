"""Build libpgemm.so (the HIP kernels and the C-ABI host code) for gfx950.

Each translation unit is compiled in parallel with hipcc, then linked into
one shared library next to this file. Run as ``python -m
persistent_tile_scheduling_macro_amd.build`` or through
``__graft_entry__.build()``.

The compiler's per-kernel resource remarks (VGPRs, AGPRs, SGPRs, scratch
bytes per lane, occupancy, LDS) are collected from the same compile and
written to _build/kernel_resources.txt. The build fails if a kernel that
timed runs can launch -- every kernel but the tile-trace instantiations --
uses scratch memory (register spills), since a spill inside the k-loop costs
a memory round trip per step.
"""
from __future__ import annotations

import os
import re
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libpgemm.so")
BUILD_DIR = os.path.join(HERE, "_build")
SOURCES = ["pgemm.hip", "kernels_f16.hip", "kernels_bf16.hip", "kernels_f8.hip", "kernels_pp_f16.hip",
           "kernels_pp_bf16.hip", "kernels_pp_f8.hip", "kernels_pw_f16.hip", "kernels_pw_bf16.hip", "kernels_pw_f8.hip",
           "hold.hip"]
ARCH = os.environ.get("PGEMM_ARCH", "gfx950")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# -packed-fp32-ops: keep hipcc from emitting packed fp32 VALU ops.
FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Wall",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


RESOURCES = os.path.join(BUILD_DIR, "kernel_resources.txt")
_FIELDS = {"VGPRs": "vgpr", "AGPRs": "agpr", "TotalSGPRs": "sgpr", "ScratchSize [bytes/lane]": "scratch",
           "Occupancy [waves/SIMD]": "occupancy", "LDS Size [bytes/block]": "lds"}


def parse_resource_remarks(text: str) -> list:
    """Per-kernel records from hipcc's -Rpass-analysis=kernel-resource-usage remarks."""
    out, cur = [], None
    for line in text.splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            cur = {"name": m.group(1)}
            out.append(cur)
            continue
        m = re.search(r"remark:\s+(TotalSGPRs|VGPRs|AGPRs|ScratchSize \[bytes/lane\]|Occupancy \[waves/SIMD\]|"
                      r"LDS Size \[bytes/block\]): (\d+)", line)
        if m and cur is not None:
            cur[_FIELDS[m.group(1)]] = int(m.group(2))
    return out


def is_traced(name: str) -> bool:
    """Tile-trace instantiation of a fast kernel: its first bool template argument (TRACE) is true."""
    m = re.search(r"(gemm_fast_kernel|gemm_pp_kernel|gemm_pw_kernel)I(?:Li\d+E)+Lb(\d)E", name)
    return bool(m and m.group(2) == "1")


def _compile(src: str):
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, "-Rpass-analysis=kernel-resource-usage", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj, parse_resource_remarks(r.stderr)


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 1)) as ex:
        results = list(ex.map(_compile, SOURCES))
    objs = [o for o, _ in results]
    kernels = sorted({k["name"]: k for _, ks in results for k in ks}.values(), key=lambda k: k["name"])
    with open(RESOURCES, "w") as f:
        f.write("# kernel  vgpr agpr sgpr scratch_bytes_per_lane occupancy_waves_per_simd lds_bytes traced\n")
        for k in kernels:
            f.write(f"{k['name']} {k.get('vgpr', -1)} {k.get('agpr', -1)} {k.get('sgpr', -1)} {k.get('scratch', -1)} "
                    f"{k.get('occupancy', -1)} {k.get('lds', -1)} {int(is_traced(k['name']))}\n")
    spills = [k["name"] for k in kernels if k.get("scratch", 0) > 0 and not is_traced(k["name"])]
    if spills:
        raise RuntimeError("kernels that timed runs launch use scratch memory (register spills): "
                           + ", ".join(spills) + f" (see {RESOURCES})")
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
