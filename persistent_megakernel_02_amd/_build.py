"""Build of the HIP library (libmk.so) for gfx950 with hipcc, in-tree.

Every translation unit is compiled with the compiler's kernel resource remarks;
the registers and scratch bytes of each kernel are written to
_build/kernel_resources.json, so a change that pushes the persistent kernel past
its register budget into scratch memory is caught on the CPU."""
from __future__ import annotations

import json
import os
import re
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libmk.so")
SOURCES = ["mk_kernels_valu.hip", "mk_kernels_mfma.hip", "mk_kernels_moe.hip", "mk_kernels_chunk.hip", "host.hip",
           "megakernel.hip", "conventional.hip", "bench_kernels.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
         # packed fp32 VALU forms stay off (v_pk_fma_f32 and friends)
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


RESOURCES = os.path.join(PKG, "_build", "kernel_resources.json")
_REMARK = re.compile(r"remark:\s+(Function Name|VGPRs|AGPRs|ScratchSize \[bytes/lane\]|Occupancy \[waves/SIMD\]):\s*(\S+)")


def _resources(stderr: str) -> dict:
    """{kernel symbol: {"vgpr", "agpr", "scratch", "occupancy"}} from the remarks."""
    out, cur = {}, None
    keys = {"VGPRs": "vgpr", "AGPRs": "agpr", "ScratchSize [bytes/lane]": "scratch", "Occupancy [waves/SIMD]": "occupancy"}
    for m in _REMARK.finditer(stderr):
        k, v = m.group(1), m.group(2)
        if k == "Function Name":
            cur = out.setdefault(v, {})
        elif cur is not None:
            cur[keys[k]] = int(v)
    return out


def build(verbose: bool = False, jobs: int = 7) -> str:
    objdir = os.path.join(PKG, "_build")
    os.makedirs(objdir, exist_ok=True)

    def compile_one(src: str):
        obj = os.path.join(objdir, src.replace(".hip", ".o"))
        cmd = [HIPCC, *FLAGS, "-Rpass-analysis=kernel-resource-usage", "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        err = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l and "remark:" not in l)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed for {src}:\n{err}")
        if err.strip() and verbose:
            print(err, file=sys.stderr)
        return obj, _resources(r.stderr)

    with ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        done = list(ex.map(compile_one, SOURCES))
    objs = [o for o, _ in done]
    res = {}
    for _, r in done:
        res.update(r)
    with open(RESOURCES, "w") as f:
        json.dump(res, f, indent=1, sort_keys=True)
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
