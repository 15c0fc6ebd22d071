"""Build libbakron.so (HIP, gfx950) in-tree with hipcc.

The library is written for gfx950 only. Packed fp32 instructions are disabled
(-packed-fp32-ops) for every device compile. In the LDL the fp64 MFMA
instructions take their accumulators in ordinary VGPRs (-amdgpu-mfma-vgpr-form):
with accumulation registers the compiler copied every tile's accumulators
between the two register files on each pass of the k-loop. The Hessian kernels
measured a few per cent slower with the option, so it is set per file.

The build fails if any kernel spills registers to scratch memory: several kernels
count their own loads in flight with explicit s_waitcnt vmcnt(N) (the direct-to-LDS
rings of the Hessian and the solve's far field), and spill loads and stores would
enter that count and let a wait end before the data it waits for has landed.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OUT_DIR = os.path.join(HERE, "_build")
LIB = os.path.join(OUT_DIR, "libbakron.so")
SOURCES = ["bk_api.hip", "bk_accum.hip", "bk_ldl.hip", "bk_solve.hip", "bk_rotate.hip", "bk_report.hip", "bk_sketch.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

CFLAGS = [
    "--offload-arch=" + ARCH, "-O3", "-fPIC", "-std=c++17", "-Wall", "-Wno-unused-result",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(os.path.dirname(HERE), "include"),
]
FILE_FLAGS = {"bk_ldl.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def _scratch_users(remarks: str):
    """(function, bytes per lane) for every function the resource remarks show with scratch."""
    out, name = [], None
    for ln in remarks.splitlines():
        if "remark:" not in ln:
            continue
        if "Function Name:" in ln:
            name = ln.split("Function Name:")[1].split("[")[0].strip()
        elif "ScratchSize [bytes/lane]:" in ln and name:
            n = int(ln.split("ScratchSize [bytes/lane]:")[1].split("[")[0].strip())
            if n > 0:
                out.append((name, n))
    return out


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(OUT_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *CFLAGS, *FILE_FLAGS.get(src, []), "-Rpass-analysis=kernel-resource-usage", "-c",
           os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), file=sys.stderr)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s%s" % (src, r.stdout, r.stderr))
    spills = _scratch_users(r.stderr)
    if spills:
        raise RuntimeError("%s: kernels spill to scratch memory (%s); the explicit vmcnt waits "
                           "assume none" % (src, ", ".join("%s %d B/lane" % x for x in spills)))
    warn = [ln for ln in r.stderr.splitlines()
            if "warning" in ln and "packed-fp32-ops" not in ln]
    if verbose and warn:
        print("\n".join(warn), file=sys.stderr)
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(OUT_DIR, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(4, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), file=sys.stderr)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
