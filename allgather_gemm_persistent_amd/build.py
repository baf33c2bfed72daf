"""Build libagg.so (HIP, gfx950) in-tree with hipcc.

    python -m allgather_gemm_persistent_amd.build

The library is a plain C ABI (include/agg.h); it links the system HIP runtime, whose soname
(libamdhip64.so.7) is the one torch's own copy carries, so in a process that imported torch
first both share one runtime and torch's streams are valid handles for libagg.
"""

from __future__ import annotations

import os
import re
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libagg.so")
ARCH = "gfx950"

SOURCES = ["plan.cpp", "host.hip", "kernels.hip"]

HIP_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # no packed fp32 instructions in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libagg)")


# the GEMM kernel instantiations: agg::gemm_kernel<BM, BN, dtype, epilogue>
_GEMM_KERNEL = re.compile(r"_ZN3agg11gemm_kernelILi(\d+)ELi(\d+)ELi(\d+)ELi(\d+)EEEvNS_8GemmArgsE")
_REMARK = re.compile(r"remark: ([^:\[]*?): ([^\[]*?) \[-Rpass-analysis=kernel-resource-usage\]")
THREADS = 256   # one workgroup of 4 wave64s per CU


def kernel_resources(remarks: str) -> dict:
    """Per kernel (mangled name) the resource figures hipcc reports with
    -Rpass-analysis=kernel-resource-usage, e.g. {"VGPRs": 212, "AGPRs": 256, ...}."""
    out, cur = {}, None
    for line in remarks.splitlines():
        m = _REMARK.search(line)
        if not m:
            continue
        key, val = m.group(1).strip(), m.group(2).strip()
        if key == "Function Name":
            cur = out.setdefault(val, {})
        elif cur is not None:
            try:
                cur[key] = int(val.split()[0])
            except ValueError:
                cur[key] = val
    return out


def accumulator_problems(resources: dict) -> list:
    """GEMM kernels whose accumulators do not all fit the AGPRs the compiler gave them. The
    MFMAs are inline asm tied to AGPRs, and the hardware does not interlock other instructions'
    accumulator accesses against them; a kernel holding part of its accumulators in VGPRs (copied
    to and from the AGPRs around the MFMAs) computes wrong sums. Each thread holds
    BM * BN / THREADS fp32 accumulators."""
    problems = []
    for name, r in resources.items():
        m = _GEMM_KERNEL.fullmatch(name)
        if not m:
            continue
        bm, bn = int(m.group(1)), int(m.group(2))
        need = bm * bn // THREADS
        if int(r.get("AGPRs", 0)) < need:
            problems.append(f"gemm_kernel<{bm}, {bn}, {m.group(3)}, {m.group(4)}>: {r.get('AGPRs')} AGPRs "
                            f"for {need} accumulators per thread")
    return problems


def build(verbose: bool = True) -> str:
    """Compile every source and link libagg.so next to this file. Returns its path. The kernel
    source is compiled with the compiler's resource remarks (kept in _build/kernels.resources.txt);
    a GEMM kernel whose accumulators do not fit its AGPRs fails the build."""
    out_dir = os.path.join(ROOT, "_build")
    os.makedirs(out_dir, exist_ok=True)
    objs = []
    for src in SOURCES:
        obj = os.path.join(out_dir, src + ".o")
        cmd = [hipcc(), *HIP_FLAGS, "-I", os.path.join(ROOT, "include"), "-c",
               os.path.join(CSRC, src), "-o", obj]
        if src == "kernels.hip":
            cmd.append("-Rpass-analysis=kernel-resource-usage")
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, stderr=subprocess.PIPE, text=True)
        remarks = [l for l in r.stderr.splitlines() if "kernel-resource-usage" in l]
        # (the remarks' own source excerpts: "  749 | __global__ ..." and "      | ^")
        rest = "\n".join(l for l in r.stderr.splitlines()
                         if "kernel-resource-usage" not in l and not re.match(r"^\s*\d*\s*\|", l))
        if rest.strip():
            print(rest, file=sys.stderr, flush=True)
        if r.returncode != 0:
            raise subprocess.CalledProcessError(r.returncode, cmd)
        if src == "kernels.hip":
            text = "\n".join(remarks) + "\n"
            with open(os.path.join(out_dir, "kernels.resources.txt"), "w") as f:
                f.write(text)
            res = kernel_resources(text)
            if not any(_GEMM_KERNEL.fullmatch(n) for n in res):
                raise RuntimeError("no resource remarks for the GEMM kernels")
            bad = accumulator_problems(res)
            if bad:
                raise RuntimeError("accumulators outside the AGPRs: " + "; ".join(bad))
        objs.append(obj)
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs,
           "-Wl,-rpath,/opt/rocm/lib"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(verbose="-q" not in sys.argv)
