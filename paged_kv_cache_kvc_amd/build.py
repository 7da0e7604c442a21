"""Build libkvc.so in-tree for gfx950 (MI355X).

    python -m paged_kv_cache_kvc_amd.build

HIP kernels are compiled by hipcc; the host allocator, planner and C-ABI are
plain C++17 compiled by g++ against the HIP runtime headers; hipcc links the
shared library.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libkvc.so")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
ARCH = "gfx950"

HIP_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17",
    # packed fp32 VALU forms stay disabled: plain fp32 code is used instead
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
    # MFMA accumulators in VGPRs: avoids AGPR<->VGPR copies around every MFMA
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    # scores are never NaN (masked slots are -inf): max needs no NaN quieting
    "-fno-honor-nans",
    # leading scalar kernel arguments preloaded into scalar registers at
    # dispatch (the merge kernel's plan offsets)
    "-mllvm", "-amdgpu-kernarg-preload-count=16",
]
INCLUDE = os.path.join(os.path.dirname(HERE), "include")
HIP_FLAGS.append(f"-I{INCLUDE}")
CXX_FLAGS = ["-O2", "-fPIC", "-std=c++17", "-Wall", "-Wextra", "-Wno-unused-parameter",
             "-D__HIP_PLATFORM_AMD__", f"-I{ROCM}/include", f"-I{INCLUDE}"]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines()
                    if "packed-fp32-ops" not in l and "kernel-resource-usage" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"build step failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    if verbose and out.strip():
        print(out)
    return r.stdout


# Kernels that read unit entries with scalar loads issued in inline asm
# (unit_load): the compiler takes those registers as written at the asm, so
# an SGPR spill or copy of them before the matching wait would capture values
# still in flight.  No such kernel may spill SGPRs.
ASM_SCALAR_LOAD_KERNELS = ("attn_kernel",)


def check_no_scratch(remarks: str) -> None:
    """The attention kernels count their own direct-to-LDS loads with vmcnt
    waits; a register spill inside their loops would add scratch loads to that
    count (publishing a stage too early) or force a full drain.  Refuse any
    build in which a kernel uses scratch memory, or in which a kernel of
    ASM_SCALAR_LOAD_KERNELS spills SGPRs."""
    name = None
    bad = []
    for line in remarks.splitlines():
        if "Function Name:" in line:
            name = line.split("Function Name:")[1].split()[0]
        elif "ScratchSize [bytes/lane]:" in line:
            size = int(line.split("ScratchSize [bytes/lane]:")[1].split()[0])
            if size:
                bad.append(f"{name}: {size} bytes/lane of scratch")
        elif "SGPRs Spill:" in line:
            n = int(line.split("SGPRs Spill:")[1].split()[0])
            if n and name and any(k in name for k in ASM_SCALAR_LOAD_KERNELS):
                bad.append(f"{name}: {n} SGPRs spilled in a kernel with asm scalar loads")
    if bad:
        raise RuntimeError("kernels spill registers:\n  " + "\n  ".join(bad))


def build(verbose: bool = False) -> str:
    """Compile every source and link libkvc.so; always rebuilds."""
    hipcc = os.path.join(ROCM, "bin", "hipcc")
    cxx = shutil.which("g++") or "g++"
    os.makedirs(BUILD, exist_ok=True)
    objs = []
    for src in ("kvc_kernels.hip", "kvc_attn.hip"):
        o = os.path.join(BUILD, src.replace(".hip", ".o"))
        remarks = _run([hipcc, *HIP_FLAGS, "-Rpass-analysis=kernel-resource-usage", "-c",
                        os.path.join(CSRC, src), "-o", o], verbose)
        if "ScratchSize" not in remarks:
            raise RuntimeError(f"no kernel resource usage reported by hipcc for {src}")
        check_no_scratch(remarks)
        objs.append(o)
    for src in ("kvc_host.cpp", "kvc_api.cpp"):
        o = os.path.join(BUILD, src.replace(".cpp", ".o"))
        _run([cxx, *CXX_FLAGS, "-c", os.path.join(CSRC, src), "-o", o], verbose)
        objs.append(o)
    tmp = LIB + ".tmp"
    _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp,
          f"-L{ROCM}/lib", "-lamdhip64", f"-Wl,-rpath,{ROCM}/lib"], verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
