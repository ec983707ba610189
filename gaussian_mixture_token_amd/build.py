"""Build libgma.so (HIP, gfx950) in-tree with hipcc.

Each source under csrc/ is compiled to an object in _build/ (in parallel), then linked into
gaussian_mixture_token_amd/libgma.so.  Every call rebuilds from scratch; nothing is cached
across calls except the output library itself.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import re
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_PATH = os.path.join(PKG, "libgma.so")
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
# Packed fp32 VALU instructions are disabled for all device code.
# Matrix-core results stay in VGPRs (the token-split kernels keep their [a | b] operands in AGPRs,
# where the MFMAs read them directly).
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-mllvm", "-amdgpu-mfma-vgpr-form"]
COMMON_FLAGS = ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-Wall",
                "-Wno-unused-function", "-I" + os.path.join(ROOT, "include"), "-I" + CSRC]


def sources():
    out = []
    for name in sorted(os.listdir(CSRC)):
        if name.endswith(".hip") or name.endswith(".cpp"):
            out.append(os.path.join(CSRC, name))
    return out


RESOURCE_REMARK = "-Rpass-analysis=kernel-resource-usage"


# Kernels known to spill vector registers to scratch memory, each with its reason.  Both are register-
# staged output passes (plain loads, waits placed by the compiler, so scratch accesses are counted
# correctly) of shapes outside the token-split classes: fp32 K = d_r = d_v = 128, and bf16 K = 256 with
# d_r, d_v up to 128.  Their spills cost time, not correctness.
SCRATCH_ALLOWED = {
    "_ZN3gma11main_kernelILb1ELi128ELi128ELi128ELi4ELi32ELi3ELb0ELi1EEEvNS_8MainArgsE",
    "_ZN3gma11main_kernelILb0ELi256ELi128ELi128ELi4ELi32ELi3ELb0ELi1EEEvNS_8MainArgsE",
}


def _check_resources(src: str, remarks: str) -> None:
    """Every kernel must run without scratch memory (SCRATCH_ALLOWED aside): the DMA-staged kernels
    count their outstanding vector-memory operations exactly (s_waitcnt vmcnt(N)), and scratch loads
    and stores would add to that count; elsewhere a spill is a slowdown that should not go unnoticed.
    (Scalar registers spilled into vector-register lanes use no memory.)"""
    cur = None
    bad = []
    for line in remarks.splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            cur = m.group(1)
            continue
        # "remark: <file>:<line>:<col>:     ScratchSize [bytes/lane]: N" (the location may also come
        # before "remark:")
        m = re.search(r"\s(VGPRs Spill|ScratchSize \[bytes/lane\]): (\d+)", line)
        if m and cur and int(m.group(2)) != 0 and cur not in SCRATCH_ALLOWED:
            bad.append("%s: %s = %s" % (cur, m.group(1), m.group(2)))
    if bad:
        raise RuntimeError("kernels in %s use scratch memory:\n  %s" % (src, "\n  ".join(bad)))


# Kernels that wait for their LDS-DMA prefetch with exact vmcnt counts: the token-split kernels, the
# LDS-DMA staged main_kernel instantiations (template argument DMA = true, the eighth) and the fused
# backward row kernel.
EXACT_VMCNT_KERNELS = re.compile(
    r"^(_ZN3gma10tok_kernel\S*|_ZN3gma11main_kernelILb[01](?:ELi-?\d+){6}ELb1\S*|"
    r"_ZN3gma12_GLOBAL__N_121bwd_fused_rows_kernel\S*):", re.M)
# sources whose assembly must hold such kernels (a check that finds none has a stale pattern)
EXACT_VMCNT_SOURCES = ("gma_classes_bf16", "gma_backward")


def _check_vmem_in_loops(asm_path: str) -> int:
    """The exact vmcnt counts hold only if the chunk loop issues no vector-memory operation other
    than the DMA loads (buffer_load ... lds) and the output stores.  Checked on the assembly after
    the first barrier (everything before it is the prologue): no scratch access, no other loads.
    Returns the number of kernels checked."""
    text = open(asm_path).read()
    n_checked = 0
    for m in EXACT_VMCNT_KERNELS.finditer(text):
        name = m.group(1)
        body = text[m.end(): text.index("s_endpgm", m.end())]
        loop = body[body.index("s_barrier"):] if "s_barrier" in body else ""
        bad = []
        for line in loop.splitlines():
            t = line.strip().split()
            if not t:
                continue
            op = t[0]
            # (global stores: only the aggregate epilogue, after the loop)
            if op.startswith(("global_load", "global_atomic", "flat_", "scratch_")) or \
                    (op.startswith("buffer_load") and not line.rstrip().endswith(" lds")):
                bad.append(line.strip())
        if bad:
            raise RuntimeError("%s: unexpected vector-memory operations in the chunk loop:\n  %s" % (name, "\n  ".join(bad[:8])))
        n_checked += 1
    return n_checked


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    extra = [RESOURCE_REMARK]
    if src.endswith(".hip"):
        extra += ["-save-temps=obj"]
    cmd = [HIPCC] + COMMON_FLAGS + DEVICE_FLAGS + extra + ["-c", src, "-o", obj]
    if src.endswith(".cpp"):
        cmd = [HIPCC, "-x", "hip"] + COMMON_FLAGS + DEVICE_FLAGS + extra + ["-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True, cwd=BUILD_DIR)
    lines = [l for l in r.stderr.splitlines() if "not a recognized feature" not in l]
    remarks = "\n".join(l for l in lines if "kernel-resource-usage" in l)
    err = "\n".join(l for l in lines if "kernel-resource-usage" not in l)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s" % (src, err))
    warnings = [l for l in err.splitlines() if "warning:" in l]
    if warnings:
        sys.stderr.write("\n".join(warnings) + "\n")
    _check_resources(src, remarks)
    if src.endswith(".hip"):
        base = os.path.splitext(os.path.basename(obj))[0]
        for name in os.listdir(BUILD_DIR):
            if name.startswith(base.replace(".hip", "")) and name.endswith("gfx950.s"):
                n = _check_vmem_in_loops(os.path.join(BUILD_DIR, name))
                if n == 0 and name.startswith(EXACT_VMCNT_SOURCES):
                    raise RuntimeError("%s: no exact-vmcnt kernel found to check (stale pattern?)" % name)
    return obj


def build_library(jobs: int | None = None, verbose: bool = True) -> str:
    if os.path.isdir(BUILD_DIR):
        shutil.rmtree(BUILD_DIR)
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = sources()
    jobs = jobs or min(8, os.cpu_count() or 1)
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB_PATH + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stderr)
    os.replace(tmp, LIB_PATH)
    if verbose:
        print("built %s (%d sources)" % (LIB_PATH, len(srcs)))
    return LIB_PATH


if __name__ == "__main__":
    build_library()
