"""Build libmsa.so (the HIP kernels and the C-ABI layer) for gfx950 with hipcc.

    python -m dynamic_sparse_attention_vertical_amd.build

Objects go to _build/msa/ at the repository root; the shared library is written
next to this file, where the binding loads it from.
"""

from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import re
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libmsa.so")
OBJDIR = os.path.join(ROOT, "_build", "msa")

ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
LLVM_BIN = os.environ.get("ROCM_LLVM_BIN", "/opt/rocm/llvm/bin")
CFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # No packed-fp32 instructions (v_pk_{add,mul,fma}_f32) in the device code.
    # The host (x86) pass of hipcc does not know this feature and says it
    # ignores it; the gfx950 pass honours it, and check_device_code() below
    # verifies the result on every build.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]
# Warnings that fail the build: an inline-asm block that clobbers a reserved
# register (the compiler ignores such a clobber and would assume the register
# unchanged).
FATAL_WARNINGS = ("-Winline-asm",)
PACKED_FP32 = re.compile(r"\bv_pk_(add|mul|fma)_f32\b")


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(OBJDIR, os.path.basename(src) + ".o")
    cmd = [HIPCC, *CFLAGS, "-c", src, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    bad = [ln for ln in r.stderr.splitlines() if any(w in ln for w in FATAL_WARNINGS)]
    if bad:
        raise RuntimeError(f"hipcc warnings that must not occur in {src}:\n" + "\n".join(bad[:10]))
    return obj


def device_disassembly(obj: str) -> str:
    """gfx950 disassembly of the device code hipcc embedded in an object file
    (its offload bundle, in the .hip_fatbin section; "" if it has none)."""
    secs = subprocess.run([os.path.join(LLVM_BIN, "llvm-readelf"), "-S", obj], check=True,
                          capture_output=True, text=True).stdout
    if ".hip_fatbin" not in secs:
        return ""
    with tempfile.TemporaryDirectory() as td:
        fat, co = os.path.join(td, "fatbin"), os.path.join(td, "dev.co")
        subprocess.run([os.path.join(LLVM_BIN, "llvm-objcopy"), f"--dump-section=.hip_fatbin={fat}", obj,
                        os.path.join(td, "stripped.o")], check=True, capture_output=True)
        subprocess.run([os.path.join(LLVM_BIN, "clang-offload-bundler"), "--type=o",
                        f"--targets=hipv4-amdgcn-amd-amdhsa--{ARCH}", f"--input={fat}", f"--output={co}",
                        "--unbundle"], check=True, capture_output=True)
        r = subprocess.run([os.path.join(LLVM_BIN, "llvm-objdump"), "-d", co], check=True,
                           capture_output=True, text=True)
        return r.stdout


def check_device_code(objs) -> None:
    """Fail if any packed-fp32 instruction made it into the device code."""
    for obj in objs:
        hits = PACKED_FP32.findall(device_disassembly(obj))
        if hits:
            raise RuntimeError(f"{obj}: {len(hits)} packed-fp32 instructions in the gfx950 code")


def build(verbose: bool = False, jobs: int = 8) -> str:
    """Compile every kernel source and link libmsa.so; returns its path."""
    os.makedirs(OBJDIR, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    with cf.ThreadPoolExecutor(max_workers=max(1, min(jobs, len(srcs)))) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), srcs))
    check_device_code(objs)
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
