"""Build-time guards that need no GPU: the packed-fp32 check finds such
instructions when the compiler emits them and finds none in the library's
own device code; the inline-asm copies compile without reserved-register
warnings."""

import glob
import os
import shutil
import subprocess

import pytest

from dynamic_sparse_attention_vertical_amd import build as B

pytestmark = pytest.mark.skipif(not os.path.exists(B.HIPCC), reason="hipcc not installed")

PROBE = r'''
#include <hip/hip_runtime.h>
__global__ void probe(float2 *a, const float2 *b, float s) {
    const int i = threadIdx.x + blockIdx.x * blockDim.x;
    float2 x = a[i], y = b[i];
    x.x = x.x * y.x + s;
    x.y = x.y * y.y + s;
    a[i] = x;
}
'''


def _compile(tmp_path, extra):
    src = tmp_path / "probe.hip"
    src.write_text(PROBE)
    obj = tmp_path / ("probe%d.o" % len(extra))
    subprocess.run([B.HIPCC, f"--offload-arch={B.ARCH}", "-O3", *extra, "-c", str(src), "-o", str(obj)],
                   check=True, capture_output=True)
    return str(obj)


def test_packed_fp32_check_detects_and_flag_prevents(tmp_path):
    plain = _compile(tmp_path, [])
    assert B.PACKED_FP32.search(B.device_disassembly(plain)), "expected the compiler to pair the two FMAs"
    with pytest.raises(RuntimeError):
        B.check_device_code([plain])
    guarded = _compile(tmp_path, ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"])
    B.check_device_code([guarded])


def test_library_device_code_has_no_packed_fp32():
    objs = sorted(glob.glob(os.path.join(B.OBJDIR, "*.o")))
    if not objs:
        pytest.skip("library not built")
    B.check_device_code(objs)
    # the copies really are in the code, each with M0 saved and restored
    text = B.device_disassembly(os.path.join(B.OBJDIR, "attention.hip.o"))
    assert "global_load_lds_dwordx4" in text


def test_copies_compile_without_reserved_register_warnings(tmp_path):
    r = subprocess.run([B.HIPCC, *B.CFLAGS, "-c", os.path.join(B.CSRC, "attention.hip"),
                        "-o", str(tmp_path / "a.o")], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    assert "reserved registers" not in r.stderr
