"""Build-level check of the shared elementwise steps (CPU: hipcc cross-compiles for gfx950).

Several kernels must round the RoPE rotation and the RMS tile sums with the
same bits (a decode step equals the last row of a prefill; the verify that
reuses the draft's state equals the one that recomputes it).  The toolchain's
__fmul_rn / __fadd_rn are plain operators that the compiler may fuse into a
fused multiply-add, choosing which product to fuse kernel by kernel, so the
shared helpers use operations with contraction turned off.  This test compiles
small kernels around the helpers to gfx950 assembly and checks that no fused
multiply-add appears, and that the same expression written with __fmul_rn /
__fadd_rn does fuse (so the check can see the difference)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "self_speculative_layer_amd", "csrc")
HIPCC = "/opt/rocm/bin/hipcc"

PROBE = r"""
#include <hip/hip_runtime.h>
#include "common.h"
__global__ void rot(const float* x, const float2* cs, float* y) {
  float a, b;
  ssd::rope_apply(x[threadIdx.x], x[threadIdx.x + 64], cs[threadIdx.x], a, b);
  y[threadIdx.x] = a;
  y[threadIdx.x + 64] = b;
}
__global__ void tiles(const float* x, float* y) { y[threadIdx.x] = ssd::tile16_ss_lanes(x[threadIdx.x]); }
"""

PLAIN = r"""
#include <hip/hip_runtime.h>
__global__ void rot(const float* x, const float2* cs, float* y) {
  const float x1 = x[threadIdx.x], x2 = x[threadIdx.x + 64];
  const float2 c = cs[threadIdx.x];
  y[threadIdx.x] = __fsub_rn(__fmul_rn(x1, c.x), __fmul_rn(x2, c.y));
  y[threadIdx.x + 64] = __fadd_rn(__fmul_rn(x2, c.x), __fmul_rn(x1, c.y));
}
"""


def _asm(tmp_path, src):
    p = tmp_path / "probe.hip"
    p.write_text(src)
    out = tmp_path / "probe.s"
    cmd = [HIPCC, "-O3", "--offload-arch=gfx950", "-std=c++17", "-Xclang", "-target-feature", "-Xclang",
           "-packed-fp32-ops", "-I" + CSRC, "--cuda-device-only", "-S", str(p), "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return out.read_text()


def _fused(asm):
    return [l for l in asm.splitlines() if l.strip().startswith(("v_fma_f32", "v_fmac_f32", "v_pk_fma"))]


@pytest.mark.skipif(not shutil.which(HIPCC) and not os.path.exists(HIPCC), reason="hipcc not installed")
def test_shared_steps_are_not_fused(tmp_path):
    asm = _asm(tmp_path, PROBE)
    assert "v_sub_f32" in asm and "v_mul_f32" in asm
    assert _fused(asm) == []


@pytest.mark.skipif(not shutil.which(HIPCC) and not os.path.exists(HIPCC), reason="hipcc not installed")
def test_rounding_intrinsics_alone_would_fuse(tmp_path):
    assert _fused(_asm(tmp_path, PLAIN)), "the check no longer distinguishes fused from unfused code"
