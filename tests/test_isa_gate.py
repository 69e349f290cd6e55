"""The structured-sparse gate (row a8): which sparse MFMA forms gfx950 has.

The MXFP4 backbone could use a 2:4 sparse MFMA on its own operand type only
if gfx950 had one for FP4 operands.  The ROCm assembler and compiler for
gfx950 decide it: the block-scaled FP4 MFMA and the fp16 and FP8 2:4 SMFMACs
exist (the kernels use all three); no SMFMAC form takes FP4 / f8f6f4
operands, and clang has no builtin for one.  So the MXFP4 GEMM runs its
backbone on the dense FP4 MFMA by default, and its SPARSE_MFMA variant
converts the backbone to FP8 (exact after a per-row power-of-two rebasing)
for the FP8 SMFMAC.  Host-only: nothing here runs on a GPU."""
import os
import subprocess

import pytest

LLVM_MC = "/opt/rocm/llvm/bin/llvm-mc"
HIPCC = "/opt/rocm/bin/hipcc"

ACCEPTED = [
    # the MX GEMM's MFMA: FP4 x FP4 (cbsz = blgp = 4), per-lane E8M0 scales
    "v_mfma_scale_f32_32x32x64_f8f6f4 a[0:15], v[0:3], v[4:7], a[0:15], v8, v9 op_sel_hi:[0,0,0] cbsz:4 blgp:4",
    "v_mfma_scale_f32_16x16x128_f8f6f4 a[0:3], v[0:3], v[4:7], a[0:3], v8, v9 op_sel_hi:[0,0,0] cbsz:4 blgp:4",
    # the NV GEMM's 2:4 sparse MFMA on fp16 operands
    "v_smfmac_f32_32x32x32_f16 v[0:15], v[16:19], v[20:27], v28",
    # the MX GEMM's SPARSE_MFMA variant: the backbone rebased to FP8 on the FP8 2:4 MFMA
    "v_smfmac_f32_32x32x64_fp8_fp8 v[0:15], v[16:19], v[20:27], v28",
    "v_smfmac_f32_16x16x128_fp8_fp8 v[0:3], v[4:7], v[8:15], v16",
    "v_smfmac_f32_16x16x64_f16 v[0:3], v[4:7], v[8:15], v16",
]

REJECTED = [
    "v_smfmac_f32_16x16x128_f8f6f4 v[0:3], v[4:7], v[8:15], v16",
    "v_smfmac_f32_32x32x64_f8f6f4 v[0:15], v[16:19], v[20:27], v28",
    "v_smfmac_f32_16x16x256_f8f6f4 v[0:3], v[4:7], v[8:15], v16",
    "v_smfmac_scale_f32_16x16x128_f8f6f4 v[0:3], v[4:7], v[8:15], v16",
    "v_smfmac_f32_16x16x128_fp4_fp4 v[0:3], v[4:7], v[8:15], v16",
]


def _assemble(line, tmp_path):
    src = tmp_path / "probe.s"
    src.write_text(line + "\n")
    return subprocess.run([LLVM_MC, "-arch=amdgcn", "-mcpu=gfx950", str(src), "-o", os.devnull],
                          capture_output=True, text=True)


needs_mc = pytest.mark.skipif(not os.path.exists(LLVM_MC), reason="ROCm llvm-mc not installed")
needs_hipcc = pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not installed")


@needs_mc
@pytest.mark.parametrize("line", ACCEPTED)
def test_accepted_forms_assemble(line, tmp_path):
    r = _assemble(line, tmp_path)
    assert r.returncode == 0, r.stderr


@needs_mc
@pytest.mark.parametrize("line", REJECTED)
def test_sparse_fp4_forms_do_not_exist(line, tmp_path):
    r = _assemble(line, tmp_path)
    assert r.returncode != 0 and "invalid instruction" in r.stderr, (r.returncode, r.stderr)


def _compile_device(body, tmp_path):
    src = tmp_path / "probe.hip"
    src.write_text("#include <hip/hip_runtime.h>\n"
                   "typedef _Float16 v8h __attribute__((ext_vector_type(8)));\n"
                   "typedef _Float16 v16h __attribute__((ext_vector_type(16)));\n"
                   "typedef float v16f __attribute__((ext_vector_type(16)));\n"
                   "typedef int v8i __attribute__((ext_vector_type(8)));\n"
                   "__global__ void k(v16f *o, v8h a, v16h b, v8i x, v8i y, int i) {\n"
                   f"  {body}\n"
                   "}\n")
    return subprocess.run([HIPCC, "--offload-arch=gfx950", "--cuda-device-only", "-c", "-o", os.devnull,
                           str(src)], capture_output=True, text=True)


@needs_hipcc
def test_clang_builtins(tmp_path):
    # the fp16 SMFMAC builtin exists for gfx950 ...
    ok = _compile_device("*o = __builtin_amdgcn_smfmac_f32_32x32x32_f16(a, b, *o, i, 0, 0);", tmp_path)
    assert ok.returncode == 0, ok.stderr
    # ... the scaled FP4 MFMA builtin too ...
    ok = _compile_device("*o = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(x, y, *o, 4, 4, 0, i, 0, i);",
                         tmp_path)
    assert ok.returncode == 0, ok.stderr
    # ... and no sparse builtin takes f8f6f4 operands
    bad = _compile_device("*o = __builtin_amdgcn_smfmac_f32_32x32x64_f8f6f4(x, y, *o, i, 0, 0);", tmp_path)
    assert bad.returncode != 0
