"""The build's packed-FP32 guard, checked on the built library (no GPU needed): the gfx950
code objects inside libpkv.so hold no packed-FP32 VALU instruction (v_pk_add_f32,
v_pk_mul_f32, v_pk_fma_f32). The build passes -packed-fp32-ops to the device compiler;
without it, hipcc -O3 turns two-lane float code into such instructions."""
import glob
import os
import shutil
import subprocess
import tempfile

import pytest

import paged_kv_gqa_table_amd as pkv

OBJDUMP = "/opt/rocm/llvm/bin/llvm-objdump"
PACKED_F32 = ("v_pk_add_f32", "v_pk_mul_f32", "v_pk_fma_f32")


def test_no_packed_fp32_in_device_code():
    lib = pkv.library_path()
    if not os.path.exists(lib) or not os.path.exists(OBJDUMP):
        pytest.skip("libpkv.so not built or llvm-objdump missing")
    with tempfile.TemporaryDirectory() as d:
        shutil.copy(lib, d)
        subprocess.run([OBJDUMP, "--offloading", os.path.basename(lib)], cwd=d, check=True, capture_output=True)
        objs = sorted(glob.glob(os.path.join(d, "*amdgcn-amd-amdhsa--gfx950")))
        assert objs, "no gfx950 code object in the library"
        found, kinds = [], set()
        for o in objs:  # (a translation unit without kernels has an empty code object)
            text = subprocess.run([OBJDUMP, "-d", "--mcpu=gfx950", o], check=True, capture_output=True,
                                  text=True).stdout
            kinds |= {k for k in ("v_mfma", "v_dot2", "v_exp_f32") if k in text}
            found += [(os.path.basename(o), ins) for ins in PACKED_F32 if ins in text]
        assert kinds == {"v_mfma", "v_dot2", "v_exp_f32"}, "the disassembly misses the kernels"
        assert not found, f"packed-FP32 instructions in the device code: {found}"
