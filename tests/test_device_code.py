"""Checks on the library's own gfx950 code object (CPU only: the device code
is taken out of the built libmhla.so and disassembled here).

On gfx950 a dependent MFMA of another 16x16 shape (16x16x16 reading the
accumulator that a 16x16x32 MFMA wrote just before it, or the reverse) gets
a wrong accumulator when the two issue back to back, and hipcc inserts no
wait states between them (an exact small-integer check on an MI355X: wrong
back to back, exact with 32 s_nop cycles between, exact for same-shape
chains).  The kernels therefore use one MFMA shape, v_mfma_f32_16x16x32_bf16,
for every product, with half-empty last steps where a contraction is not a
multiple of 32; this test keeps it that way.
"""
import os
import re
import shutil
import subprocess

import pytest

import token_level_head_mhla_amd as m

LLVM = "/opt/rocm/llvm/bin"


def _disassemble(tmp_path):
    tools = [os.path.join(LLVM, t) for t in ("llvm-objcopy", "clang-offload-bundler", "llvm-objdump")]
    if not all(os.path.exists(t) for t in tools) or not os.path.exists(m.library_path()):
        pytest.skip("ROCm LLVM tools or the built library are missing")
    fat, co = str(tmp_path / "fatbin.bin"), str(tmp_path / "dev.co")
    subprocess.run([tools[0], "--dump-section", ".hip_fatbin=" + fat, m.library_path()],
                   check=True, capture_output=True)
    subprocess.run([tools[1], "--unbundle", "--type=o", "--input=" + fat,
                    "--targets=hipv4-amdgcn-amd-amdhsa--gfx950", "--output=" + co],
                   check=True, capture_output=True)
    res = subprocess.run([tools[2], "-d", co], check=True, capture_output=True, text=True)
    return res.stdout


def test_one_mfma_shape_only(tmp_path):
    text = _disassemble(tmp_path)
    ops = set(re.findall(r"\bv_mfma_[a-z0-9_]+", text))
    assert ops == {"v_mfma_f32_16x16x32_bf16"}, ops
