"""The gfx950 assembly of every kernel, checked on the CPU (hipcc compiles it without a
GPU): no packed FP32 arithmetic, no scratch memory or register spills, FP32 and FP16/FP64
denormals preserved, and every scalar instruction from a list of ALU, branch, wait and
load families, so that scalar memory is only ever read."""
import os
import re
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

from mixed_precision_zero_amd import build  # noqa: E402

# Scalar instruction families the kernels may use: ALU, compare, select, shifts and bit
# fields, moves, exec-mask updates, branches, waits, barriers, program end, and scalar
# loads.  Anything else shows up here and has to be looked at.
SCALAR_OK = (
    "s_add", "s_addc", "s_addk", "s_sub", "s_subb", "s_mul", "s_mulk", "s_min", "s_max",
    "s_abs", "s_absdiff", "s_and", "s_andn1", "s_andn2", "s_or", "s_orn1", "s_orn2", "s_xor",
    "s_xnor", "s_nand", "s_nor", "s_not", "s_mov", "s_movk", "s_cmov", "s_cmovk", "s_cmp",
    "s_cmpk", "s_cselect", "s_lshl", "s_lshr", "s_ashr", "s_bfe", "s_bfm", "s_bitcmp",
    "s_bitset", "s_brev", "s_bcnt", "s_ff0", "s_ff1", "s_flbit", "s_sext", "s_pack",
    "s_branch", "s_cbranch", "s_waitcnt", "s_nop", "s_barrier", "s_endpgm", "s_sleep",
    "s_setprio", "s_getpc", "s_setpc", "s_swappc", "s_load_", "s_buffer_load_",
)
PACKED_FP32 = re.compile(r"^\s*v_pk_\w*_f32\b", re.M)


def _device_asm(src, tmp_path):
    out = str(tmp_path / (os.path.basename(src) + ".s"))
    flags = [f for f in build.FLAGS if f not in ("-fPIC", "-shared")]
    res = subprocess.run([build.HIPCC, *flags, "--cuda-device-only", "-S", src, "-o", out],
                         capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    with open(out) as f:
        return f.read()


@pytest.mark.parametrize("src", build.SOURCES[:1] + build.PROBE_SOURCES,
                         ids=lambda p: os.path.basename(p))
def test_kernel_assembly(src, tmp_path):
    if not os.path.exists(build.HIPCC):
        pytest.skip("hipcc not available")
    asm = _device_asm(src, tmp_path)
    kernels = re.findall(r"^\s*\.amdhsa_kernel\s+(\S+)", asm, re.M)
    assert kernels, "no kernels in the assembly"
    n = len(kernels)
    # denormals kept (3 = preserve on input and output), no scratch, no spills
    for field, want in ((r"\.amdhsa_float_denorm_mode_32", "3"),
                        (r"\.amdhsa_float_denorm_mode_16_64", "3"),
                        (r"\.amdhsa_private_segment_fixed_size", "0")):
        got = re.findall(field + r"\s+(\d+)", asm)
        assert got == [want] * n, (field, got)
    for field in ("vgpr_spill_count", "sgpr_spill_count", "private_segment_fixed_size"):
        got = re.findall(r"\." + field + r":\s+(\d+)", asm)
        assert len(got) == n and set(got) == {"0"}, (field, got)
    assert not re.search(r"^\s*scratch_", asm, re.M)
    assert not PACKED_FP32.search(asm), PACKED_FP32.search(asm).group(0)
    scalar = set(re.findall(r"^\s+(s_[a-z0-9_]+)", asm, re.M))
    odd = sorted(m for m in scalar if not m.startswith(SCALAR_OK))
    assert not odd, f"scalar instructions outside the allowed families: {odd}"
