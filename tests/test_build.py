"""Host-side checks of the build script: the compiler resource report parser
that makes a build fail when a kernel would use scratch memory, and the
assembly check that no kernel loads through a loop over lane values."""
import os
import shutil

import pytest

from dense_gemm_fp8_amd import build

REPORT = """\
k.hip:9:1: remark: Function Name: _Zok [-Rpass-analysis=kernel-resource-usage]
k.hip:9:1: remark:     VGPRs: 256 [-Rpass-analysis=kernel-resource-usage]
k.hip:9:1: remark:     ScratchSize [bytes/lane]: 0 [-Rpass-analysis=kernel-resource-usage]
k.hip:9:1: remark:     VGPRs Spill: 0 [-Rpass-analysis=kernel-resource-usage]
k.hip:9:1: remark: Function Name: _Zbad [-Rpass-analysis=kernel-resource-usage]
k.hip:9:1: remark:     ScratchSize [bytes/lane]: 1552 [-Rpass-analysis=kernel-resource-usage]
k.hip:9:1: remark:     VGPRs Spill: 3 [-Rpass-analysis=kernel-resource-usage]
k.hip:9:1: remark:     SGPRs Spill: 0 [-Rpass-analysis=kernel-resource-usage]
"""


def test_scratch_users_flags_only_offending_kernels():
    assert build.scratch_users(REPORT) == [("_Zbad", "ScratchSize [bytes/lane]", 1552),
                                           ("_Zbad", "VGPRs Spill", 3)]


def test_scratch_users_empty_report():
    assert build.scratch_users("") == []


def test_build_requests_the_resource_report():
    assert build.RESOURCE_REMARKS == "-Rpass-analysis=kernel-resource-usage"


ASM = """\
_Zgood:
.LBB0_1:
\tbuffer_load_dwordx4 v1, s[0:3], s4 offen lds
\ts_cbranch_scc1 .LBB0_1
.LBB0_2:
\tv_add_u32_e32 v2, 1, v2
\ts_cbranch_execnz .LBB0_2
_Zbad:
.LBB1_3:
\tv_readfirstlane_b32 s8, v2
\tv_cmp_eq_u32_e32 vcc, s8, v2
\ts_and_saveexec_b64 vcc, vcc
\tbuffer_load_dwordx4 v1, s[0:3], s8 offen lds
\ts_xor_b64 exec, exec, vcc
\ts_cbranch_execnz .LBB1_3
\ts_cbranch_execnz .LBB1_9
"""


def test_waterfall_loops_flags_only_loads_in_exec_loops():
    # _Zgood: a load in a uniform loop and an exec loop without a load;
    # _Zbad: a load in a loop over lane values (and a forward exec branch)
    assert build.waterfall_loops(ASM) == [("_Zbad", ".LBB1_3")]
    assert build.waterfall_loops("") == []


@pytest.mark.skipif(not shutil.which(build.hipcc()), reason="hipcc not available")
def test_kernels_issue_no_load_in_a_loop_over_lane_values(tmp_path):
    """Every buffer load of every kernel takes its scalar operands from scalar
    registers as compiled (13 s of hipcc on the CPU)."""
    out = os.path.join(tmp_path, "gemm_kernels.s")
    build.device_asm(out)
    asm = open(out).read()
    assert "gemm4_kernel" in asm and "gemm_kernel" in asm
    assert build.waterfall_loops(asm) == []
