"""Host-side checks of the build script: the compiler resource report parser
that makes a build fail when a kernel would use scratch memory."""
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
