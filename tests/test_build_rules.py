"""Host-side checks of the build rules (no GPU, no compile): the
resource-usage remarks parser that makes build() refuse decode kernels with
register spills."""
from compressed_cache_decode_jolt_amd.build import scratch_users

REMARKS = """\
x.inc:225:1: remark: Function Name: _ZN9jolt_mfma11decode_mfmaILi4E [-Rpass-analysis=kernel-resource-usage]
x.inc:225:1: remark:     VGPRs: 256 [-Rpass-analysis=kernel-resource-usage]
x.inc:225:1: remark:     ScratchSize [bytes/lane]: 36 [-Rpass-analysis=kernel-resource-usage]
x.inc:225:1: remark: Function Name: _ZN9jolt_mfma11decode_mfmaILi8E [-Rpass-analysis=kernel-resource-usage]
x.inc:225:1: remark:     ScratchSize [bytes/lane]: 0 [-Rpass-analysis=kernel-resource-usage]
"""


def test_scratch_users_finds_spilling_kernels_only():
    assert scratch_users(REMARKS) == {"_ZN9jolt_mfma11decode_mfmaILi4E": 36}
    assert scratch_users("") == {}
