"""Host logic of the build: kernels whose explicit vmcnt waits count only their
own global loads must compile without scratch (a spill would add scratch
accesses to the same counter)."""
import pytest

from chunkwise_delta_rule_amd import build

REMARK = """{src}:283:1: remark: Function Name: {name} [-Rpass-analysis=kernel-resource-usage]
{src}:283:1: remark:     VGPRs: 255 [-Rpass-analysis=kernel-resource-usage]
{src}:283:1: remark:     ScratchSize [bytes/lane]: {scratch} [-Rpass-analysis=kernel-resource-usage]
"""


@pytest.mark.parametrize("src,name", [
    ("chunk_fused.hip", "_ZN3mdn22chunk_fwd_fused_kernelILi128ELi128EEEvPKDF16bS3_S3_PKfS5_S5_PS1_PfS7_iiii"),
    ("chunk_fwd.hip", "_ZN3mdn22chunk_scan_bf16_kernelILi128ELi128EEEvPKDF16b"),
])
def test_scratch_in_a_waited_kernel_fails_the_build(src, name):
    build._check_no_scratch(src, REMARK.format(src=src, name=name, scratch=0))
    with pytest.raises(RuntimeError, match="scratch"):
        build._check_no_scratch(src, REMARK.format(src=src, name=name, scratch=16))


def test_scratch_elsewhere_is_allowed():
    build._check_no_scratch("chunk_fwd.hip",
                            REMARK.format(src="chunk_fwd.hip", name="_ZN3mdn17chunk_prep_kernel",
                                          scratch=64))
    build._check_no_scratch("decode.hip",
                            REMARK.format(src="decode.hip", name="_ZN3mdn18decode_step_kernel",
                                          scratch=64))
