"""The build rejects a private-tail ring kernel that spills: its explicit s_waitcnt
counts assume no other vector-memory operation (such as a scratch access) is issued
inside the ring. Checked on synthetic compiler resource reports (no compiler run)."""
import pytest

from prefix_shared_kv_radix_amd import build


def _report(name, scratch):
    return (f"remark: attn_gqa.hip:1:0: Function Name: {name} [-Rpass-analysis=kernel-resource-usage]\n"
            f"remark: attn_gqa.hip:1:0:     VGPRs: 250 [-Rpass-analysis=kernel-resource-usage]\n"
            f"remark: attn_gqa.hip:1:0:     ScratchSize [bytes/lane]: {scratch} "
            f"[-Rpass-analysis=kernel-resource-usage]\n")


TAIL4 = "_ZN12_GLOBAL__N_116tail_bf16_kernelILi4EEEvN12radix_launch8AttnArgsEii"
FUSED2 = "_ZN12_GLOBAL__N_119decode_fused_kernelILi2EEEvN12radix_launch8AttnArgsEiiii"
FUSED8 = "_ZN12_GLOBAL__N_119decode_fused_kernelILi8EEEvN12radix_launch8AttnArgsEiiii"
EXTEND4 = "_ZN12_GLOBAL__N_116attn_mfma_kernelILi4EEEvN12radix_launch8AttnArgsEii"


@pytest.mark.parametrize("name", [TAIL4, FUSED2])
def test_ring_kernel_with_scratch_is_rejected(name):
    with pytest.raises(RuntimeError, match="spills"):
        build._check_scratch(_report(name, 8), "attn_gqa.hip")


@pytest.mark.parametrize("name,scratch", [(TAIL4, 0), (FUSED2, 0), (FUSED8, 476), (EXTEND4, 64)])
def test_other_reports_pass(name, scratch):
    build._check_scratch(_report(name, scratch), "attn_gqa.hip")
