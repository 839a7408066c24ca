"""The build's spill guard for kernels whose inline-asm LDS reads are waited on
later: its remark parser flags scratch and spills and finds the kernels."""
import pytest

from sparse_attention_04_amd.build import check_no_spills

R = "x.hip:1:1: remark: {} [-Rpass-analysis=kernel-resource-usage]"


def _remarks(name, scratch=0, vspill=0):
    return "\n".join(R.format(t) for t in [f"Function Name: {name}", "VGPRs: 256",
                                            f"ScratchSize [bytes/lane]: {scratch}", "SGPRs Spill: 0",
                                            f"VGPRs Spill: {vspill}"])


def test_clean_kernel_passes():
    assert check_no_spills(_remarks("_ZN3dsa15sfa_bf16_kernelI"), ("sfa_bf16_kernel",)) == []


@pytest.mark.parametrize("kw", [dict(scratch=16), dict(vspill=3)])
def test_spills_are_reported(kw):
    assert check_no_spills(_remarks("_ZN3dsa15sfa_bf16_kernelI", **kw), ("sfa_bf16_kernel",))


def test_other_kernels_are_ignored_but_some_must_be_seen():
    assert check_no_spills(_remarks("_ZN3dsa15sfa_bf16_kernelI") + "\n" + _remarks("other", scratch=8),
                           ("sfa_bf16_kernel",)) == []
    with pytest.raises(RuntimeError):
        check_no_spills(_remarks("other"), ("sfa_bf16_kernel",))
