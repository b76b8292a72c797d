"""Host-side build checks (no GPU): the scratch-spill detector reads the
compiler's resource-usage remarks."""

from blockwise_bit_codebook_amd import build


def test_scratch_detector_flags_spilling_kernels():
    lines = [
        "q.hip:10:1: remark: Function Name: kern_a [-Rpass-analysis=kernel-resource-usage]",
        "q.hip:10:1: remark:     VGPRs: 64 [-Rpass-analysis=kernel-resource-usage]",
        "q.hip:10:1: remark:     ScratchSize [bytes/lane]: 0 [-Rpass-analysis=kernel-resource-usage]",
        "q.hip:20:1: remark: Function Name: kern_b [-Rpass-analysis=kernel-resource-usage]",
        "q.hip:20:1: remark:     ScratchSize [bytes/lane]: 80 [-Rpass-analysis=kernel-resource-usage]",
    ]
    assert build._scratch_kernels(lines) == [("kern_b", 80)]


def test_scratch_detector_passes_clean_output():
    lines = ["x.hip:1:1: remark: Function Name: k [-Rpass-analysis=kernel-resource-usage]",
             "x.hip:1:1: remark:     ScratchSize [bytes/lane]: 0 [-Rpass-analysis=kernel-resource-usage]"]
    assert build._scratch_kernels(lines) == []
