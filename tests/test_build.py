"""Host checks of the build script (no GPU): the scratch-use guard on the kernels that
count their own global->LDS transfers."""
from int4_quantized_kv_amd import build


def test_scratch_guard_reads_the_resource_remarks():
    text = "\n".join([
        "decode_mfma.hip:1:1: remark: Function Name: kern_a [-Rpass-analysis=kernel-resource-usage]",
        "decode_mfma.hip:1:1: remark:     VGPRs: 142 [-Rpass-analysis=kernel-resource-usage]",
        "decode_mfma.hip:1:1: remark:     ScratchSize [bytes/lane]: 0 [-Rpass-analysis=kernel-resource-usage]",
        "decode_mfma.hip:2:1: remark: Function Name: kern_b [-Rpass-analysis=kernel-resource-usage]",
        "decode_mfma.hip:2:1: remark:     ScratchSize [bytes/lane]: 24 [-Rpass-analysis=kernel-resource-usage]",
    ])
    assert build._scratch_users(text) == ["kern_b (24 bytes/lane)"]
    assert build._scratch_users("") == []


def test_guarded_sources_are_compiled_with_the_remarks():
    assert "decode_mfma.hip" in build.NO_SCRATCH
    assert all(src in build.SOURCES for src in build.NO_SCRATCH)
    assert build.RESOURCE_REMARKS == ["-Rpass-analysis=kernel-resource-usage"]
