"""The build's resource check: a kernel that spills VGPRs or uses stack stops the build."""
import pytest

from rope_context_extension_amd import build as B

REPORT_OK = """x.hip:5:1: remark: Function Name: k1 [-Rpass-analysis=kernel-resource-usage]
x.hip:5:1: remark:     VGPRs: 216 [-Rpass-analysis=kernel-resource-usage]
x.hip:5:1: remark:     ScratchSize [bytes/lane]: 0 [-Rpass-analysis=kernel-resource-usage]
x.hip:5:1: remark:     SGPRs Spill: 4 [-Rpass-analysis=kernel-resource-usage]
x.hip:5:1: remark:     VGPRs Spill: 0 [-Rpass-analysis=kernel-resource-usage]
"""


def test_clean_report_passes():
    B._check_resources("x.hip", REPORT_OK)


@pytest.mark.parametrize("line", ["ScratchSize [bytes/lane]: 704", "VGPRs Spill: 3"])
def test_stack_or_vgpr_spill_stops_the_build(line):
    bad = REPORT_OK + ("x.hip:9:1: remark: Function Name: k2 [-Rpass-analysis=kernel-resource-usage]\n"
                       f"x.hip:9:1: remark:     {line} [-Rpass-analysis=kernel-resource-usage]\n")
    with pytest.raises(RuntimeError, match="k2"):
        B._check_resources("x.hip", bad)
