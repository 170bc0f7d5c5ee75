"""The build's kernel resource check (CPU only): the compiler's resource remarks are parsed per kernel, and a
kernel that spills to scratch, exceeds the register file or asks for more LDS than a CU has fails the build."""
import pytest

from gemm_epilogue_fusion_amd import build as B

REMARKS = """\
k.hip:105:1: remark: Function Name: _ZN4coda20gemm_epilogue_kernelILi3ELb0EE [-Rpass-analysis=kernel-resource-usage]
k.hip:105:1: remark:     VGPRs: 234 [-Rpass-analysis=kernel-resource-usage]
k.hip:105:1: remark:     ScratchSize [bytes/lane]: 0 [-Rpass-analysis=kernel-resource-usage]
k.hip:105:1: remark:     Occupancy [waves/SIMD]: 2 [-Rpass-analysis=kernel-resource-usage]
k.hip:105:1: remark:     LDS Size [bytes/block]: 131072 [-Rpass-analysis=kernel-resource-usage]
  105 | __global__ void k() {
      | ^
k.hip:279:1: remark: Function Name: _ZN4coda18prms_reduce_kernelEPKfiiffPf [-Rpass-analysis=kernel-resource-usage]
k.hip:279:1: remark:     VGPRs: 8 [-Rpass-analysis=kernel-resource-usage]
k.hip:279:1: remark:     ScratchSize [bytes/lane]: 0 [-Rpass-analysis=kernel-resource-usage]
k.hip:279:1: remark:     LDS Size [bytes/block]: 0 [-Rpass-analysis=kernel-resource-usage]
"""


def test_parse_remarks():
    u = B.resource_usage(REMARKS)
    assert set(u) == {"_ZN4coda20gemm_epilogue_kernelILi3ELb0EE", "_ZN4coda18prms_reduce_kernelEPKfiiffPf"}
    g = u["_ZN4coda20gemm_epilogue_kernelILi3ELb0EE"]
    assert g["VGPRs"] == "234" and g["ScratchSize"] == "0" and g["LDS"] == "131072" and g["Occupancy"] == "2"
    B.check_usage(u)


@pytest.mark.parametrize("field,value,what", [("ScratchSize", "452", "scratch"), ("VGPRs", "300", "VGPRs"),
                                              ("LDS", str(192 * 1024), "LDS")])
def test_check_rejects(field, value, what):
    u = B.resource_usage(REMARKS)
    u["_ZN4coda20gemm_epilogue_kernelILi3ELb0EE"][field] = value
    with pytest.raises(RuntimeError, match=what):
        B.check_usage(u)
