"""The build rejects product kernels that use scratch memory (CPU only)."""
from quantized_gemm_rtn_amd.build import scratch_users


def test_scratch_guard_reads_resource_remarks():
    remarks = "\n".join([
        "gemv.hip:1:1: remark: Function Name: _Z7kernelAv [-Rpass-analysis=kernel-resource-usage]",
        "gemv.hip:1:1: remark:     VGPRs: 96 [-Rpass-analysis=kernel-resource-usage]",
        "gemv.hip:1:1: remark:     ScratchSize [bytes/lane]: 0 [-Rpass-analysis=kernel-resource-usage]",
        "gemv.hip:9:1: remark: Function Name: _Z7kernelBv [-Rpass-analysis=kernel-resource-usage]",
        "gemv.hip:9:1: remark:     ScratchSize [bytes/lane]: 48 [-Rpass-analysis=kernel-resource-usage]",
    ])
    assert scratch_users(remarks) == {"_Z7kernelBv": 48}
    assert scratch_users("") == {}
