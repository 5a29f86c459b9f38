"""The build refuses a bwd_kv kernel that uses scratch memory: its tile
barrier keeps exactly the wave's own LDS DMA of the iteration in flight
(s_waitcnt vmcnt(n)), which a register spill to scratch inside the loop
would break.  The check reads the compiler's resource-usage remarks."""

import pytest

from block_sparse_long_03_amd import build as b

REPORT = """\
attn_bwd.hip:266:1: remark: Function Name: _ZN4moba18bwd_kv_pair_kernelILi128EEEvNS_7BwdArgsE [-Rpass-analysis=kernel-resource-usage]
attn_bwd.hip:266:1: remark:     VGPRs: 115 [-Rpass-analysis=kernel-resource-usage]
attn_bwd.hip:266:1: remark:     ScratchSize [bytes/lane]: {n} [-Rpass-analysis=kernel-resource-usage]
attn_bwd.hip:600:1: remark: Function Name: _ZN4moba12bwd_q_kernelILi128ELi0EEEvNS_7BwdArgsE [-Rpass-analysis=kernel-resource-usage]
attn_bwd.hip:600:1: remark:     ScratchSize [bytes/lane]: {m} [-Rpass-analysis=kernel-resource-usage]
"""


def test_no_scratch_passes():
    b._check_scratch("attn_bwd.hip", REPORT.format(n=0, m=0))


def test_scratch_in_guarded_kernel_fails():
    with pytest.raises(RuntimeError, match="bwd_kv_pair_kernel"):
        b._check_scratch("attn_bwd.hip", REPORT.format(n=16, m=0))


def test_scratch_elsewhere_is_not_guarded():
    b._check_scratch("attn_bwd.hip", REPORT.format(n=0, m=12))
