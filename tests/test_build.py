"""Host-side checks of the build script (no GPU): a kernel that spills to scratch fails the
build, since hand-counted vmcnt waits in the attention kernels assume no other memory
operations in their loops."""

import pytest

from deterministic_paged_kv_amd import build

REMARKS = """a.hip:3:1: remark: Function Name: kern_a [-Rpass-analysis=kernel-resource-usage]
a.hip:3:1: remark:     VGPRs: 100 [-Rpass-analysis=kernel-resource-usage]
a.hip:3:1: remark:     ScratchSize [bytes/lane]: 0 [-Rpass-analysis=kernel-resource-usage]
a.hip:9:1: remark: Function Name: kern_b [-Rpass-analysis=kernel-resource-usage]
a.hip:9:1: remark:     ScratchSize [bytes/lane]: {b} [-Rpass-analysis=kernel-resource-usage]
"""


def test_no_scratch_accepts_clean_kernels():
    build.check_no_scratch("a.hip", REMARKS.format(b=0))


def test_no_scratch_names_the_spilling_kernel():
    with pytest.raises(RuntimeError, match="kern_b uses 24 bytes"):
        build.check_no_scratch("a.hip", REMARKS.format(b=24))
