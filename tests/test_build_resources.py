"""The built kernels keep every value in registers.

The build records the compiler's per-kernel resource report
(flashattention_backward_pass_attn_amd/libattn_resources.txt); a kernel that
spills vector registers to scratch memory pays memory latency inside its
loops, so the report must show no scratch and no vector-register spills for
any kernel.  Runs on the CPU from the last build's report.
"""
import os

import pytest

from flashattention_backward_pass_attn_amd import build as attn_build


def _kernels():
    if not os.path.exists(attn_build.RESOURCES_PATH):
        pytest.skip("libattn.so has not been built here (no resource report)")
    kernels, cur = {}, None
    with open(attn_build.RESOURCES_PATH) as f:
        for line in f:
            line = line.strip()
            if line.startswith("Function Name:"):
                cur = line.split(":", 1)[1].strip()
                kernels[cur] = {}
            elif cur and ":" in line:
                k, v = line.split(":", 1)
                kernels[cur][k.strip()] = v.strip()
    return kernels


def test_report_covers_every_kernel_family():
    names = " ".join(_kernels())
    for fam in ("attn_fwd_kernel", "attn_bwd_pre_kernel", "attn_bwd_dkdv_kernel", "attn_bwd_dq_recompute_kernel",
                "attn_bwd_dq_wide_kernel"):
        assert fam in names, fam


def test_no_kernel_spills():
    bad = {name: (r.get("ScratchSize [bytes/lane]"), r.get("VGPRs Spill"))
           for name, r in _kernels().items()
           if r.get("ScratchSize [bytes/lane]") != "0" or r.get("VGPRs Spill") != "0"}
    assert not bad, bad
