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


def _instructions(asm_text):
    """Per kernel, its instruction lines (labels, directives, comments dropped)."""
    import re
    out, cur = {}, None
    for line in asm_text.splitlines():
        m = re.match(r"^(_Z\w+):", line)
        if m:
            cur = m.group(1)
            out[cur] = []
            continue
        if cur is None:
            continue
        if line.startswith(".Lfunc_end"):
            cur = None
            continue
        t = line.split(";", 1)[0].strip()
        if t and not t.startswith(".") and not t.endswith(":"):
            out[cur].append(t)
    return out


def _sgprs(operand):
    import re
    m = re.fullmatch(r"s(\d+)", operand) or re.fullmatch(r"s\[(\d+):(\d+)\]", operand)
    if not m:
        return set()
    lo, hi = int(m.group(1)), int(m.groups()[-1])
    return set(range(lo, hi + 1))


def test_direct_lds_loads_have_their_wait_states():
    """Every inline-asm global->LDS load (buffer_load ... lds) is preceded by
    the s_nop its asm carries (one wait state after the compiler's scalar
    write of M0), and no vector instruction writes one of its descriptor's
    scalar registers within the five instructions before it (a VALU write of
    an SGPR that a vector-memory instruction reads needs five wait states,
    which the compiler does not insert for asm it cannot see into)."""
    if not os.path.exists(attn_build.ASM_PATH):
        pytest.skip("libattn.so has not been built here (no device assembly)")
    with open(attn_build.ASM_PATH) as f:
        kernels = _instructions(f.read())
    n_loads, bad = 0, []
    for name, ins in kernels.items():
        for i, t in enumerate(ins):
            op = t.split()[0]
            if not (op.startswith("buffer_load") and t.endswith(" lds")):
                continue
            n_loads += 1
            if i == 0 or ins[i - 1] != "s_nop 0":
                bad.append((name, i, "no s_nop before", ins[i - 1] if i else ""))
            srd = _sgprs(t.split()[2].rstrip(","))
            states = 0
            for k in range(i - 1, -1, -1):
                prev = ins[k]
                pop = prev.split()
                if pop[0].startswith("v_") and len(pop) > 1 and _sgprs(pop[1].rstrip(",")) & srd:
                    bad.append((name, i, "VALU write of the descriptor", prev, states))
                    break
                states += int(pop[1]) + 1 if pop[0] == "s_nop" else 1
                if states >= 5:
                    break
    assert n_loads > 0, "no direct LDS loads found in the assembly"
    assert not bad, bad[:10]
