"""Compile the gfx950 HIP library libattn.so in-tree.

``python -m flashattention_backward_pass_attn_amd.build`` (or ``build()``)
runs hipcc on csrc/attn_api.hip, which includes every kernel, and writes
``flashattention_backward_pass_attn_amd/libattn.so``.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
LIB_PATH = os.path.join(PKG_DIR, "libattn.so")
# per-kernel register, scratch and LDS use reported by the compiler for the
# last build (tests/test_build_resources.py checks that no kernel spills)
RESOURCES_PATH = os.path.join(PKG_DIR, "libattn_resources.txt")
# gfx950 assembly of the same build (tests/test_build_resources.py checks the
# wait states before every inline-asm direct global->LDS load)
ASM_PATH = os.path.join(PKG_DIR, "libattn_device.s")
SOURCES = [os.path.join(CSRC, "attn_api.hip")]
HEADERS = [os.path.join(CSRC, f) for f in ("attn_device.h", "attn_fwd.h", "attn_bwd.h", "attn_bwd_split.h",
                                              "attn_bwd_dq.h")] + [os.path.join(ROOT, "include", "attn.h")]

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # no packed-fp32 VALU instructions in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-result",
]


def hipcc_path() -> str:
    p = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(p):
        raise RuntimeError("hipcc not found: the HIP toolchain is required to build libattn.so")
    return p


def build(verbose: bool = False, extra_flags=None, out_path: str = LIB_PATH) -> str:
    """Compile libattn.so (always recompiles).  Returns the library path."""
    tmp = out_path + ".tmp"
    cmd = [hipcc_path(), *HIPCC_FLAGS, *(extra_flags or []), "-Rpass-analysis=kernel-resource-usage",
           "-I", os.path.join(ROOT, "include"), *SOURCES, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    # the device assembly of the same sources and flags, compiled alongside
    asm_proc = None
    if out_path == LIB_PATH:
        asm = [hipcc_path(), *[f for f in HIPCC_FLAGS if f not in ("-fPIC", "-shared")], *(extra_flags or []),
               "--cuda-device-only", "-S", "-I", os.path.join(ROOT, "include"), *SOURCES, "-o", ASM_PATH]
        asm_proc = subprocess.Popen(asm, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    asm_out = asm_proc.communicate() if asm_proc is not None else ("", "")
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed building libattn.so")
    if asm_proc is not None and asm_proc.returncode != 0:
        sys.stderr.write(asm_out[0] + asm_out[1])
        raise RuntimeError("hipcc failed writing the device assembly")
    remarks = [ln.split("remark:", 1)[1].split("[-Rpass-analysis")[0].rstrip()
               for ln in res.stderr.splitlines() if "remark:" in ln and "kernel-resource-usage" in ln]
    other = [ln for ln in res.stderr.splitlines() if "kernel-resource-usage" not in ln]
    if verbose and any(ln.strip() for ln in other):
        sys.stderr.write("\n".join(other) + "\n")
    os.replace(tmp, out_path)
    if out_path == LIB_PATH:
        with open(RESOURCES_PATH, "w") as f:
            f.write("\n".join(remarks) + "\n")
    return out_path


if __name__ == "__main__":
    print(build(verbose=True))
