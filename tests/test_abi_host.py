"""Host-side checks of the C ABI that need no GPU: the library loads, exports
every symbol the header declares, and rejects invalid arguments before
launching anything (flash-attention CK mha_bwd.cpp, mha_bwd: the TORCH_CHECKs
on dtype, contiguity, batch, head_dim and the head ratio)."""
import ctypes
import os
import re

import pytest

import flashattention_backward_pass_attn_amd as fa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def clib():
    if not os.path.exists(fa.LIB_PATH):
        pytest.fail("libattn.so is not built (run __graft_entry__.build())")
    return fa.load_library()


def _declared_functions():
    src = open(os.path.join(ROOT, "include", "attn.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(attn_\w+)\s*\(", src, flags=re.M)))


def test_header_declares_the_entry_points():
    assert _declared_functions() == sorted(fa.EXPORTED_SYMBOLS)


def test_library_exports_every_declared_symbol(clib):
    for name in _declared_functions():
        assert hasattr(clib, name), name
    assert "gfx950" in fa.version()


def test_exported_symbols_have_c_linkage():
    out = os.popen(f"nm -D --defined-only {fa.LIB_PATH}").read()
    for name in fa.EXPORTED_SYMBOLS:
        assert re.search(rf"\bT {name}$", out, flags=re.M), name


def test_status_strings(clib):
    for s in range(5):
        assert len(fa.status_string(s)) > 0
    assert fa.status_string(3) == "workspace too small"


def _params(**kw):
    p = fa.attn_params()
    p.dtype = fa.ATTN_FP16
    p.batch, p.seqlen_q, p.seqlen_k = 2, 128, 128
    p.heads_q, p.heads_kv, p.head_dim = 8, 2, 64
    p.softmax_scale = 0.125
    p.causal, p.deterministic = 1, 0
    p.window_left, p.window_right = -1, -1
    for t in ("q", "o", "dout", "dq"):
        setattr(p, t, fa.attn_strides(128 * 8 * 64, 8 * 64, 64))
    for t in ("k", "v", "dk", "dv"):
        setattr(p, t, fa.attn_strides(128 * 2 * 64, 2 * 64, 64))
    for k, v in kw.items():
        setattr(p, k, v)
    return p


FAKE = 1 << 20  # non-null, 256-byte aligned; validation rejects before any use


def _bwd(clib, p, ws_bytes=1 << 30, ptr=FAKE):
    return clib.attn_bwd(ctypes.byref(p), ptr, ptr, ptr, ptr, ptr, ptr, ptr, ptr, ptr, FAKE, ws_bytes, None, None)


def _fwd(clib, p, ptr=FAKE):
    return clib.attn_fwd(ctypes.byref(p), ptr, ptr, ptr, ptr, ptr, None)


@pytest.mark.parametrize("field,value,expect", [
    ("dtype", 7, fa.ATTN_ERR_INVALID_ARGUMENT),
    ("batch", 0, fa.ATTN_ERR_INVALID_ARGUMENT),
    ("head_dim", 60, fa.ATTN_ERR_INVALID_ARGUMENT),       # not a multiple of 8
    ("head_dim", 264, fa.ATTN_ERR_INVALID_ARGUMENT),      # above 256
    ("heads_kv", 3, fa.ATTN_ERR_INVALID_ARGUMENT),        # 8 % 3 != 0
    ("seqlen_q", -1, fa.ATTN_ERR_INVALID_ARGUMENT),
    ("causal", 2, fa.ATTN_ERR_INVALID_ARGUMENT),
    ("softmax_scale", float("nan"), fa.ATTN_ERR_INVALID_ARGUMENT),
    ("softmax_scale", -0.5, fa.ATTN_ERR_INVALID_ARGUMENT),
    ("softmax_scale", 0.0, fa.ATTN_ERR_INVALID_ARGUMENT),
    ("window_left", -2, fa.ATTN_ERR_INVALID_ARGUMENT),
    ("window_right", -5, fa.ATTN_ERR_INVALID_ARGUMENT),
])
def test_invalid_parameters_rejected(clib, field, value, expect):
    p = _params(**{field: value})
    assert _bwd(clib, p) == expect
    assert _fwd(clib, p) == expect
    n = ctypes.c_size_t(0)
    assert clib.attn_bwd_workspace_size(ctypes.byref(p), ctypes.byref(n)) == expect


def test_null_pointers_rejected(clib):
    assert _bwd(clib, _params(), ptr=None) == fa.ATTN_ERR_INVALID_ARGUMENT
    assert _fwd(clib, _params(), ptr=None) == fa.ATTN_ERR_INVALID_ARGUMENT
    assert clib.attn_fwd(None, FAKE, FAKE, FAKE, FAKE, FAKE, None) == fa.ATTN_ERR_INVALID_ARGUMENT


def test_misaligned_strides_unsupported(clib):
    p = _params()
    p.q = fa.attn_strides(128 * 8 * 64, 8 * 64 + 4, 64)
    assert _bwd(clib, p) == fa.ATTN_ERR_UNSUPPORTED
    assert _fwd(clib, p) == fa.ATTN_ERR_UNSUPPORTED
    assert _bwd(clib, _params(), ptr=FAKE + 2) == fa.ATTN_ERR_UNSUPPORTED


def test_half_varlen_rejected(clib):
    p = _params()
    p.cu_seqlens_q = FAKE
    assert _bwd(clib, p) == fa.ATTN_ERR_INVALID_ARGUMENT


def test_workspace_size_and_too_small(clib):
    p = _params()
    n = ctypes.c_size_t(0)
    nmin = ctypes.c_size_t(0)
    assert clib.attn_bwd_workspace_size(ctypes.byref(p), ctypes.byref(n)) == fa.ATTN_OK
    assert clib.attn_bwd_workspace_size_min(ctypes.byref(p), ctypes.byref(nmin)) == fa.ATTN_OK
    stat = 2 * 8 * 128  # Delta: fp32 [B, H, Sq]
    assert nmin.value >= stat * 4 and nmin.value % 256 == 0
    # the full workspace adds the dS tiles: at least Hq * Sq * Sk bf16/fp16 values per sequence
    assert n.value >= nmin.value + 2 * 8 * 128 * 128 * 2 and n.value % 256 == 0
    # below the minimum nothing is launched
    assert _bwd(clib, p, ws_bytes=nmin.value - 1) == fa.ATTN_ERR_WORKSPACE_TOO_SMALL
    # neither size depends on the deterministic flag (no dQ accumulator)
    pd = _params(deterministic=1)
    nd = ctypes.c_size_t(0)
    assert clib.attn_bwd_workspace_size(ctypes.byref(pd), ctypes.byref(nd)) == fa.ATTN_OK
    assert nd.value == n.value
    # unaligned workspace
    assert clib.attn_bwd(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE + 16,
                         n.value, None, None) == fa.ATTN_ERR_INVALID_ARGUMENT


def test_bad_phase_mask_rejected(clib):
    p = _params()
    for bad in (0, 8, 15):
        assert clib.attn_bwd_phases(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                    1 << 30, None, None, bad) == fa.ATTN_ERR_INVALID_ARGUMENT


def test_binding_refuses_cpu_tensors():
    torch = pytest.importorskip("torch")
    q = torch.zeros(1, 8, 2, 64, dtype=torch.float16)
    with pytest.raises(ValueError):
        fa.attn_fwd(q, q, q)


def test_wide_head_dim_needs_the_full_workspace(clib):
    """Head dims above 128 (the 256-wide tile) have only the stored-dS path: the
    minimum workspace is the full one, and a Delta-only workspace is refused
    before anything is launched."""
    for d in (136, 192, 256):
        p = _params(head_dim=d)
        n = ctypes.c_size_t(0)
        nmin = ctypes.c_size_t(0)
        assert clib.attn_bwd_workspace_size(ctypes.byref(p), ctypes.byref(n)) == fa.ATTN_OK
        assert clib.attn_bwd_workspace_size_min(ctypes.byref(p), ctypes.byref(nmin)) == fa.ATTN_OK
        assert nmin.value == n.value
        assert _bwd(clib, p, ws_bytes=n.value - 256) == fa.ATTN_ERR_WORKSPACE_TOO_SMALL
