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
    """The workspace is the two fp32 row statistics only: 2 * 4 bytes per
    (query head, query row), each rounded up to 256 bytes, whatever the key
    length, head dim, mask or deterministic flag."""
    p = _params()
    n = ctypes.c_size_t(0)
    assert clib.attn_bwd_workspace_size(ctypes.byref(p), ctypes.byref(n)) == fa.ATTN_OK
    stat = 2 * 8 * 128 * 4  # fp32 [B, H, Sq]
    assert n.value == 2 * ((stat + 255) // 256 * 256)
    # below it nothing is launched
    assert _bwd(clib, p, ws_bytes=n.value - 1) == fa.ATTN_ERR_WORKSPACE_TOO_SMALL
    for kw in (dict(deterministic=1), dict(causal=0), dict(seqlen_k=5000), dict(head_dim=256),
               dict(window_left=10, window_right=3)):
        q = _params(**kw)
        m = ctypes.c_size_t(0)
        assert clib.attn_bwd_workspace_size(ctypes.byref(q), ctypes.byref(m)) == fa.ATTN_OK
        assert m.value == n.value, kw
    # unaligned workspace
    assert clib.attn_bwd(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE + 16,
                         n.value, None, None) == fa.ATTN_ERR_INVALID_ARGUMENT


def test_workspace_is_linear_in_the_query_length(clib):
    """O(S) memory at long sequences: B1 H32 S32768 d128 needs 2 * 4 * 32 * 32768
    bytes (8 MiB), and S65536 twice that -- nothing quadratic."""
    for s_len in (32768, 65536):
        p = _params(batch=1, seqlen_q=s_len, seqlen_k=s_len, heads_q=32, heads_kv=32, head_dim=128)
        for t in ("q", "o", "dout", "dq", "k", "v", "dk", "dv"):
            setattr(p, t, fa.attn_strides(s_len * 32 * 128, 32 * 128, 128))
        n = ctypes.c_size_t(0)
        assert clib.attn_bwd_workspace_size(ctypes.byref(p), ctypes.byref(n)) == fa.ATTN_OK
        assert n.value == 2 * 4 * 32 * s_len


def test_varlen_workspace_follows_total_q(clib):
    p = _params(cu_seqlens_q=FAKE, cu_seqlens_k=FAKE, total_q=1000, total_k=1234)
    for t in ("q", "o", "dout", "dq"):
        setattr(p, t, fa.attn_strides(0, 8 * 64, 64))
    for t in ("k", "v", "dk", "dv"):
        setattr(p, t, fa.attn_strides(0, 2 * 64, 64))
    n = ctypes.c_size_t(0)
    assert clib.attn_bwd_workspace_size(ctypes.byref(p), ctypes.byref(n)) == fa.ATTN_OK
    stat = 8 * 1000 * 4  # fp32 [H, total_q]
    assert n.value == 2 * ((stat + 255) // 256 * 256)


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


def _noalloc(clib, p, ptr=FAKE):
    return clib.attn_bwd_noalloc(ctypes.byref(p), ptr, ptr, ptr, ptr, ptr, ptr, ptr, ptr, ptr, None, None)


def test_noalloc_validates_before_anything_else(clib):
    """attn_bwd_noalloc checks its arguments like attn_bwd, and refuses a
    problem whose statistics exceed the static array, before any HIP call."""
    assert _noalloc(clib, _params(batch=0)) == fa.ATTN_ERR_INVALID_ARGUMENT
    assert _noalloc(clib, _params(head_dim=60)) == fa.ATTN_ERR_INVALID_ARGUMENT
    rows = fa.NOALLOC_SCRATCH_BYTES // 8 // 8 + 64  # per head, 8 query heads
    p = _params(batch=1, seqlen_q=rows, seqlen_k=rows)
    for t in ("q", "o", "dout", "dq"):
        setattr(p, t, fa.attn_strides(rows * 8 * 64, 8 * 64, 64))
    for t in ("k", "v", "dk", "dv"):
        setattr(p, t, fa.attn_strides(rows * 2 * 64, 2 * 64, 64))
    n = ctypes.c_size_t(0)
    assert clib.attn_bwd_workspace_size(ctypes.byref(p), ctypes.byref(n)) == fa.ATTN_OK
    assert n.value > fa.NOALLOC_SCRATCH_BYTES
    assert _noalloc(clib, p) == fa.ATTN_ERR_WORKSPACE_TOO_SMALL


def test_noalloc_scratch_size_matches_header():
    src = open(os.path.join(ROOT, "include", "attn.h")).read()
    m = re.search(r"#define ATTN_NOALLOC_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", src)
    assert m and int(m.group(1)) << int(m.group(2)) == fa.NOALLOC_SCRATCH_BYTES
