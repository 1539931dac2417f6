"""The no-allocation backward entry point (attn_bwd_noalloc) against attn_bwd.

Both run the same kernels; attn_bwd_noalloc only takes its statistics
workspace from the library's static device array instead of the caller's
buffer.  Two calls in a row, the second on a smaller problem (so the array
holds the first call's statistics when the second starts), must each give
dQ, dK, dV and Delta bit-identical to attn_bwd on the same inputs, and
within the oracle's tolerance.
"""
import pytest

from helpers import TOL, assert_close, make_case, oracle_run, to_f64, upload

pytestmark = pytest.mark.gpu


def _run_both(lib, inp, causal):
    import torch
    dt = inp["dtype"]
    q, k, v, do = (upload(inp[n + "_bits"], dt) for n in ("q", "k", "v", "do"))
    o, lse = lib.attn_fwd(q, k, v, causal=causal)
    ref = lib.attn_bwd(q, k, v, o, lse, do, causal=causal, return_delta=True)
    got = lib.attn_bwd_noalloc(q, k, v, o, lse, do, causal=causal, return_delta=True)
    torch.cuda.synchronize()
    return ref, got


@pytest.mark.parametrize("first,second", [
    (("bf16", 2, 8, 2, 1000, 1000, 128, True), ("bf16", 1, 4, 4, 300, 300, 128, True)),
    (("fp16", 1, 4, 2, 777, 777, 64, False), ("fp16", 1, 2, 1, 129, 129, 64, True)),
])
def test_noalloc_matches_attn_bwd_twice(lib, first, second):
    import torch
    for i, case in enumerate((first, second)):
        dt, b, h, hk, sq, sk, d, causal = case
        print(f"[gpu] attn_bwd_noalloc call {i}: {case}", flush=True)
        inp = make_case(dt, b, h, hk, sq, sk, d, seed=300 + i)
        ref, got = _run_both(lib, inp, causal)
        for name, a, bb in zip(("dq", "dk", "dv", "delta"), ref, got):
            assert a.shape == bb.shape
            assert torch.equal(a.contiguous().view(-1).view(torch.uint8),
                               bb.contiguous().view(-1).view(torch.uint8)), (i, name)
        want = oracle_run(inp, causal)
        for name, t in zip(("dq", "dk", "dv", "delta"), got):
            assert_close(name, to_f64(t), want[name], TOL[dt])


def test_noalloc_rejects_problems_beyond_the_array(lib):
    """More (query head, query row) pairs than the static array holds: refused
    before any launch with ATTN_ERR_WORKSPACE_TOO_SMALL."""
    import torch
    heads = 64
    s = lib.NOALLOC_SCRATCH_BYTES // 8 // heads + 64  # (query head, row) pairs just past the array
    q = torch.zeros(1, s, heads, 8, dtype=torch.float16, device="cuda")
    lse = torch.zeros(1, heads, s, dtype=torch.float32, device="cuda")
    with pytest.raises(lib.AttnError) as e:
        lib.attn_bwd_noalloc(q, q, q, q, lse, q)
    assert e.value.status == lib.ATTN_ERR_WORKSPACE_TOO_SMALL
