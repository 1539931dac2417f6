"""GPU parity: the HIP path (through the C ABI) against the fp64 CPU oracle.

Element-by-element comparison on seeded inputs at sizes the oracle finishes in
seconds (several tiles, ragged tails, GQA, varlen, causal with Sq != Sk, rows
that see no key), and at the full workload sizes on sampled heads plus
properties that hold at any size.  Bar: max|err| <= 2e-2 * max|ref| (fp16) or
4e-2 * max|ref| (bf16) per output tensor; |LSE err| <= 1e-3; the deterministic
mode is bit-identical from run to run.
"""
import math

import numpy as np
import pytest

import workloads
from helpers import (TOL, assert_close, assert_lse_close, gpu_run, make_case, oracle_run, to_f64, upload)

pytestmark = pytest.mark.gpu

# name, dtype, b, h, hk, sq, sk, d, causal, (lengths_q, lengths_k) or None
SMALL_CASES = [
    ("mha_fp16_b1_h2_s128_d64", "fp16", 1, 2, 2, 128, 128, 64, False, None),
    ("ragged_bf16_causal_d128", "bf16", 2, 4, 2, 200, 200, 128, True, None),
    ("sq_lt_sk_fp16_causal_d64", "fp16", 1, 2, 1, 77, 301, 64, True, None),
    ("sq_gt_sk_bf16_causal_d128", "bf16", 1, 2, 2, 300, 130, 128, True, None),
    ("gqa_fp16_noncausal_d128", "fp16", 1, 8, 2, 257, 190, 128, False, None),
    ("gqa_bf16_causal_d64_mqa", "bf16", 2, 4, 1, 150, 150, 64, True, None),
    ("varlen_fp16_causal_d96", "fp16", 4, 4, 2, 0, 0, 96, True, ([1, 130, 257, 64], [1, 130, 257, 64])),
    ("varlen_bf16_noncausal_d96_klen", "bf16", 3, 2, 2, 0, 0, 96, False, ([100, 3, 65], [40, 129, 1])),
    ("varlen_fp16_causal_d128_empty_seq", "fp16", 3, 2, 2, 0, 0, 128, True, ([5, 0, 70], [5, 0, 70])),
    ("d32_fp16_causal", "fp16", 1, 2, 2, 70, 70, 32, True, None),
    ("d8_bf16", "bf16", 2, 1, 1, 33, 45, 8, False, None),
    ("s1_fp16_causal", "fp16", 1, 2, 2, 1, 1, 64, True, None),
]


def _bits(t):
    import torch
    return t.contiguous().view(torch.int16).cpu().numpy().copy()


def _inputs(case, seed=1234):
    name, dt, b, h, hk, sq, sk, d, causal, lens = case
    if lens is None:
        return make_case(dt, b, h, hk, sq, sk, d, seed)
    return make_case(dt, b, h, hk, 0, 0, d, seed, lengths_q=lens[0], lengths_k=lens[1])


def _compare(out, ref, dt, what=("o", "dq", "dk", "dv", "delta")):
    tol = TOL[dt]
    errs = {}
    for name in what:
        errs[name] = assert_close(name, to_f64(out[name]), ref[name], tol)
    assert_lse_close(to_f64(out["lse"]), ref["lse"])
    return errs


@pytest.mark.parametrize("case", SMALL_CASES, ids=[c[0] for c in SMALL_CASES])
def test_small_parity(lib, case):
    print(f"[gpu] small parity {case[0]}", flush=True)
    inp = _inputs(case)
    causal = case[8]
    out = gpu_run(lib, inp, causal)
    ref = oracle_run(inp, causal)
    _compare(out, ref, case[1])


@pytest.mark.parametrize("case", SMALL_CASES, ids=[c[0] for c in SMALL_CASES])
def test_small_parity_minimal_workspace(lib, case):
    """The path for a Delta-only workspace: the dQ kernel recomputes dS."""
    print(f"[gpu] small parity, minimal workspace {case[0]}", flush=True)
    inp = _inputs(case, seed=4321)
    causal = case[8]
    out = gpu_run(lib, inp, causal, minimal_workspace=True)
    ref = oracle_run(inp, causal)
    _compare(out, ref, case[1])


# Head dims above 128 run the 256-wide tile (dK/dV in one kernel, dQ as two
# 128-wide halves of the stored-dS product); same layout as SMALL_CASES.
WIDE_CASES = [
    ("d256_bf16_causal_ragged", "bf16", 2, 4, 2, 200, 200, 256, True, None),
    ("d192_fp16_noncausal_gqa", "fp16", 1, 8, 2, 257, 190, 192, False, None),
    ("d256_fp16_causal_sq_lt_sk", "fp16", 1, 2, 1, 77, 301, 256, True, None),
    ("d192_bf16_varlen_causal", "bf16", 4, 4, 2, 0, 0, 192, True, ([1, 130, 257, 64], [1, 130, 257, 64])),
    ("d136_fp16_causal", "fp16", 1, 2, 2, 150, 150, 136, True, None),
    ("d256_bf16_noncausal_s1", "bf16", 1, 2, 2, 1, 1, 256, False, None),
]


@pytest.mark.parametrize("case", WIDE_CASES, ids=[c[0] for c in WIDE_CASES])
def test_wide_head_dim_parity(lib, case):
    print(f"[gpu] wide head dim parity {case[0]}", flush=True)
    inp = _inputs(case, seed=777)
    causal = case[8]
    out = gpu_run(lib, inp, causal)
    ref = oracle_run(inp, causal)
    _compare(out, ref, case[1])


def test_wide_head_dim_window_and_determinism(lib):
    """A local window at d = 256, and bit-identical gradients from run to run."""
    print("[gpu] wide head dim window + determinism d256 bf16", flush=True)
    case = ("d256_window", "bf16", 1, 2, 2, 300, 300, 256, False, None)
    inp = _inputs(case, seed=778)
    a = gpu_run(lib, inp, False, window=(100, 20))
    b = gpu_run(lib, inp, False, window=(100, 20))
    ref = oracle_run(inp, False, window=(100, 20))
    _compare(a, ref, "bf16")
    for name in ("dq", "dk", "dv"):
        assert np.array_equal(_bits(a[name]), _bits(b[name])), name


# local (sliding-window) attention: name, dtype, b, h, hk, sq, sk, d, causal, lens, (left, right)
WINDOW_CASES = [
    ("window_fp16_l100_r30_d64", "fp16", 1, 2, 2, 300, 300, 64, False, None, (100, 30)),
    ("window_bf16_causal_l150_d128", "bf16", 2, 4, 2, 333, 333, 128, True, None, (150, -1)),
    ("window_bf16_sq_lt_sk_l0_r70_d128", "bf16", 1, 2, 1, 90, 260, 128, False, None, (0, 70)),
    ("window_fp16_sq_gt_sk_l40_r0_d64", "fp16", 1, 2, 2, 270, 100, 64, False, None, (40, 0)),
    ("window_fp16_left_only_d96", "fp16", 1, 2, 2, 200, 200, 96, False, None, (70, -1)),
    ("window_bf16_varlen_l64_r64_d128", "bf16", 3, 2, 2, 0, 0, 128, False, ([300, 17, 129], [300, 17, 129]), (64, 64)),
    ("window_fp16_tiny_l0_r0_d32", "fp16", 1, 2, 2, 100, 100, 32, False, None, (0, 0)),
]


@pytest.mark.parametrize("minimal", [False, True], ids=["stored_ds", "recompute"])
@pytest.mark.parametrize("case", WINDOW_CASES, ids=[c[0] for c in WINDOW_CASES])
def test_window_parity(lib, case, minimal):
    print(f"[gpu] window parity {case[0]} minimal={minimal}", flush=True)
    inp = _inputs(case[:10], seed=2024)
    causal, window = case[8], case[10]
    out = gpu_run(lib, inp, causal, minimal_workspace=minimal, window=window)
    ref = oracle_run(inp, causal, window=window)
    _compare(out, ref, case[1])


def test_both_workspace_paths_agree(lib):
    """dK, dV identical; dQ within the rounding of the same operations."""
    print("[gpu] fast vs minimal workspace, ragged causal bf16 d128", flush=True)
    case = SMALL_CASES[1]
    inp = _inputs(case, seed=7)
    a = gpu_run(lib, inp, True)
    b = gpu_run(lib, inp, True, minimal_workspace=True)
    for n in ("dk", "dv"):
        assert np.array_equal(_bits(a[n]), _bits(b[n])), n
    da, db = to_f64(a["dq"]), to_f64(b["dq"])
    assert np.max(np.abs(da - db)) <= 1e-2 * np.max(np.abs(db))


@pytest.mark.parametrize("case", [SMALL_CASES[1], SMALL_CASES[4], SMALL_CASES[6]], ids=lambda c: c[0])
def test_small_parity_deterministic(lib, case):
    print(f"[gpu] deterministic parity {case[0]}", flush=True)
    inp = _inputs(case, seed=99)
    causal = case[8]
    out = gpu_run(lib, inp, causal, deterministic=True)
    ref = oracle_run(inp, causal)
    _compare(out, ref, case[1])
    out2 = gpu_run(lib, inp, causal, deterministic=True)
    for n in ("dq", "dk", "dv"):
        assert np.array_equal(_bits(out[n]), _bits(out2[n])), n


def test_softmax_scale_is_a_parameter(lib):
    print("[gpu] custom softmax scale", flush=True)
    inp = make_case("fp16", 1, 2, 2, 96, 96, 64, 7)
    out = gpu_run(lib, inp, True, scale=0.05)
    ref = oracle_run(inp, True, scale=0.05)
    _compare(out, ref, "fp16")


def test_workload_mha_fp16_b1_h2_s128_d64(lib):
    """Forward + backward at the full size of the small non-causal workload."""
    name = "mha_fp16_b1_h2_s128_d64"
    print(f"[gpu] workload {name}", flush=True)
    w = workloads.ALL_WORKLOADS[name]
    inp = workloads.make_workload_inputs(name)
    out = gpu_run(lib, inp, w.causal)
    ref = oracle_run(inp, w.causal)
    _compare(out, ref, w.dtype)


def test_workload_mha_causal_fp16_b2_h8_s1024_d64_atomic_and_deterministic(lib):
    name = "mha_causal_fp16_b2_h8_s1024_d64"
    print(f"[gpu] workload {name}", flush=True)
    w = workloads.WORKLOADS[name]
    inp = workloads.make_workload_inputs(name)
    ref = oracle_run(inp, w.causal)
    out = gpu_run(lib, inp, w.causal, deterministic=False)
    _compare(out, ref, w.dtype)
    first = None
    for it in range(10):
        out_d = gpu_run(lib, inp, w.causal, deterministic=True)
        if first is None:
            _compare(out_d, ref, w.dtype)
            first = {n: _bits(out_d[n]) for n in ("dq", "dk", "dv")}
        else:
            for n in ("dq", "dk", "dv"):
                assert np.array_equal(first[n], _bits(out_d[n])), (it, n)


def _full_size_sampled(lib, name, samples):
    """Run the whole workload on the GPU; compare sampled (sequence, KV head) slices to the oracle."""
    import oracle
    w = workloads.ALL_WORKLOADS[name]
    inp = workloads.make_workload_inputs(name)
    out = gpu_run(lib, inp, w.causal)
    scale = 1.0 / math.sqrt(w.head_dim)
    G = w.heads_q // w.heads_kv
    tol = TOL[w.dtype]
    res = {n: to_f64(out[n]) for n in ("o", "lse", "dq", "dk", "dv", "delta")}
    for z, g in samples:
        heads = list(range(g * G, (g + 1) * G))
        if w.varlen:
            cq = inp["cu_seqlens_q"]
            a, e = int(cq[z]), int(cq[z + 1])
            sl = slice(a, e)
            q, k, v, do = (inp[n][None, sl] for n in ("q", "k", "v", "do"))
            got = {n: res[n][None, sl] for n in ("o", "dq", "dk", "dv")}
            got["lse"] = res["lse"][None, :, sl]
            got["delta"] = res["delta"][None, :, sl]
        else:
            q, k, v, do = (inp[n][z:z + 1] for n in ("q", "k", "v", "do"))
            got = {n: res[n][z:z + 1] for n in ("o", "dq", "dk", "dv")}
            got["lse"] = res["lse"][z:z + 1]
            got["delta"] = res["delta"][z:z + 1]
        o, lse = oracle.attention_forward(q, k, v, scale, w.causal, heads=heads)
        dq, dk, dv, delta = oracle.attention_backward(q, k, v, do, scale, w.causal, heads=heads)
        hs = np.array(heads)
        assert_close("o", got["o"][:, :, hs], o[:, :, hs], tol)
        assert_lse_close(got["lse"][:, hs], lse[:, hs])
        assert_close("delta", got["delta"][:, hs], delta[:, hs], tol)
        assert_close("dq", got["dq"][:, :, hs], dq[:, :, hs], tol)
        assert_close("dk", got["dk"][:, :, g], dk[:, :, g], tol)
        assert_close("dv", got["dv"][:, :, g], dv[:, :, g], tol)
    # properties at any size: sum over keys of dK is ~0; sum over keys of dV = sum of the group's dO
    dk_all, dv_all = res["dk"], res["dv"]
    do_all = inp["do"].astype(np.float64)
    if w.varlen:
        cq = inp["cu_seqlens_q"]
        for z in range(len(cq) - 1):
            sl = slice(int(cq[z]), int(cq[z + 1]))
            _sum_checks(dk_all[sl][None], dv_all[sl][None], do_all[sl][None], G)
    else:
        _sum_checks(dk_all, dv_all, do_all, G)
    return res


def _sum_checks(dk, dv, do, G):
    b, sk, hk, d = dk.shape
    s_dk = dk.sum(axis=1)
    assert np.abs(s_dk).max() <= 1e-2 * np.abs(dk).sum(axis=1).max() + 1e-6
    want = do.sum(axis=1).reshape(b, hk, G, d).sum(axis=2)
    assert np.abs(dv.sum(axis=1) - want).max() <= 2e-2 * max(np.abs(want).max(), 1e-6)


def test_measured_shape_causal_bf16_b2_h16_s4096_d256_sampled(lib):
    """The head-dim-256 shape bench.py measures, at full size in its launch
    configuration: sampled heads against the oracle plus the sum properties."""
    print("[gpu] full-size causal bf16 B2 H16 S4096 d256 (sampled heads)", flush=True)
    _full_size_sampled(lib, "mha_causal_bf16_b2_h16_s4096_d256", [(0, 0), (1, 15)])


def test_measured_shape_causal_fp16_b4_h16_s4096_d128_sampled(lib):
    print("[gpu] full-size causal fp16 B4 H16 S4096 d128 (sampled heads)", flush=True)
    _full_size_sampled(lib, "mha_causal_fp16_b4_h16_s4096_d128", [(2, 7)])


def test_workload_mha_causal_bf16_b4_h16_s4096_d128_sampled(lib):
    print("[gpu] full-size causal bf16 B4 H16 S4096 d128 (sampled heads)", flush=True)
    _full_size_sampled(lib, "mha_causal_bf16_b4_h16_s4096_d128", [(0, 0), (3, 15)])


def test_workload_gqa_bf16_b2_hq32_hk8_s4096_d128_sampled(lib):
    print("[gpu] full-size GQA bf16 B2 Hq32 Hk8 S4096 d128 (sampled KV head)", flush=True)
    _full_size_sampled(lib, "gqa_bf16_b2_hq32_hk8_s4096_d128", [(1, 5)])


def test_workload_varlen_causal_fp16_16seq_h16_d96_sampled(lib):
    print("[gpu] full-size varlen causal fp16 16 seqs H16 d96 (sampled sequences)", flush=True)
    _full_size_sampled(lib, "varlen_causal_fp16_16seq_h16_d96", [(3, 2), (9, 11)])


def test_empty_query_gives_zero_dk_dv(lib):
    import torch
    print("[gpu] Sq == 0", flush=True)
    q = torch.zeros(1, 0, 2, 64, dtype=torch.float16, device="cuda")
    k = torch.randn(1, 70, 2, 64, dtype=torch.float16, device="cuda")
    v = torch.randn_like(k)
    o = torch.zeros_like(q)
    lse = torch.zeros(1, 2, 0, dtype=torch.float32, device="cuda")
    dk = torch.full_like(k, 7.0)
    dv = torch.full_like(v, 7.0)
    lib.attn_bwd(q, k, v, o, lse, q, causal=False, dk=dk, dv=dv)
    torch.cuda.synchronize()
    assert dk.abs().max().item() == 0.0 and dv.abs().max().item() == 0.0


def test_empty_keys_give_zero_output_and_dq(lib):
    import torch
    print("[gpu] Sk == 0", flush=True)
    q = torch.randn(1, 40, 2, 64, dtype=torch.bfloat16, device="cuda")
    k = torch.zeros(1, 0, 2, 64, dtype=torch.bfloat16, device="cuda")
    o, lse = lib.attn_fwd(q, k, k, causal=False)
    dq, dk, dv = lib.attn_bwd(q, k, k, o, lse, torch.randn_like(q), causal=False)
    torch.cuda.synchronize()
    assert o.abs().max().item() == 0.0
    assert torch.isinf(lse).all().item()
    assert dq.abs().max().item() == 0.0


def test_causal_row_zero_of_dq(lib):
    """Query 0 sees only key 0: P00 = 1 and dS00 = 0, so dQ row 0 is ~0."""
    print("[gpu] causal dQ row 0", flush=True)
    inp = make_case("bf16", 2, 4, 4, 256, 256, 128, 17)
    out = gpu_run(lib, inp, True)
    dq = to_f64(out["dq"])
    assert np.abs(dq[:, 0]).max() <= 1e-3 * np.abs(dq).max()


def test_outputs_fully_overwritten(lib):
    """dq/dk/dv buffers pre-filled with garbage are fully overwritten."""
    import torch
    print("[gpu] outputs overwritten", flush=True)
    inp = make_case("fp16", 2, 4, 2, 100, 100, 64, 5)
    q, k, v, do = (upload(inp[n + "_bits"], "fp16") for n in ("q", "k", "v", "do"))
    o, lse = lib.attn_fwd(q, k, v, causal=True)
    dq = torch.full_like(q, float("nan"))
    dk = torch.full_like(k, float("nan"))
    dv = torch.full_like(v, float("nan"))
    ws = torch.full((1 << 22,), 255, dtype=torch.uint8, device="cuda")
    lib.attn_bwd(q, k, v, o, lse, do, causal=True, dq=dq, dk=dk, dv=dv, workspace=ws)
    torch.cuda.synchronize()
    for t in (dq, dk, dv):
        assert torch.isfinite(t).all().item()
    ref = oracle_run(inp, True)
    assert_close("dq", to_f64(dq), ref["dq"], TOL["fp16"])
