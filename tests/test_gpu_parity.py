"""GPU parity: the HIP path (through the C ABI) against the fp64 CPU oracle.

Element-by-element comparison on seeded inputs at sizes the oracle finishes in
seconds (several tiles, ragged tails, GQA, varlen, causal with Sq != Sk, rows
that see no key), and at the full workload sizes on every (sequence, head),
in the launch configuration bench.py times.  Bar: max|err| <= 2e-2 * max|ref|
(fp16) or 4e-2 * max|ref| (bf16) per output tensor; |LSE err| <= 1e-3; the
deterministic mode is bit-identical from run to run.
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
    # head dims 72-96 compute a 96-wide tile inside the 128-wide stored one
    ("d80_bf16_causal_gqa", "bf16", 2, 4, 2, 190, 190, 80, True, None),
    ("d72_fp16_noncausal_sq_lt_sk", "fp16", 1, 2, 2, 140, 203, 72, False, None),
    ("d104_fp16_causal", "fp16", 1, 2, 1, 160, 160, 104, True, None),
    # causal MHA at fixed lengths runs the four-wave dK/dV kernel (64-key
    # blocks): the 96-wide compute tile, a ragged last block, Sq != Sk
    ("d96_bf16_causal_mha_ragged", "bf16", 2, 2, 2, 190, 190, 96, True, None),
    ("d80_fp16_causal_mha_sq_gt_sk", "fp16", 1, 3, 3, 230, 101, 80, True, None),
    ("ragged_bf16_causal_mha_d128", "bf16", 2, 4, 4, 200, 200, 128, True, None),
    # the 64-wide tile: varlen with an empty and a short sequence, a 48-wide
    # head with Sq > Sk
    ("varlen_bf16_causal_d64_ragged", "bf16", 4, 4, 2, 0, 0, 64, True, ([33, 0, 200, 129], [33, 0, 200, 129])),
    ("d48_fp16_noncausal_sq_gt_sk", "fp16", 1, 2, 2, 260, 150, 48, False, None),
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


# Head dims above 128 run the 256-wide tile (the dK/dV kernel at one wave per
# SIMD, the four-wave dQ kernel with 32-key tiles); same layout as SMALL_CASES.
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


@pytest.mark.parametrize("case", WINDOW_CASES, ids=[c[0] for c in WINDOW_CASES])
def test_window_parity(lib, case):
    print(f"[gpu] window parity {case[0]}", flush=True)
    inp = _inputs(case[:10], seed=2024)
    causal, window = case[8], case[10]
    out = gpu_run(lib, inp, causal, window=window)
    ref = oracle_run(inp, causal, window=window)
    _compare(out, ref, case[1])


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


def _bits_t(t):
    return t.contiguous().view(-1).view(__import__("torch").int16)


def _repeat_identical(lib, inp, causal, runs, deterministic=True):
    """Backward `runs` times on the same GPU forward output; every run's dQ,
    dK, dV must be bit-identical to the first (compared on the GPU)."""
    import torch
    dt = inp["dtype"]
    q, k, v, do = (upload(inp[n + "_bits"], dt) for n in ("q", "k", "v", "do"))
    kw = {}
    if "cu_seqlens_q" in inp:
        kw = dict(cu_seqlens_q=torch.from_numpy(inp["cu_seqlens_q"]).cuda(),
                  cu_seqlens_k=torch.from_numpy(inp["cu_seqlens_k"]).cuda(),
                  max_seqlen_q=int(inp["lengths_q"].max()), max_seqlen_k=int(inp["lengths_k"].max()))
    o, lse = lib.attn_fwd(q, k, v, causal=causal, **kw)
    first = lib.attn_bwd(q, k, v, o, lse, do, causal=causal, deterministic=deterministic, **kw)
    for it in range(1, runs):
        out = lib.attn_bwd(q, k, v, o, lse, do, causal=causal, deterministic=deterministic, **kw)
        for name, a_, b_ in zip(("dq", "dk", "dv"), first, out):
            assert torch.equal(_bits_t(a_), _bits_t(b_)), (it, name)
    torch.cuda.synchronize()
    return first


def test_workload_mha_causal_fp16_b2_h8_s1024_d64_deterministic(lib):
    """The causal fp16 S1024 workload: parity with the oracle with and without
    the deterministic flag, and 10 backward runs bit-identical.  dQ never uses
    atomics here, so the two flag values run the same ordered path and must
    agree bit for bit too."""
    name = "mha_causal_fp16_b2_h8_s1024_d64"
    print(f"[gpu] workload {name}", flush=True)
    w = workloads.WORKLOADS[name]
    inp = workloads.make_workload_inputs(name)
    ref = oracle_run(inp, w.causal)
    out = gpu_run(lib, inp, w.causal, deterministic=False)
    _compare(out, ref, w.dtype)
    out_d = gpu_run(lib, inp, w.causal, deterministic=True)
    _compare(out_d, ref, w.dtype)
    for n in ("dq", "dk", "dv"):
        assert np.array_equal(_bits(out[n]), _bits(out_d[n])), n
    _repeat_identical(lib, inp, w.causal, 10)


def test_workload_mha_causal_bf16_b4_h16_s4096_d128_bit_identical(lib):
    """The timed workload: 10 backward runs bit-identical."""
    name = "mha_causal_bf16_b4_h16_s4096_d128"
    print(f"[gpu] bit identity {name}", flush=True)
    w = workloads.WORKLOADS[name]
    _repeat_identical(lib, workloads.make_workload_inputs(name), w.causal, 10)


def _full_size(lib, name):
    """Run the whole workload on the GPU as bench.py launches it; compare every
    (sequence, KV head group) -- O, LSE, Delta, dQ, dK, dV -- to the oracle."""
    import oracle
    w = workloads.ALL_WORKLOADS[name]
    inp = workloads.make_workload_inputs(name)
    out = gpu_run(lib, inp, w.causal)
    scale = 1.0 / math.sqrt(w.head_dim)
    G = w.heads_q // w.heads_kv
    tol = TOL[w.dtype]
    res = {n: to_f64(out[n]) for n in ("o", "lse", "dq", "dk", "dv", "delta")}
    del out
    nseq = len(inp["lengths_q"]) if w.varlen else w.batch
    want = {n: np.zeros_like(res[n]) for n in res}
    for z in range(nseq):
        if w.varlen:
            cq = inp["cu_seqlens_q"]
            sl = slice(int(cq[z]), int(cq[z + 1]))
            q, k, v, do = (inp[n][None, sl] for n in ("q", "k", "v", "do"))
        else:
            q, k, v, do = (inp[n][z:z + 1] for n in ("q", "k", "v", "do"))
        for g in range(w.heads_kv):
            heads = list(range(g * G, (g + 1) * G))
            hs = np.array(heads)
            o, lse = oracle.attention_forward(q, k, v, scale, w.causal, heads=heads)
            dq, dk, dv, delta = oracle.attention_backward(q, k, v, do, scale, w.causal, heads=heads)
            if w.varlen:
                want["o"][sl, hs] = o[0][:, hs]
                want["dq"][sl, hs] = dq[0][:, hs]
                want["dk"][sl, g] = dk[0][:, g]
                want["dv"][sl, g] = dv[0][:, g]
                want["lse"][hs, sl] = lse[0][hs]
                want["delta"][hs, sl] = delta[0][hs]
            else:
                want["o"][z][:, hs] = o[0][:, hs]
                want["dq"][z][:, hs] = dq[0][:, hs]
                want["dk"][z][:, g] = dk[0][:, g]
                want["dv"][z][:, g] = dv[0][:, g]
                want["lse"][z][hs] = lse[0][hs]
                want["delta"][z][hs] = delta[0][hs]
    errs = {}
    for n in ("o", "delta", "dq", "dk", "dv"):
        errs[n] = assert_close(n, res[n], want[n], tol)
    assert_lse_close(res["lse"], want["lse"])
    print(f"[gpu] {name}: " + " ".join(f"{n} {e:.2e}" for n, e in errs.items()), flush=True)
    return res


def test_workload_mha_causal_bf16_b4_h16_s4096_d128_full(lib):
    print("[gpu] full-size causal bf16 B4 H16 S4096 d128, every head", flush=True)
    _full_size(lib, "mha_causal_bf16_b4_h16_s4096_d128")


def test_workload_gqa_bf16_b2_hq32_hk8_s4096_d128_full(lib):
    print("[gpu] full-size GQA bf16 B2 Hq32 Hk8 S4096 d128, every head", flush=True)
    _full_size(lib, "gqa_bf16_b2_hq32_hk8_s4096_d128")


def test_workload_varlen_causal_fp16_16seq_h16_d96_full(lib):
    print("[gpu] full-size varlen causal fp16 16 seqs H16 d96, every sequence and head", flush=True)
    _full_size(lib, "varlen_causal_fp16_16seq_h16_d96")


def test_measured_shape_causal_fp16_b4_h16_s4096_d128_full(lib):
    print("[gpu] full-size causal fp16 B4 H16 S4096 d128, every head", flush=True)
    _full_size(lib, "mha_causal_fp16_b4_h16_s4096_d128")


def test_measured_shape_causal_bf16_b2_h16_s4096_d256_full(lib):
    print("[gpu] full-size causal bf16 B2 H16 S4096 d256, every head", flush=True)
    _full_size(lib, "mha_causal_bf16_b2_h16_s4096_d256")


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


def test_strided_layouts_packed_qkv(lib):
    """Q, K, V as views of one packed [B, S, 3, H, d] tensor, dO with a padded
    head stride, and dQ, dK, dV written into views of a packed gradient
    tensor: the kernels follow the strides (row and head strides are
    multiples of 8 elements, the last dimension contiguous)."""
    import torch
    print("[gpu] strided layouts: packed qkv, padded dO, packed gradients", flush=True)
    b, h, s_len, d = 2, 4, 200, 64
    inp = make_case("bf16", b, h, h, s_len, s_len, d, seed=4242)
    q, k, v, do = (upload(inp[n + "_bits"], "bf16") for n in ("q", "k", "v", "do"))
    qkv = torch.empty(b, s_len, 3, h, d, dtype=q.dtype, device=q.device)
    qkv[:, :, 0], qkv[:, :, 1], qkv[:, :, 2] = q, k, v
    qs, ks, vs = qkv.unbind(2)
    assert qs.stride(1) == 3 * h * d and not qs.is_contiguous()
    dop = torch.zeros(b, s_len, h, d + 8, dtype=q.dtype, device=q.device)
    dop[..., :d] = do
    dos = dop[..., :d]
    grads = torch.full((b, s_len, 3, h, d), float("nan"), dtype=q.dtype, device=q.device)
    dqs, dks, dvs = grads.unbind(2)
    scale = 1.0 / math.sqrt(d)
    o, lse = lib.attn_fwd(qs, ks, vs, causal=True, softmax_scale=scale)
    res = lib.attn_bwd(qs, ks, vs, o, lse, dos, causal=True, softmax_scale=scale, dq=dqs, dk=dks, dv=dvs,
                       return_delta=True)
    torch.cuda.synchronize()
    ref = oracle_run(inp, True)
    out = {"o": o, "lse": lse, "dq": dqs, "dk": dks, "dv": dvs, "delta": res[3]}
    _compare(out, ref, "bf16")
    # the same gradients as the contiguous layout, bit for bit
    base = gpu_run(lib, inp, True)
    for name, t in (("dq", dqs), ("dk", dks), ("dv", dvs)):
        assert np.array_equal(_bits(t), _bits(base[name])), name


def test_strided_layouts_packed_kv_gqa(lib):
    """GQA with K and V as views of one packed [B, S, 2, Hk, d] tensor."""
    import torch
    print("[gpu] strided layouts: packed kv, GQA", flush=True)
    b, h, hk, s_len, d = 1, 8, 2, 190, 128
    inp = make_case("fp16", b, h, hk, s_len, s_len, d, seed=4243)
    q, k, v, do = (upload(inp[n + "_bits"], "fp16") for n in ("q", "k", "v", "do"))
    kv = torch.empty(b, s_len, 2, hk, d, dtype=q.dtype, device=q.device)
    kv[:, :, 0], kv[:, :, 1] = k, v
    ks, vs = kv.unbind(2)
    scale = 1.0 / math.sqrt(d)
    o, lse = lib.attn_fwd(q, ks, vs, causal=False, softmax_scale=scale)
    dq, dk, dv, delta = lib.attn_bwd(q, ks, vs, o, lse, do, causal=False, softmax_scale=scale, return_delta=True)
    torch.cuda.synchronize()
    ref = oracle_run(inp, False)
    _compare({"o": o, "lse": lse, "dq": dq, "dk": dk, "dv": dv, "delta": delta}, ref, "fp16")


# The phase API: the dQ kernel runs the preprocess for its own rows, so
# DQ then DKDV is the full backward; the standalone preprocess (PREPROCESS
# without DQ) writes the same workspace rows for a later dK/dV launch.
PHASE_CASES = [
    ("phases_bf16_causal_ragged_d128", "bf16", 2, 4, 2, 200, 200, 128, True, None),
    ("phases_fp16_varlen_d96", "fp16", 4, 4, 2, 0, 0, 96, True, ([1, 130, 257, 64], [1, 130, 257, 64])),
    ("phases_bf16_gqa_d256", "bf16", 1, 4, 2, 150, 170, 256, False, None),
]


@pytest.mark.parametrize("case", PHASE_CASES, ids=[c[0] for c in PHASE_CASES])
def test_phases_split_matches_full(lib, case):
    import torch
    print(f"[gpu] phases {case[0]}", flush=True)
    inp = _inputs(case, seed=77)
    name, dt, causal = case[0], case[1], case[8]
    q, k, v, do = (upload(inp[n + "_bits"], dt) for n in ("q", "k", "v", "do"))
    kw = {}
    if "cu_seqlens_q" in inp:
        kw = dict(cu_seqlens_q=torch.from_numpy(inp["cu_seqlens_q"]).cuda(),
                  cu_seqlens_k=torch.from_numpy(inp["cu_seqlens_k"]).cuda(),
                  max_seqlen_q=int(inp["lengths_q"].max()), max_seqlen_k=int(inp["lengths_k"].max()))
    scale = 1.0 / math.sqrt(q.shape[-1])
    o, lse = lib.attn_fwd(q, k, v, causal=causal, softmax_scale=scale, **kw)
    p = lib.make_params(q, k, causal, scale, False, kw.get("cu_seqlens_q"), kw.get("cu_seqlens_k"),
                        kw.get("max_seqlen_q"), kw.get("max_seqlen_k"))
    nbytes = max(lib.bwd_workspace_size(p), 256)

    def fresh_ws():  # NaN bit patterns: a phase that reads unwritten rows shows up
        return torch.full((nbytes,), 0xFF, dtype=torch.uint8, device="cuda")

    def outs():
        return torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)

    full = lib.attn_bwd(q, k, v, o, lse, do, causal=causal, softmax_scale=scale, return_delta=True,
                        workspace=fresh_ws(), **kw)
    # dQ (with its preprocess), then dK/dV in a second call on the same workspace
    ws = fresh_ws()
    dq, dk, dv = outs()
    common = dict(causal=causal, softmax_scale=scale, dq=dq, dk=dk, dv=dv, workspace=ws, **kw)
    r1 = lib.attn_bwd(q, k, v, o, lse, do, phases=lib.PHASE_DQ, return_delta=True, **common)
    lib.attn_bwd(q, k, v, o, lse, do, phases=lib.PHASE_DKDV, **common)
    torch.cuda.synchronize()
    for a_, b_, n in ((dq, full[0], "dq"), (dk, full[1], "dk"), (dv, full[2], "dv"), (r1[3], full[3], "delta")):
        assert torch.equal(a_.view(torch.int16) if a_.dtype != torch.float32 else a_.view(torch.int32),
                           b_.view(torch.int16) if b_.dtype != torch.float32 else b_.view(torch.int32)), n
    # the standalone preprocess, then dK/dV and dQ one call each
    ws = fresh_ws()
    dq, dk, dv = outs()
    common = dict(causal=causal, softmax_scale=scale, dq=dq, dk=dk, dv=dv, workspace=ws, **kw)
    r0 = lib.attn_bwd(q, k, v, o, lse, do, phases=lib.PHASE_PREPROCESS, return_delta=True, **common)
    lib.attn_bwd(q, k, v, o, lse, do, phases=lib.PHASE_DKDV, **common)
    lib.attn_bwd(q, k, v, o, lse, do, phases=lib.PHASE_DQ, **common)
    torch.cuda.synchronize()
    assert torch.equal(dq.view(torch.int16), full[0].view(torch.int16)), "dq"
    ref = oracle_run(inp, causal)
    got = {"o": o, "lse": lse, "dq": dq, "dk": dk, "dv": dv, "delta": r0[3]}
    _compare(got, ref, dt)
    # both preprocess paths give Delta to fp32 rounding
    d0, d1 = to_f64(r0[3]), to_f64(full[3])
    assert np.abs(d0 - d1).max() <= 1e-5 * max(1.0, np.abs(d1).max())
