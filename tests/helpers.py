"""Shared test helpers: upload seeded inputs, run the GPU path, compare to the oracle."""
from __future__ import annotations

import math

import numpy as np

import workloads

# Tolerances on max|err| relative to max|ref| per output tensor.
TOL = {"fp16": 2e-2, "bf16": 4e-2}
LSE_ABS_TOL = 1e-3


def torch_dtype(name):
    import torch
    return {"fp16": torch.float16, "bf16": torch.bfloat16}[name]


def upload(bits: np.ndarray, dtype: str, device="cuda"):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(torch_dtype(dtype)).to(device)


def to_f64(t) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def rel_err(got: np.ndarray, ref: np.ndarray) -> float:
    scale = float(np.abs(ref).max()) if ref.size else 0.0
    if scale == 0.0:
        return float(np.abs(got).max()) if got.size else 0.0
    return float(np.abs(got - ref).max()) / scale


def assert_close(name: str, got: np.ndarray, ref: np.ndarray, tol: float):
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{name}: non-finite values"
    e = rel_err(got, ref)
    assert e <= tol, f"{name}: max|err|/max|ref| = {e:.3e} > {tol:.1e}"
    return e


def assert_lse_close(got: np.ndarray, ref: np.ndarray):
    inf_ref = np.isinf(ref)
    assert np.array_equal(np.isinf(got), inf_ref), "LSE: +inf pattern differs"
    if (~inf_ref).any():
        err = float(np.abs(got[~inf_ref] - ref[~inf_ref]).max())
        assert err <= LSE_ABS_TOL, f"LSE abs err {err:.3e}"


def make_case(dtype, b, h, hk, sq, sk, d, seed, lengths_q=None, lengths_k=None, do_scale=1.0):
    return workloads.make_inputs(dtype, b, h, hk, sq, sk, d, seed, do_scale=do_scale,
                                 varlen_lengths_q=lengths_q, varlen_lengths_k=lengths_k)


def gpu_run(lib, inp, causal, deterministic=False, scale=None, return_delta=True, window=(-1, -1)):
    """Forward then backward on the GPU through the C ABI."""
    import torch
    dt = inp["dtype"]
    q, k, v, do = (upload(inp[n + "_bits"], dt) for n in ("q", "k", "v", "do"))
    d = q.shape[-1]
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    kw = {}
    if "cu_seqlens_q" in inp:
        kw = dict(cu_seqlens_q=torch.from_numpy(inp["cu_seqlens_q"]).cuda(),
                  cu_seqlens_k=torch.from_numpy(inp["cu_seqlens_k"]).cuda(),
                  max_seqlen_q=int(inp["lengths_q"].max()) if len(inp["lengths_q"]) else 0,
                  max_seqlen_k=int(inp["lengths_k"].max()) if len(inp["lengths_k"]) else 0)
    o, lse = lib.attn_fwd(q, k, v, causal=causal, softmax_scale=scale, window=window, **kw)
    res = lib.attn_bwd(q, k, v, o, lse, do, causal=causal, softmax_scale=scale, deterministic=deterministic,
                       return_delta=return_delta, window=window, **kw)
    torch.cuda.synchronize()
    out = {"o": o, "lse": lse, "dq": res[0], "dk": res[1], "dv": res[2]}
    if return_delta:
        out["delta"] = res[3]
    return out


def oracle_run(inp, causal, scale=None, heads=None, window=(-1, -1)):
    import oracle
    d = inp["q"].shape[-1]
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    cq = inp.get("cu_seqlens_q")
    ck = inp.get("cu_seqlens_k")
    o, lse = oracle.attention_forward(inp["q"], inp["k"], inp["v"], scale, causal, cq, ck, heads=heads,
                                      window=window)
    dq, dk, dv, delta = oracle.attention_backward(inp["q"], inp["k"], inp["v"], inp["do"], scale, causal, cq, ck,
                                                  heads=heads, window=window)
    return {"o": o, "lse": lse, "dq": dq, "dk": dk, "dv": dv, "delta": delta}
