"""Seeded synthetic inputs for attention forward/backward.

This module only draws random numbers and rounds them to the 16-bit storage
types; it holds none of the attention arithmetic.  Both the CPU oracle's tests
and the GPU path's tests/bench take their inputs from here, so both sides see
bit-identical values.

Recipe (every workload):
  * ``rng = numpy.random.default_rng(seed)``;
  * varlen only: ``lengths = rng.integers(lo, hi, size=n_seq, endpoint=True)``
    and ``cu_seqlens = [0, cumsum(lengths)]`` (int32);
  * then Q, K, V, dO in that order, each ``rng.standard_normal(shape, float32)``;
  * optional ``dO *= do_scale`` (0.1 for the bf16 causal d=128 workload);
  * round to fp16 (IEEE round-to-nearest-even via numpy) or to bf16
    (round-to-nearest-even on the float32 bit pattern).

Layouts: fixed length ``[batch, seq, heads, head_dim]``; varlen packed
``[total, heads, head_dim]``.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

__all__ = [
    "Workload",
    "WORKLOADS",
    "DEFAULT_BENCH_WORKLOAD",
    "BENCH_EXTRA",
    "ALL_WORKLOADS",
    "PARITY_SMALL_WORKLOAD",
    "round_bf16_bits",
    "bf16_bits_to_f32",
    "make_inputs",
    "attention_flops",
]


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    dtype: str  # "fp16" | "bf16"
    batch: int  # number of sequences when varlen
    heads_q: int
    heads_kv: int
    seqlen: int  # fixed length (Sq == Sk); 0 for varlen
    head_dim: int
    causal: bool
    seed: int
    do_scale: float = 1.0
    varlen_range: Optional[tuple] = None  # (lo, hi) inclusive, lengths ~ U[lo, hi]
    deterministic_too: bool = False
    note: str = ""

    @property
    def varlen(self) -> bool:
        return self.varlen_range is not None


# The five workloads the method is exercised on.  Seeds 42..46 in this order.
WORKLOADS = {
    w.name: w
    for w in [
        Workload("mha_fp16_b1_h2_s128_d64", "fp16", 1, 2, 2, 128, 64, False, 42,
                 note="forward + backward, non-causal"),
        Workload("mha_causal_fp16_b2_h8_s1024_d64", "fp16", 2, 8, 8, 1024, 64, True, 43,
                 deterministic_too=True, note="atomic and deterministic dQ"),
        Workload("mha_causal_bf16_b4_h16_s4096_d128", "bf16", 4, 16, 16, 4096, 128, True, 44,
                 do_scale=0.1, note="dO scaled by 0.1; the timed workload"),
        Workload("gqa_bf16_b2_hq32_hk8_s4096_d128", "bf16", 2, 32, 8, 4096, 128, False, 45,
                 note="dK/dV summed over the 4 query heads of a KV head"),
        Workload("varlen_causal_fp16_16seq_h16_d96", "fp16", 16, 16, 16, 0, 96, True, 46,
                 varlen_range=(256, 4096), note="packed sequences, causal per sequence"),
    ]
}
# Measurement-only shapes for bench.py --workload (not parity configs): the
# timed workload in fp16 (the fp16/bf16 matrix peaks are equal), and the
# 256-wide head-dim tile.  Seeds continue after the five above.
BENCH_EXTRA = {
    w.name: w
    for w in [
        Workload("mha_causal_fp16_b4_h16_s4096_d128", "fp16", 4, 16, 16, 4096, 128, True, 47,
                 do_scale=0.1, note="the timed workload in fp16"),
        Workload("mha_causal_bf16_b2_h16_s4096_d256", "bf16", 2, 16, 16, 4096, 256, True, 48,
                 do_scale=0.1, note="head dim 256"),
    ]
}
ALL_WORKLOADS = {**WORKLOADS, **BENCH_EXTRA}
DEFAULT_BENCH_WORKLOAD = "mha_causal_bf16_b4_h16_s4096_d128"
PARITY_SMALL_WORKLOAD = "mha_fp16_b1_h2_s128_d64"


def round_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit pattern (uint16), round to nearest, ties to even."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (b + 0x7FFF + ((b >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _round(x: np.ndarray, dtype: str):
    """Return (bits uint16, exact value as float32) of x rounded to dtype."""
    if dtype == "fp16":
        h = x.astype(np.float16)
        return h.view(np.uint16), h.astype(np.float32)
    if dtype == "bf16":
        bits = round_bf16_bits(x)
        return bits, bf16_bits_to_f32(bits)
    raise ValueError(dtype)


def make_inputs(
    dtype: str,
    batch: int,
    heads_q: int,
    heads_kv: int,
    seqlen_q: int,
    seqlen_k: int,
    head_dim: int,
    seed: int,
    do_scale: float = 1.0,
    varlen_lengths_q=None,
    varlen_lengths_k=None,
    varlen_range=None,
    dist: str = "normal",
):
    """Draw Q, K, V, dO.

    Returns a dict with float32 arrays holding the exactly-rounded values
    (``q, k, v, do``), their 16-bit patterns (``q_bits`` ...), and for varlen
    ``cu_seqlens_q``/``cu_seqlens_k`` (int32) and ``lengths_q``/``lengths_k``.
    ``varlen_range=(lo, hi)`` draws ``batch`` lengths first (shared by q and k).
    """
    rng = np.random.default_rng(seed)
    out = {"dtype": dtype, "seed": seed}
    if varlen_range is not None:
        lo, hi = varlen_range
        lengths = rng.integers(lo, hi, size=batch, endpoint=True).astype(np.int64)
        varlen_lengths_q = lengths
        varlen_lengths_k = lengths
    if varlen_lengths_q is not None:
        lq = np.asarray(varlen_lengths_q, dtype=np.int64)
        lk = np.asarray(varlen_lengths_k if varlen_lengths_k is not None else lq, dtype=np.int64)
        assert lq.shape == (batch,) and lk.shape == (batch,)
        cu_q = np.concatenate([[0], np.cumsum(lq)]).astype(np.int32)
        cu_k = np.concatenate([[0], np.cumsum(lk)]).astype(np.int32)
        out.update(cu_seqlens_q=cu_q, cu_seqlens_k=cu_k, lengths_q=lq, lengths_k=lk)
        shape_q = (int(cu_q[-1]), heads_q, head_dim)
        shape_k = (int(cu_k[-1]), heads_kv, head_dim)
    else:
        shape_q = (batch, seqlen_q, heads_q, head_dim)
        shape_k = (batch, seqlen_k, heads_kv, head_dim)

    def draw(shape):
        if dist == "normal":
            return rng.standard_normal(shape, dtype=np.float32)
        if dist == "uniform":
            return rng.uniform(-1.0, 1.0, size=shape).astype(np.float32)
        raise ValueError(dist)

    raw = {"q": draw(shape_q), "k": draw(shape_k), "v": draw(shape_k), "do": draw(shape_q)}
    if do_scale != 1.0:
        raw["do"] = raw["do"] * np.float32(do_scale)
    for name, x in raw.items():
        bits, val = _round(x, dtype)
        out[name] = val
        out[name + "_bits"] = bits
    return out


def make_workload_inputs(name: str, seed: Optional[int] = None):
    w = ALL_WORKLOADS[name]
    return make_inputs(
        w.dtype, w.batch, w.heads_q, w.heads_kv, w.seqlen, w.seqlen, w.head_dim,
        w.seed if seed is None else seed, do_scale=w.do_scale, varlen_range=w.varlen_range,
    )


def attention_flops(batch, heads_q, seqlen_q, seqlen_k, head_dim, causal, lengths=None):
    """Backward work count: 10*b*h*Sq*Sk*d, halved when causal.

    Varlen sums 10*h*L_i^2*d (halved when causal) over the sequences.  Padded
    head-dim columns and masked tile halves are not counted.
    """
    if lengths is not None:
        tot = sum(10.0 * heads_q * float(L) * float(L) * head_dim for L in lengths)
    else:
        tot = 10.0 * batch * heads_q * seqlen_q * seqlen_k * head_dim
    return tot * (0.5 if causal else 1.0)
