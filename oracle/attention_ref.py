"""Plain, slow, fp64 CPU reference for attention forward and backward.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module.  The GPU library
never calls it, and this module shares no code with it.

What is computed, and where the pages state it
----------------------------------------------
Forward -- tilelang ``test_tilelang_kernel_mha_bwd.py``, ``ref_program``:
scores ``S = Q K^T / sqrt(d)`` (einsum over the head dim, divided by the
square root of the head dim), causal positions set to ``-inf``, a softmax over
the keys, then ``O = P V``.  The softmax scale is a parameter here (the
flash-attention CK ``mha_bwd.cpp`` page passes ``softmax_scale`` explicitly);
the tests pass ``1/sqrt(d)``.

The log-sum-exp the forward hands to the backward is returned in natural-log
units, as the CK ``mha_bwd.cpp`` page's ``softmax_lse`` argument and the
Hopper ``flash_bwd_launch_template.h`` page's ``softmax_lse_ptr`` (with a
separate log2 copy) take it.  The tilelang page stores a log2-domain value
instead; the two differ by the factor log2(e).

Backward -- the exact gradient of the forward.  Its steps, as the tilelang
page's ``flashattn_bwd`` kernel lays them out per tile (here evaluated densely,
one head at a time):
  P  = exp(S - LSE)              recomputed from the saved LSE
  dP = dO V^T
  Delta_i = sum_j P_ij dP_ij     (equals rowsum(dO o O), the preprocess
                                  ``flashattn_bwd_preprocess``)
  dS = P o (dP - Delta)
  dV = P^T dO
  dK = scale * dS^T Q
  dQ = scale * dS K
The scale is applied to dK and dQ (the Hopper launch template's postprocess
multiplies dQ by ``scale_softmax``; the tilelang kernel multiplies dS by
``sm_scale`` first -- the same product).

GQA / MQA -- the CK page reshapes the per-query-head dK/dV to
``[b, s_k, h_k, h/h_k, d]`` and sums over the group axis, so query head ``h``
reads KV head ``h // (h/h_k)``.

Varlen -- packed ``[total, h, d]`` tensors with ``cu_seqlens`` prefix sums
(CuTe-DSL ``flash_bwd_postprocess.py`` ``__call__``: ``num_batch =
len(cu_seqlens) - 1``); every sequence is an independent attention problem.
LSE and Delta are ``[h, total_q]``.

Readings where the pages are silent:
  * causal alignment when Sq != Sk is bottom-right: key j is visible to
    query i iff ``j <= i + (Sk - Sq)`` (identical to the tilelang page's
    ``q >= k`` when Sq == Sk);
  * a query row that sees no key has O = 0, LSE = +inf and a zero P row.
"""
from __future__ import annotations

import math

import numpy as np

LOG2E = math.log2(math.e)

__all__ = [
    "LOG2E",
    "visible_mask",
    "head_forward",
    "head_backward",
    "attention_forward",
    "attention_backward",
    "delta_from_output",
    "kv_head_of",
]


def kv_head_of(h: int, heads_q: int, heads_kv: int) -> int:
    """KV head read by query head h (CK ``mha_bwd.cpp``: reshape to
    ``[b, s_k, h_k, h/h_k, d]``, i.e. contiguous groups)."""
    if heads_q % heads_kv:
        raise ValueError("heads_q must be a multiple of heads_kv")
    return h // (heads_q // heads_kv)


def visible_mask(sq: int, sk: int, causal: bool, window=(-1, -1)) -> np.ndarray:
    """Boolean [sq, sk]: True where key j contributes to query i.

    Causal follows the tilelang page (``tril``, i.e. keep j <= i) aligned to
    the bottom-right corner when the lengths differ.  ``window = (left,
    right)`` is the local (sliding-window) mask of the CK ``mha_bwd.cpp``
    page's ``window_size_left`` / ``window_size_right``, also bottom-right
    aligned (its ``"b:left,right"`` mask): key j is visible to query i iff
    ``i + (Sk - Sq) - left <= j <= i + (Sk - Sq) + right``, a negative size
    meaning no bound on that side; causal sets ``right = 0`` as that page
    does.
    """
    left, right = window
    if causal:
        right = 0
    i = np.arange(sq)[:, None]
    j = np.arange(sk)[None, :]
    diag = i + (sk - sq)
    vis = np.ones((sq, sk), dtype=bool)
    if right >= 0:
        vis &= j <= diag + right
    if left >= 0:
        vis &= j >= diag - left
    return vis


def head_forward(qh, kh, vh, scale: float, causal: bool, window=(-1, -1)):
    """One (sequence, query head): qh [Sq,d], kh/vh [Sk,d] -> (O [Sq,d], LSE [Sq]).

    tilelang ``ref_program``: scores, mask to -inf, softmax, times V.
    """
    qh = np.asarray(qh, dtype=np.float64)
    kh = np.asarray(kh, dtype=np.float64)
    vh = np.asarray(vh, dtype=np.float64)
    sq, sk = qh.shape[0], kh.shape[0]
    s = scale * (qh @ kh.T)
    s = np.where(visible_mask(sq, sk, causal, window), s, -np.inf)
    if sk == 0:
        m = np.full(sq, -np.inf)
    else:
        m = s.max(axis=1)
    m_ref = np.where(np.isfinite(m), m, 0.0)  # rows with no visible key
    e = np.exp(s - m_ref[:, None])
    l = e.sum(axis=1)
    with np.errstate(divide="ignore"):
        lse = np.where(l > 0.0, m_ref + np.log(np.where(l > 0.0, l, 1.0)), np.inf)
    p = np.exp(s - lse[:, None])  # softmax rows; exactly 0 for a row with LSE=+inf
    o = p @ vh
    return o, lse


def head_backward(qh, kh, vh, doh, scale: float, causal: bool, lse=None, window=(-1, -1)):
    """Gradient of sum(O o dO) for one (sequence, query head).

    Returns (dQ [Sq,d], dK [Sk,d], dV [Sk,d], Delta [Sq]).  If ``lse`` is
    given, P is recomputed from it (the saved-statistics form); otherwise the
    forward's own LSE is used.
    """
    qh = np.asarray(qh, dtype=np.float64)
    kh = np.asarray(kh, dtype=np.float64)
    vh = np.asarray(vh, dtype=np.float64)
    doh = np.asarray(doh, dtype=np.float64)
    sq, sk = qh.shape[0], kh.shape[0]
    if lse is None:
        _, lse = head_forward(qh, kh, vh, scale, causal, window)
    lse = np.asarray(lse, dtype=np.float64)
    s = scale * (qh @ kh.T)
    s = np.where(visible_mask(sq, sk, causal, window), s, -np.inf)
    p = np.exp(s - lse[:, None])
    dp = doh @ vh.T
    delta = (p * dp).sum(axis=1)
    ds = p * (dp - delta[:, None])
    dq = scale * (ds @ kh)
    dk = scale * (ds.T @ qh)
    dv = p.T @ doh
    return dq, dk, dv, delta


def _sequences(q, k, cu_seqlens_q, cu_seqlens_k):
    """Yield (z, q_slice_fn, k_slice_fn) over batch entries or packed sequences."""
    if cu_seqlens_q is None:
        for z in range(q.shape[0]):
            yield z, (lambda x, z=z: x[z]), (lambda x, z=z: x[z])
    else:
        cq = np.asarray(cu_seqlens_q, dtype=np.int64)
        ck = np.asarray(cu_seqlens_k, dtype=np.int64)
        for z in range(len(cq) - 1):
            yield z, (lambda x, a=cq[z], b=cq[z + 1]: x[a:b]), (lambda x, a=ck[z], b=ck[z + 1]: x[a:b])


def attention_forward(q, k, v, scale: float, causal: bool, cu_seqlens_q=None, cu_seqlens_k=None,
                      heads=None, window=(-1, -1)):
    """Full forward.

    Fixed length: q [b,Sq,H,d], k/v [b,Sk,Hk,d] -> O [b,Sq,H,d], LSE [b,H,Sq].
    Varlen: q [Tq,H,d], k/v [Tk,Hk,d] -> O [Tq,H,d], LSE [H,Tq].
    ``heads`` optionally restricts the query heads evaluated (others left 0).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    H, Hk = q.shape[-2], k.shape[-2]
    o = np.zeros(q.shape, dtype=np.float64)
    varlen = cu_seqlens_q is not None
    if varlen:
        lse = np.zeros((H, q.shape[0]), dtype=np.float64)
    else:
        lse = np.zeros((q.shape[0], H, q.shape[1]), dtype=np.float64)
    hs = range(H) if heads is None else heads
    for z, selq, selk in _sequences(q, k, cu_seqlens_q, cu_seqlens_k):
        qz, kz, vz = selq(q), selk(k), selk(v)
        oz = selq(o)
        for h in hs:
            g = kv_head_of(h, H, Hk)
            oh, lh = head_forward(qz[:, h, :], kz[:, g, :], vz[:, g, :], scale, causal, window)
            oz[:, h, :] = oh
            if varlen:
                a = int(np.asarray(cu_seqlens_q)[z])
                lse[h, a:a + oh.shape[0]] = lh
            else:
                lse[z, h, :] = lh
    return o, lse


def attention_backward(q, k, v, do, scale: float, causal: bool, cu_seqlens_q=None,
                       cu_seqlens_k=None, lse=None, heads=None, window=(-1, -1)):
    """Full backward: returns (dQ, dK, dV, Delta) in the layouts of the inputs.

    dK/dV of a KV head are summed over the query heads of its group (CK
    ``mha_bwd.cpp``, GQA ``sum_out``).  ``lse`` (natural log, [b,H,Sq] or
    [H,Tq]) is optional; without it the forward statistics are recomputed.
    ``heads`` restricts the query heads evaluated (dK/dV then hold only those
    heads' contributions).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    H, Hk = q.shape[-2], k.shape[-2]
    varlen = cu_seqlens_q is not None
    dq = np.zeros(q.shape, dtype=np.float64)
    dk = np.zeros(k.shape, dtype=np.float64)
    dv = np.zeros(v.shape, dtype=np.float64)
    if varlen:
        delta = np.zeros((H, q.shape[0]), dtype=np.float64)
    else:
        delta = np.zeros((q.shape[0], H, q.shape[1]), dtype=np.float64)
    hs = range(H) if heads is None else heads
    for z, selq, selk in _sequences(q, k, cu_seqlens_q, cu_seqlens_k):
        qz, kz, vz, doz = selq(q), selk(k), selk(v), selq(do)
        dqz, dkz, dvz = selq(dq), selk(dk), selk(dv)
        for h in hs:
            g = kv_head_of(h, H, Hk)
            if lse is None:
                lh = None
            elif varlen:
                a = int(np.asarray(cu_seqlens_q)[z])
                lh = np.asarray(lse)[h, a:a + qz.shape[0]]
            else:
                lh = np.asarray(lse)[z, h, :]
            dqh, dkh, dvh, dh = head_backward(qz[:, h, :], kz[:, g, :], vz[:, g, :], doz[:, h, :],
                                              scale, causal, lse=lh, window=window)
            dqz[:, h, :] = dqh
            dkz[:, g, :] += dkh
            dvz[:, g, :] += dvh
            if varlen:
                a = int(np.asarray(cu_seqlens_q)[z])
                delta[h, a:a + qz.shape[0]] = dh
            else:
                delta[z, h, :] = dh
    return dq, dk, dv, delta


def delta_from_output(o, do, varlen: bool = False):
    """Backward preprocess (tilelang ``flashattn_bwd_preprocess``):
    Delta = sum over the head dim of O * dO, laid out [b,H,S] (varlen [H,T])."""
    o = np.asarray(o, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    r = (o * do).sum(axis=-1)  # [b,S,H] or [T,H]
    if varlen:
        return r.T.copy()
    return np.transpose(r, (0, 2, 1)).copy()
