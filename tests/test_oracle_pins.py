"""Pins for the fp64 CPU oracle: it is checked against things other than itself.

* hand-derived worked examples (tests/golden/hand_examples.json);
* brute force on tiny inputs with pure-Python loops and no max shift;
* central finite differences of sum(O * dO) for every element of Q, K, V;
* closed forms (uniform keys, a single key, a single query);
* invariants (sum over keys of dK is 0, sum over keys of dV is the sum of dO,
  Delta = rowsum(dO * O), rows of dS sum to 0);
* causal zero patterns;
* special cases that reduce to a library routine (torch float64 SDPA on CPU);
* GQA = MHA with repeated KV heads then group-summed; varlen = per-sequence.
A mutation test at the end plants plausible mistakes in the oracle and checks
that the pins catch each one.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle
from oracle import attention_ref as ref

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_examples.json")


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _case(b, h, hk, sq, sk, d, seed=0):
    q = _rand((b, sq, h, d), seed)
    k = _rand((b, sk, hk, d), seed + 1)
    v = _rand((b, sk, hk, d), seed + 2)
    do = _rand((b, sq, h, d), seed + 3)
    return q, k, v, do


def _varlen_case(lengths_q, lengths_k, h, hk, d, seed=0):
    cq = np.concatenate([[0], np.cumsum(lengths_q)]).astype(np.int32)
    ck = np.concatenate([[0], np.cumsum(lengths_k)]).astype(np.int32)
    q = _rand((cq[-1], h, d), seed)
    k = _rand((ck[-1], hk, d), seed + 1)
    v = _rand((ck[-1], hk, d), seed + 2)
    do = _rand((cq[-1], h, d), seed + 3)
    return q, k, v, do, cq, ck


# ----------------------------------------------------------------------------
# worked examples
# ----------------------------------------------------------------------------
def _parse(x):
    if isinstance(x, list):
        return [_parse(y) for y in x]
    if isinstance(x, str):
        return float(eval(x, {"__builtins__": {}},
                          {"LN2": math.log(2.0), "LN3": math.log(3.0), "LN4": math.log(4.0),
                           "LN5": math.log(5.0)}))
    return float(x)


def _golden():
    with open(GOLDEN) as f:
        return json.load(f)["examples"]


@pytest.mark.parametrize("ex", _golden(), ids=lambda e: e["name"])
def test_hand_worked_examples(ex):
    g = {k: np.array(_parse(ex[k])) for k in ("q", "k", "v", "do", "o", "lse", "dq", "dk", "dv", "delta")}
    o, lse = oracle.attention_forward(g["q"], g["k"], g["v"], ex["scale"], ex["causal"])
    dq, dk, dv, delta = oracle.attention_backward(g["q"], g["k"], g["v"], g["do"], ex["scale"], ex["causal"])
    for name, got in (("o", o), ("lse", lse), ("dq", dq), ("dk", dk), ("dv", dv), ("delta", delta)):
        np.testing.assert_allclose(got, g[name], rtol=1e-13, atol=1e-13, err_msg=name)


# ----------------------------------------------------------------------------
# brute force forward with pure-Python loops (no max shift, direct exp sums)
# ----------------------------------------------------------------------------
def _brute_forward(q, k, v, scale, causal, window=(-1, -1)):
    b, sq, h, d = q.shape
    wl, wr = window
    sk, hk = k.shape[1], k.shape[2]
    o = np.zeros_like(q)
    lse = np.zeros((b, h, sq))
    grp = h // hk
    for z in range(b):
        for hh in range(h):
            g = hh // grp
            for i in range(sq):
                ws = []
                for j in range(sk):
                    if causal and j > i + (sk - sq):
                        continue
                    if wr >= 0 and j > i + (sk - sq) + wr:
                        continue
                    if wl >= 0 and j < i + (sk - sq) - wl:
                        continue
                    s = 0.0
                    for t in range(d):
                        s += q[z, i, hh, t] * k[z, j, g, t]
                    ws.append((math.exp(scale * s), j))
                tot = sum(w for w, _ in ws)
                if tot == 0.0:
                    lse[z, hh, i] = math.inf
                    continue
                lse[z, hh, i] = math.log(tot)
                for t in range(d):
                    o[z, i, hh, t] = sum(w * v[z, j, g, t] for w, j in ws) / tot
    return o, lse


BRUTE_CASES = [
    # b, h, hk, sq, sk, d, causal
    (2, 2, 2, 5, 5, 4, False),
    (1, 4, 2, 6, 6, 3, True),
    (1, 2, 1, 3, 7, 4, True),   # Sq < Sk: bottom-right alignment
    (1, 1, 1, 7, 4, 2, True),   # Sq > Sk: first rows see no key
    (1, 2, 2, 1, 9, 5, False),
]


@pytest.mark.parametrize("b,h,hk,sq,sk,d,causal", BRUTE_CASES)
def test_forward_matches_brute_force(b, h, hk, sq, sk, d, causal):
    q, k, v, _ = _case(b, h, hk, sq, sk, d, seed=11)
    scale = 1.0 / math.sqrt(d)
    o, lse = oracle.attention_forward(q, k, v, scale, causal)
    ob, lb = _brute_forward(q, k, v, scale, causal)
    np.testing.assert_allclose(o, ob, rtol=1e-12, atol=1e-12)
    np.testing.assert_array_equal(np.isinf(lse), np.isinf(lb))
    fin = np.isfinite(lb)
    np.testing.assert_allclose(lse[fin], lb[fin], rtol=1e-12, atol=1e-12)


# ----------------------------------------------------------------------------
# central finite differences of L = sum(O * dO)
# ----------------------------------------------------------------------------
def fd_max_rel_error(b, h, hk, sq, sk, d, causal, seed=0, varlen=None, eps=1e-6, window=(-1, -1)):
    """Max |numeric - analytic| / max|analytic| over every element of Q, K, V."""
    if varlen is None:
        q, k, v, do = _case(b, h, hk, sq, sk, d, seed)
        cq = ck = None
    else:
        q, k, v, do, cq, ck = _varlen_case(varlen[0], varlen[1], h, hk, d, seed)
    scale = 1.0 / math.sqrt(d)

    def loss(q_, k_, v_):
        o, _ = oracle.attention_forward(q_, k_, v_, scale, causal, cq, ck, window=window)
        return float((o * do).sum())

    dq, dk, dv, _ = oracle.attention_backward(q, k, v, do, scale, causal, cq, ck, window=window)
    worst = 0.0
    for which, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        num = np.zeros_like(x)
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            xp = x.copy()
            xp[idx] += eps
            xm = x.copy()
            xm[idx] -= eps
            args_p = {"q": q, "k": k, "v": v}
            args_m = {"q": q, "k": k, "v": v}
            args_p[which] = xp
            args_m[which] = xm
            num[idx] = (loss(args_p["q"], args_p["k"], args_p["v"])
                        - loss(args_m["q"], args_m["k"], args_m["v"])) / (2 * eps)
        scale_ref = max(np.abs(g).max(), 1e-3)
        worst = max(worst, np.abs(num - g).max() / scale_ref)
    return worst


FD_CASES = [
    # b, h, hk, sq, sk, d, causal, varlen
    (2, 2, 2, 3, 3, 4, False, None),
    (1, 4, 2, 7, 7, 4, True, None),
    (1, 2, 1, 3, 7, 8, True, None),     # Sq < Sk
    (1, 1, 1, 7, 3, 4, True, None),     # Sq > Sk: rows without keys
    (1, 1, 1, 16, 16, 4, False, None),
    (1, 2, 1, 1, 1, 4, True, None),     # S = 1
    (3, 2, 1, 0, 0, 4, True, ([1, 5, 9], [1, 5, 9])),
    (3, 2, 2, 0, 0, 4, False, ([1, 5, 9], [2, 5, 3])),
]


@pytest.mark.parametrize("b,h,hk,sq,sk,d,causal,varlen", FD_CASES)
def test_backward_matches_finite_differences(b, h, hk, sq, sk, d, causal, varlen):
    assert fd_max_rel_error(b, h, hk, sq, sk, d, causal, seed=5, varlen=varlen) < 1e-7


# ----------------------------------------------------------------------------
# closed forms
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("causal", [False, True])
def test_uniform_keys_closed_form(causal):
    rng = np.random.default_rng(3)
    b, s, h, d = 1, 9, 2, 4
    q = rng.standard_normal((b, s, h, d))
    k = np.broadcast_to(rng.standard_normal((1, 1, h, d)), (b, s, h, d)).copy()
    v = rng.standard_normal((b, s, h, d))
    scale = 0.3
    o, lse = oracle.attention_forward(q, k, v, scale, causal)
    for hh in range(h):
        for i in range(s):
            n = i + 1 if causal else s
            sc = scale * float(q[0, i, hh] @ k[0, 0, hh])
            np.testing.assert_allclose(o[0, i, hh], v[0, :n, hh].mean(axis=0), rtol=1e-12, atol=1e-12)
            np.testing.assert_allclose(lse[0, hh, i], sc + math.log(n), rtol=1e-12, atol=1e-12)
    # equal keys: every row of dS sums to 0, so dQ = scale * (sum_j dS_ij) k = 0
    do = rng.standard_normal(q.shape)
    dq, dk, dv, _ = oracle.attention_backward(q, k, v, do, scale, causal)
    assert np.abs(dq).max() < 1e-12


def test_single_key():
    q, k, v, do = _case(2, 2, 1, 5, 1, 4, seed=9)
    o, lse = oracle.attention_forward(q, k, v, 0.5, False)
    np.testing.assert_allclose(o, np.broadcast_to(v, o.shape), rtol=1e-14)
    s = 0.5 * np.einsum("bqhd,bkd->bhq", q, k[:, :, 0, :])
    np.testing.assert_allclose(lse, s, rtol=1e-13, atol=1e-13)


def test_single_query_single_key_gradients():
    q, k, v, do = _case(2, 3, 3, 1, 1, 8, seed=4)
    dq, dk, dv, _ = oracle.attention_backward(q, k, v, do, 0.25, True)
    assert np.abs(dq).max() == 0.0 and np.abs(dk).max() == 0.0
    np.testing.assert_allclose(dv, do, rtol=0, atol=0)


# ----------------------------------------------------------------------------
# invariants
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("h,hk", [(2, 2), (4, 1), (6, 2)])
def test_invariants(causal, h, hk):
    b, s, d = 2, 13, 8
    q, k, v, do = _case(b, h, hk, s, s, d, seed=21)
    scale = d ** -0.5
    o, lse = oracle.attention_forward(q, k, v, scale, causal)
    dq, dk, dv, delta = oracle.attention_backward(q, k, v, do, scale, causal)
    # shifting every key by a constant shifts each score row by a constant
    assert np.abs(dk.sum(axis=1)).max() < 1e-12 * max(1.0, np.abs(dk).max()) * s
    # sum over keys of dV = sum over the group's query heads and queries of dO
    g = h // hk
    dosum = do.sum(axis=1).reshape(b, hk, g, d).sum(axis=2)
    np.testing.assert_allclose(dv.sum(axis=1), dosum, rtol=1e-12, atol=1e-12)
    # Delta = rowsum(P * dP) equals rowsum(dO * O)
    np.testing.assert_allclose(delta, oracle.delta_from_output(o, do), rtol=1e-12, atol=1e-12)
    # the saved-statistics form gives the same gradient
    dq2, dk2, dv2, _ = oracle.attention_backward(q, k, v, do, scale, causal, lse=lse)
    np.testing.assert_allclose(dq2, dq, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(dk2, dk, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(dv2, dv, rtol=1e-12, atol=1e-12)


def test_rows_of_ds_sum_to_zero():
    rng = np.random.default_rng(8)
    sq, sk, d = 11, 11, 4
    qh, kh, vh, doh = (rng.standard_normal((n, d)) for n in (sq, sk, sk, sq))
    _, lse = ref.head_forward(qh, kh, vh, 0.5, True)
    s = 0.5 * qh @ kh.T
    p = np.where(ref.visible_mask(sq, sk, True), np.exp(s - lse[:, None]), 0.0)
    dp = doh @ vh.T
    delta = (p * dp).sum(1)
    ds = p * (dp - delta[:, None])
    assert np.abs(ds.sum(1)).max() < 1e-13
    # and the oracle's dQ equals 0.5 * dS K built here from the same definition
    dq, _, _, _ = ref.head_backward(qh, kh, vh, doh, 0.5, True)
    np.testing.assert_allclose(dq, 0.5 * ds @ kh, rtol=1e-12, atol=1e-12)


# ----------------------------------------------------------------------------
# causal zero patterns
# ----------------------------------------------------------------------------
def test_causal_zero_patterns():
    b, s, h, d = 1, 10, 2, 4
    q, k, v, do = _case(b, h, h, s, s, d, seed=31)
    scale = 0.5
    dq, dk, dv, _ = oracle.attention_backward(q, k, v, do, scale, True)
    assert np.abs(dq[:, 0]).max() == 0.0  # row 0 sees only key 0: P00 = 1, dS00 = 0
    i0 = 4
    do1 = np.zeros_like(do)
    do1[:, i0] = do[:, i0]
    _, dk1, dv1, _ = oracle.attention_backward(q, k, v, do1, scale, True)
    assert np.abs(dk1[:, i0 + 1:]).max() == 0.0
    assert np.abs(dv1[:, i0 + 1:]).max() == 0.0
    # perturbing keys/values after row i leaves O_i unchanged
    o, _ = oracle.attention_forward(q, k, v, scale, True)
    k2, v2 = k.copy(), v.copy()
    k2[:, i0 + 1:] += 3.0
    v2[:, i0 + 1:] -= 2.0
    o2, _ = oracle.attention_forward(q, k2, v2, scale, True)
    np.testing.assert_array_equal(o2[:, : i0 + 1], o[:, : i0 + 1])


# ----------------------------------------------------------------------------
# library routine: torch float64 scaled_dot_product_attention on the CPU
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("h,hk,sq,sk", [(4, 4, 33, 33), (4, 2, 20, 20), (2, 1, 9, 17)])
def test_matches_torch_sdpa_float64(causal, h, hk, sq, sk):
    torch = pytest.importorskip("torch")
    b, d = 2, 16
    q, k, v, do = _case(b, h, hk, sq, sk, d, seed=41)
    scale = d ** -0.5
    o, lse = oracle.attention_forward(q, k, v, scale, causal)
    dq, dk, dv, _ = oracle.attention_backward(q, k, v, do, scale, causal)
    tq, tk, tv = (torch.tensor(x.transpose(0, 2, 1, 3), dtype=torch.float64, requires_grad=True)
                  for x in (q, k, v))
    g = h // hk
    tk_r = tk.repeat_interleave(g, dim=1)
    tv_r = tv.repeat_interleave(g, dim=1)
    mask = None
    if causal:
        mask = torch.tensor(ref.visible_mask(sq, sk, True))
    to = torch.nn.functional.scaled_dot_product_attention(tq, tk_r, tv_r, attn_mask=mask, scale=scale)
    to.backward(torch.tensor(do.transpose(0, 2, 1, 3)))
    np.testing.assert_allclose(o, to.detach().numpy().transpose(0, 2, 1, 3), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(dq, tq.grad.numpy().transpose(0, 2, 1, 3), rtol=1e-10, atol=1e-11)
    np.testing.assert_allclose(dk, tk.grad.numpy().transpose(0, 2, 1, 3), rtol=1e-10, atol=1e-11)
    np.testing.assert_allclose(dv, tv.grad.numpy().transpose(0, 2, 1, 3), rtol=1e-10, atol=1e-11)
    # LSE against a library log-sum-exp of the masked scores
    s = scale * torch.einsum("bhqd,bhkd->bhqk", tq.detach(), tk_r.detach())
    if causal:
        s = s.masked_fill(~mask, float("-inf"))
    np.testing.assert_allclose(lse, torch.logsumexp(s, dim=-1).numpy(), rtol=1e-12, atol=1e-12)


# ----------------------------------------------------------------------------
# GQA and varlen structure
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("causal", [False, True])
def test_gqa_equals_repeated_mha(causal):
    b, s, h, hk, d = 2, 12, 8, 2, 4
    q, k, v, do = _case(b, h, hk, s, s, d, seed=51)
    g = h // hk
    kr, vr = np.repeat(k, g, axis=2), np.repeat(v, g, axis=2)
    o, lse = oracle.attention_forward(q, k, v, 0.5, causal)
    o2, lse2 = oracle.attention_forward(q, kr, vr, 0.5, causal)
    np.testing.assert_allclose(o, o2, rtol=1e-13, atol=1e-13)
    dq, dk, dv, _ = oracle.attention_backward(q, k, v, do, 0.5, causal)
    dq2, dk2, dv2, _ = oracle.attention_backward(q, kr, vr, do, 0.5, causal)
    np.testing.assert_allclose(dq, dq2, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(dk, dk2.reshape(b, s, hk, g, d).sum(3), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(dv, dv2.reshape(b, s, hk, g, d).sum(3), rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_varlen_equals_per_sequence(causal):
    lq, lk = [3, 1, 8, 5], [3, 4, 8, 2]
    h, hk, d = 4, 2, 4
    q, k, v, do, cq, ck = _varlen_case(lq, lk, h, hk, d, seed=61)
    o, lse = oracle.attention_forward(q, k, v, 0.5, causal, cq, ck)
    dq, dk, dv, delta = oracle.attention_backward(q, k, v, do, 0.5, causal, cq, ck)
    for z in range(len(lq)):
        a, e = cq[z], cq[z + 1]
        ka, ke = ck[z], ck[z + 1]
        oz, lz = oracle.attention_forward(q[None, a:e], k[None, ka:ke], v[None, ka:ke], 0.5, causal)
        np.testing.assert_allclose(o[a:e], oz[0], rtol=1e-13, atol=1e-13)
        np.testing.assert_allclose(lse[:, a:e], lz[0], rtol=1e-13, atol=1e-13)
        dqz, dkz, dvz, dz = oracle.attention_backward(q[None, a:e], k[None, ka:ke], v[None, ka:ke],
                                                      do[None, a:e], 0.5, causal)
        np.testing.assert_allclose(dq[a:e], dqz[0], rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(dk[ka:ke], dkz[0], rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(dv[ka:ke], dvz[0], rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(delta[:, a:e], dz[0], rtol=1e-12, atol=1e-12)


def test_delta_layout_varlen():
    q, k, v, do, cq, ck = _varlen_case([2, 3], [2, 3], 2, 2, 4, seed=71)
    o, _ = oracle.attention_forward(q, k, v, 0.5, True, cq, ck)
    _, _, _, delta = oracle.attention_backward(q, k, v, do, 0.5, True, cq, ck)
    np.testing.assert_allclose(delta, oracle.delta_from_output(o, do, varlen=True), rtol=1e-12, atol=1e-12)


# ----------------------------------------------------------------------------
# mutation test: plausible mistakes planted in the oracle must fail a pin
# ----------------------------------------------------------------------------
def _mutant_backward(kind):
    def hb(qh, kh, vh, doh, scale, causal, lse=None, window=(-1, -1)):
        sq, sk = qh.shape[0], kh.shape[0]
        if lse is None:
            _, lse = ref.head_forward(qh, kh, vh, scale, causal, window)
        s = scale * (qh @ kh.T)
        s = np.where(ref.visible_mask(sq, sk, causal, window), s, -np.inf)
        p = np.exp(s - lse[:, None])
        dp = doh @ vh.T
        delta = (p * dp).sum(axis=1)
        if kind == "drop_delta":
            ds = p * dp
        elif kind == "sign":
            ds = p * (delta[:, None] - dp)
        else:
            ds = p * (dp - delta[:, None])
        dq = scale * (ds @ kh)
        dk = scale * (ds.T @ qh)
        dv = p.T @ doh
        if kind == "dk_unscaled":
            dk = ds.T @ qh
        if kind == "dv_transposed":
            dv = p @ doh
        if kind == "dq_with_q":
            dq = scale * (ds @ qh)
        return dq, dk, dv, delta
    return hb


@pytest.mark.parametrize("kind", ["drop_delta", "sign", "dk_unscaled", "dv_transposed", "dq_with_q"])
def test_pins_catch_planted_backward_mistakes(kind, monkeypatch):
    monkeypatch.setattr(ref, "head_backward", _mutant_backward(kind))
    assert fd_max_rel_error(1, 2, 2, 5, 5, 4, True, seed=5) > 1e-3


def test_pins_catch_planted_gqa_mapping_mistake(monkeypatch):
    monkeypatch.setattr(ref, "kv_head_of", lambda h, H, Hk: h % Hk)
    with pytest.raises(AssertionError):
        test_gqa_equals_repeated_mha(False)


def test_pins_catch_planted_mask_off_by_one(monkeypatch):
    def bad_mask(sq, sk, causal, window=(-1, -1)):
        if not causal:
            return np.ones((sq, sk), dtype=bool)
        i = np.arange(sq)[:, None]
        j = np.arange(sk)[None, :]
        return j < i + (sk - sq) + 2
    monkeypatch.setattr(ref, "visible_mask", bad_mask)
    with pytest.raises(AssertionError):
        test_forward_matches_brute_force(1, 4, 2, 6, 6, 3, True)


# ----------------------------------------------------------------------------
# local (sliding-window) mask: the CK mha_bwd.cpp page's window_size_left /
# window_size_right, bottom-right aligned
# ----------------------------------------------------------------------------
WINDOW_CASES = [
    # b, h, hk, sq, sk, d, causal, (left, right)
    (1, 2, 2, 9, 9, 4, False, (2, 1)),
    (1, 2, 1, 7, 7, 3, True, (3, -1)),    # causal + left window
    (2, 1, 1, 5, 9, 4, False, (1, 3)),    # Sq < Sk
    (1, 2, 2, 9, 4, 2, False, (0, 2)),    # Sq > Sk: some rows see no key
    (1, 1, 1, 6, 6, 4, False, (-1, 0)),   # = causal
    (1, 1, 1, 6, 6, 4, False, (0, -1)),
]


@pytest.mark.parametrize("b,h,hk,sq,sk,d,causal,window", WINDOW_CASES)
def test_window_forward_matches_brute_force(b, h, hk, sq, sk, d, causal, window):
    q, k, v, _ = _case(b, h, hk, sq, sk, d, seed=13)
    scale = 1.0 / math.sqrt(d)
    o, lse = oracle.attention_forward(q, k, v, scale, causal, window=window)
    ob, lb = _brute_forward(q, k, v, scale, causal, window)
    np.testing.assert_allclose(o, ob, rtol=1e-12, atol=1e-12)
    np.testing.assert_array_equal(np.isinf(lse), np.isinf(lb))
    fin = np.isfinite(lb)
    np.testing.assert_allclose(lse[fin], lb[fin], rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("b,h,hk,sq,sk,d,causal,window", WINDOW_CASES[:4])
def test_window_backward_matches_finite_differences(b, h, hk, sq, sk, d, causal, window):
    assert fd_max_rel_error(b, h, hk, sq, sk, d, causal, seed=17, window=window) < 1e-7


def test_window_special_cases():
    b, s, h, d = 1, 8, 2, 4
    q, k, v, do = _case(b, h, h, s, s, d, seed=19)
    scale = 0.5
    # (0, 0): every query sees only its own key -> O = V, dQ = dK = 0, dV = dO
    o, lse = oracle.attention_forward(q, k, v, scale, False, window=(0, 0))
    dq, dk, dv, _ = oracle.attention_backward(q, k, v, do, scale, False, window=(0, 0))
    np.testing.assert_allclose(o, v, atol=1e-14)
    np.testing.assert_allclose(lse, scale * np.einsum("bshd,bshd->bhs", q, k), atol=1e-13)
    np.testing.assert_allclose(dq, 0.0, atol=1e-14)
    np.testing.assert_allclose(dk, 0.0, atol=1e-14)
    np.testing.assert_allclose(dv, do, atol=1e-14)
    # unbounded on both sides = no mask; (-1, 0) = causal; windows wider than
    # the sequence = no bound
    for causal, window, same in ((False, (-1, -1), (False, (-1, -1))), (False, (-1, 0), (True, (-1, -1))),
                                 (False, (s, s), (False, (-1, -1))), (True, (s, 3), (True, (-1, -1)))):
        a = oracle.attention_backward(q, k, v, do, scale, causal, window=window)
        r = oracle.attention_backward(q, k, v, do, scale, same[0], window=same[1])
        for x, y in zip(a, r):
            np.testing.assert_allclose(x, y, rtol=1e-13, atol=1e-13)


def test_window_matches_torch_sdpa_float64():
    torch = pytest.importorskip("torch")
    b, h, hk, sq, sk, d = 2, 4, 2, 11, 13, 8
    wl, wr = 3, 2
    q, k, v, do = _case(b, h, hk, sq, sk, d, seed=23)
    scale = d ** -0.5
    o, _ = oracle.attention_forward(q, k, v, scale, False, window=(wl, wr))
    dq, dk, dv, _ = oracle.attention_backward(q, k, v, do, scale, False, window=(wl, wr))
    # the mask written out entry by entry, independently of the oracle
    m = np.zeros((sq, sk), dtype=bool)
    for i in range(sq):
        for j in range(sk):
            m[i, j] = (i + sk - sq - wl) <= j <= (i + sk - sq + wr)
    tq, tk, tv = (torch.tensor(x.transpose(0, 2, 1, 3), dtype=torch.float64, requires_grad=True)
                  for x in (q, k, v))
    g = h // hk
    to = torch.nn.functional.scaled_dot_product_attention(
        tq, tk.repeat_interleave(g, dim=1), tv.repeat_interleave(g, dim=1), attn_mask=torch.tensor(m), scale=scale)
    to.backward(torch.tensor(do.transpose(0, 2, 1, 3)))
    np.testing.assert_allclose(o, to.detach().numpy().transpose(0, 2, 1, 3), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(dq, tq.grad.numpy().transpose(0, 2, 1, 3), rtol=1e-10, atol=1e-11)
    np.testing.assert_allclose(dk, tk.grad.numpy().transpose(0, 2, 1, 3), rtol=1e-10, atol=1e-11)
    np.testing.assert_allclose(dv, tv.grad.numpy().transpose(0, 2, 1, 3), rtol=1e-10, atol=1e-11)


def test_pins_catch_planted_window_off_by_one(monkeypatch):
    real = oracle.attention_ref.visible_mask

    def shifted(sq, sk, causal, window=(-1, -1)):
        wl, wr = window
        return real(sq, sk, causal, (wl + 1 if wl >= 0 else wl, wr))

    monkeypatch.setattr(oracle.attention_ref, "visible_mask", shifted)
    q, k, v, _ = _case(1, 2, 2, 9, 9, 4, seed=13)
    o, _ = oracle.attention_forward(q, k, v, 0.5, False, window=(2, 1))
    ob, _ = _brute_forward(q, k, v, 0.5, False, (2, 1))
    assert np.abs(o - ob).max() > 1e-3
