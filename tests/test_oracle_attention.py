"""Pins of the oracle's attention forward and straight-through backward.

Each pin comes from outside the oracle's own code:
* with P quantization off the forward is textbook attention, checked against
  torch's float64 CPU ``scaled_dot_product_attention`` and ``logsumexp``, and
  the backward against torch autograd of that library routine;
* closed forms: a zero Q gives uniform P (every P code is FMAX, lse = ln Nkv,
  O = O_hp = mean of V); one key gives O = O_hp = V; the first causal row sees
  only key 0;
* invariants: rows of P sum to 1, sum_j dK_j = 0 (which needs Delta from
  O_hp), Delta_i = sum_j P_ij dP_ij, causal rows ignore later keys;
* straight-through gradients equal central finite differences of the
  un-quantized high-precision attention at the quantized point (dQ, dK) and
  of the linear map V -> sum dO o (P^ V) (dV);
* the source's online form (running max, quantizing the un-normalised tile,
  rescaling both accumulators, l from the high-precision P) gives the same
  outputs as the plain definition the oracle uses;
* P-quant groups are 64 absolute key columns: changing keys of one group
  rescales the other group's quantized P exactly, but only with that group
  width.
"""
import math

import numpy as np
import pytest
import torch

from oracle import fp8
from oracle import qat_attention as qa


def _rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


def _sdpa(q, k, v, scale, causal):
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float64))
    return torch.nn.functional.scaled_dot_product_attention(
        t(q), t(k), t(v), is_causal=causal, scale=scale).numpy()


@pytest.mark.parametrize("Nq,Nkv,causal", [(16, 16, False), (37, 37, True), (20, 70, False), (5, 1, False)])
def test_quant_off_is_textbook_attention(Nq, Nkv, causal):
    D = 32
    q, k, v = _rand((2, 3, Nq, D), 1), _rand((2, 3, Nkv, D), 2), _rand((2, 3, Nkv, D), 3)
    sc = 1 / math.sqrt(D)
    O, O_hp, lse = qa.attention_forward(q, k, v, sc, causal=causal, p_quant=False)
    ref = _sdpa(q, k, v, sc, causal)
    assert np.allclose(O, ref, atol=1e-12) and np.allclose(O_hp, ref, atol=1e-12)
    S = torch.from_numpy(q) @ torch.from_numpy(k).transpose(-1, -2) * sc
    if causal:
        S = S.masked_fill(torch.ones(Nq, Nkv, dtype=torch.bool).triu(1), -math.inf)
    assert np.allclose(lse, torch.logsumexp(S, -1).numpy(), atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_quant_off_backward_is_autograd(causal):
    N, D = 24, 16
    q, k, v, do = (_rand((1, 2, N, D), s) for s in (4, 5, 6, 7))
    sc = 0.3
    dQ, dK, dV = qa.attention_backward(q, k, v, do, sc, causal=causal, p_quant=False)
    t = [torch.tensor(a, requires_grad=True) for a in (q, k, v)]
    out = torch.nn.functional.scaled_dot_product_attention(*t, is_causal=causal, scale=sc)
    out.backward(torch.from_numpy(do))
    for ours, ref in zip((dQ, dK, dV), t):
        assert np.allclose(ours, ref.grad.numpy(), atol=1e-11)


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_zero_q_closed_form(fmt):
    Nkv, D = 100, 8
    q = np.zeros((1, 1, 5, D))
    k, v = _rand((1, 1, Nkv, D), 8), _rand((1, 1, Nkv, D), 9)
    O, O_hp, lse = qa.attention_forward(q, k, v, 0.5, p_fmt=fmt)
    mean_v = v[0, 0].mean(axis=0)
    assert np.allclose(lse, math.log(Nkv), atol=1e-14)
    assert np.allclose(O_hp[0, 0], mean_v[None], atol=1e-14)
    # every P entry is its group's absmax, so P^ = P up to fp32 rounding
    assert np.allclose(O[0, 0], mean_v[None], rtol=0, atol=1e-6)


def test_single_key_closed_form():
    q, k, v = _rand((2, 2, 7, 16), 10), _rand((2, 2, 1, 16), 11), _rand((2, 2, 1, 16), 12)
    O, O_hp, lse = qa.attention_forward(q, k, v, 0.25)
    assert np.array_equal(O, np.broadcast_to(v, O.shape))      # P = 1, P^ = fp32(448*fp32(1/448)) = 1
    assert np.allclose(O_hp, np.broadcast_to(v, O.shape), atol=0)
    assert np.allclose(lse, 0.25 * np.einsum("bhnd,bhd->bhn", q, k[:, :, 0]), atol=1e-12)


def test_causal_first_row_and_future_independence():
    N, D = 40, 16
    q, k, v = _rand((1, 1, N, D), 13), _rand((1, 1, N, D), 14), _rand((1, 1, N, D), 15)
    O, O_hp, lse = qa.attention_forward(q, k, v, 0.25, causal=True)
    assert np.allclose(O[0, 0, 0], v[0, 0, 0]) and np.allclose(O_hp[0, 0, 0], v[0, 0, 0])
    assert np.isclose(lse[0, 0, 0], 0.25 * q[0, 0, 0] @ k[0, 0, 0])
    v2, k2 = v.copy(), k.copy()
    v2[0, 0, 25:] += 5.0
    k2[0, 0, 25:] -= 3.0
    O2, O_hp2, lse2 = qa.attention_forward(q, k2, v2, 0.25, causal=True)
    assert np.array_equal(O[0, 0, :25], O2[0, 0, :25]) and np.array_equal(lse[0, 0, :25], lse2[0, 0, :25])


def test_rows_sum_to_one_and_delta_identity():
    qh, kh, vh, do = _rand((30, 8), 16), _rand((50, 8), 17), _rand((50, 8), 18), _rand((30, 8), 19)
    S = qa._scores(qh, kh, 0.7, False, np.arange(30))
    P, lse = qa._softmax_rows(S)
    assert np.allclose(P.sum(axis=1), 1.0, atol=1e-14)
    O_hp = P @ vh
    Delta = np.sum(do * O_hp, axis=1)
    dP = do @ vh.T
    assert np.allclose(Delta, np.sum(P * dP, axis=1), atol=1e-12)


@pytest.mark.parametrize("causal,qkv", [(False, False), (True, False), (False, True)])
def test_dk_sums_to_zero(causal, qkv):
    N, D = 70, 16
    q, k, v, do = (_rand((1, 2, N, D), s) for s in (20, 21, 22, 23))
    dQ, dK, dV = qa.attention_backward(q, k, v, do, 0.25, causal=causal, qkv_quant=qkv)
    assert np.allclose(dK.sum(axis=2), 0.0, atol=1e-11)


def _fd(f, x, h=1e-6):
    g = np.zeros_like(x)
    it = np.nditer(x, flags=["multi_index"])
    for _ in it:
        i = it.multi_index
        xp, xm = x.copy(), x.copy()
        xp[i] += h
        xm[i] -= h
        g[i] = (f(xp) - f(xm)) / (2 * h)
    return g


@pytest.mark.parametrize("causal,qkv,fmt", [(False, False, "e4m3"), (True, False, "e4m3"),
                                            (False, True, "e4m3"), (False, False, "e5m2")])
def test_ste_gradients_equal_finite_differences(causal, qkv, fmt):
    N, Nkv, D = 6, 6 if causal else 9, 4
    q, k, v, do = _rand((1, 1, N, D), 24), _rand((1, 1, Nkv, D), 25), _rand((1, 1, Nkv, D), 26), _rand((1, 1, N, D), 27)
    sc = 0.6
    dQ, dK, dV = qa.attention_backward(q, k, v, do, sc, causal=causal, p_fmt=fmt, qkv_quant=qkv, group=4)
    qh, kh, vh = qa.prepare_inputs(q, k, v, qkv_quant=qkv)
    qh, kh, vh, dO = qh[0, 0], kh[0, 0], vh[0, 0], do[0, 0]

    def L_hp(Q, K, V):  # high-precision attention, torch library routine
        return float((_sdpa(Q[None], K[None], V[None], sc, causal)[0] * dO).sum())

    assert np.allclose(dQ[0, 0], _fd(lambda x: L_hp(x, kh, vh), qh), rtol=1e-6, atol=1e-7)
    assert np.allclose(dK[0, 0], _fd(lambda x: L_hp(qh, x, vh), kh), rtol=1e-6, atol=1e-7)
    # dV: derivative of the linear map V -> sum dO o (P^ V), P^ fixed at the point
    S = qa._scores(qh, kh, sc, causal, np.arange(N))
    P, _ = qa._softmax_rows(S)
    Ph = qa.fake_quant_groups(P, fmt, 4)[2].astype(np.float64)
    assert np.allclose(dV[0, 0], _fd(lambda x: float(((Ph @ x) * dO).sum()), vh), rtol=1e-6, atol=1e-7)


def _online_forward(qh, kh, vh, sc, causal, fmt, group, block_n):
    """The source's tile loop in float64: running max m, un-normalised tile
    p = exp(s - m) quantized per row per group, both accumulators rescaled by
    alpha, l summed from the high-precision tile; O /= l at the end."""
    Nq, D = qh.shape
    Nkv = kh.shape[0]
    m = np.full(Nq, -np.inf)
    l = np.zeros(Nq)
    acc = np.zeros((Nq, D))
    acc_hp = np.zeros((Nq, D))
    for n0 in range(0, Nkv, block_n):
        n1 = min(Nkv, n0 + block_n)
        s = sc * (qh @ kh[n0:n1].T)
        if causal:
            s = np.where(np.arange(n0, n1)[None, :] > np.arange(Nq)[:, None], -np.inf, s)
        m_new = np.maximum(m, s.max(axis=1))
        p = np.exp(s - m_new[:, None])
        ph = qa.fake_quant_groups(p, fmt, group)[2].astype(np.float64)
        alpha = np.exp(m - m_new)
        acc = acc * alpha[:, None] + ph @ vh[n0:n1]
        acc_hp = acc_hp * alpha[:, None] + p @ vh[n0:n1]
        l = l * alpha + p.sum(axis=1)
        m = m_new
    return acc / l[:, None], acc_hp / l[:, None], m + np.log(l)


@pytest.mark.parametrize("causal", [False, True])
def test_online_form_equals_plain_definition(causal):
    N, D = 256, 32
    qh, kh, vh = _rand((N, D), 28, 1.5), _rand((N, D), 29), _rand((N, D), 30)
    O, O_hp, lse = qa.forward_head(qh, kh, vh, 0.2, causal=causal)
    Oo, Oo_hp, lse_o = _online_forward(qh, kh, vh, 0.2, causal, "e4m3", 64, 64)
    assert np.allclose(O_hp, Oo_hp, atol=1e-12) and np.allclose(lse, lse_o, atol=1e-12)
    rel = np.linalg.norm(O - Oo) / np.linalg.norm(O)
    assert rel < 1e-5       # fp32 rounding of the differently scaled inputs only
    # the tile-local quantization differs from quantizing P by at most rare bin
    # flips: nearly every row matches to fp32 precision
    row_err = np.abs(O - Oo).max(axis=1) / np.abs(O).max()
    assert np.mean(row_err < 1e-6) > 0.8


def test_p_groups_are_64_absolute_columns():
    D, Nkv = 8, 128
    qh = _rand((4, D), 31)
    kh = _rand((Nkv, D), 32) * 0.3
    vh = _rand((Nkv, D), 33)
    vh[64:] = 0.0                    # keys of group 1 carry no value
    O1, _, lse1 = qa.forward_head(qh, kh, vh, 1.0)
    k2 = kh.copy()
    k2[70] = qh[0] * 4.0             # one dominant key in group 1 (for row 0)
    O2, _, lse2 = qa.forward_head(qh, k2, vh, 1.0)
    gamma = np.exp(lse1 - lse2)
    # group 0's quantized P only rescales by gamma: O scales exactly
    assert np.allclose(O2[0], gamma[0] * O1[0], rtol=1e-6, atol=1e-12)
    # with a 128-wide group the dominant key would set row 0's scale and
    # crush group 0's values: the same check fails
    O1w, _, _ = qa.forward_head(qh, kh, vh, 1.0, group=128)
    O2w, _, _ = qa.forward_head(qh, k2, vh, 1.0, group=128)
    assert not np.allclose(O2w[0], gamma[0] * O1w[0], rtol=1e-3)


def test_row_and_key_subsets_match_full():
    q, k, v, do = _rand((1, 1, 90, 16), 34), _rand((1, 1, 90, 16), 35), _rand((1, 1, 90, 16), 36), _rand((1, 1, 90, 16), 37)
    qh, kh, vh = q[0, 0], k[0, 0], v[0, 0]
    O, O_hp, lse = qa.forward_head(qh, kh, vh, 0.3, causal=True)
    rows = np.array([0, 7, 63, 64, 89])
    Os, Os_hp, lses = qa.forward_head(qh, kh, vh, 0.3, causal=True, rows=rows)
    assert np.array_equal(Os, O[rows]) and np.array_equal(lses, lse[rows])
    dQ, dK, dV = qa.backward_head(qh, kh, vh, do[0, 0], 0.3, causal=True)
    dQs, dKs, dVs = qa.backward_head(qh, kh, vh, do[0, 0], 0.3, causal=True, q_rows=rows, k_rows=rows, row_block=32)
    assert np.allclose(dQs, dQ[rows], atol=1e-12) and np.allclose(dKs, dK[rows], atol=1e-12)
    assert np.allclose(dVs, dV[rows], atol=1e-12)


def test_fp8_v_path():
    q, k = _rand((1, 2, 10, 16), 38), _rand((1, 2, 30, 16), 39)
    vf = _rand((1, 2, 30, 16), 40)
    codes, vs = qa.quantize_v_channels(vf)
    O, O_hp, _ = qa.attention_forward(q, k, None, 0.25, p_fmt="e5m2", v_codes=codes, v_scale=vs)
    vh = qa.dequant_v_channels(codes, vs)
    O_ref, O_hp_ref, _ = qa.attention_forward(q, k, vh, 0.25, p_fmt="e5m2")
    assert np.array_equal(O, O_ref) and np.array_equal(O_hp, O_hp_ref)
    # e5m2 V codes hold about 2 mantissa bits: V^ is within 1/8 relative of V per channel
    assert np.max(np.abs(vh - vf) / np.abs(vf).max(axis=2, keepdims=True)) <= 2.0 ** -3
