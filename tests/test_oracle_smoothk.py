"""Pins of the oracle's K smoothing (FastVideo attn_qat_train.py,
_attention.forward "smoothing k" and the SMOOTH_K term of _attn_bwd_dq).

Softmax is invariant to a per-row shift of the scores, and S_s = Q (K - c)^T
= S - Q c shifts row i by q_i . c.  With inputs built so that K - c is exact
in the storage dtype, smoothing must leave O, O_hp, dQ (with its
rowsum(dS) k_mean term), dK and dV unchanged and move lse by
-sm_scale q_i . c; with Q/K/V quantization on, smoothing must happen before
K is quantized.
"""
import numpy as np
import pytest

from oracle import qat_attention as qa


def _shift_inputs(seed, B=1, H=2, N=24, D=16):
    """K = K0 + c with every channel of K0 made of +/- pairs (column mean 0
    over batch, heads and tokens) on a 1/8 grid, c on a 1/4 grid: K, c and
    K - c are exact in bf16."""
    rng = np.random.default_rng(seed)
    half = rng.integers(-24, 25, size=(B, H, N // 2, D)) / 8.0
    k0 = np.concatenate([half, -half], axis=2)
    c = rng.integers(-6, 7, size=D) / 4.0
    q = rng.integers(-16, 17, size=(B, H, N, D)) / 8.0
    v = rng.standard_normal((B, H, N, D))
    do = rng.standard_normal((B, H, N, D))
    return q, k0 + c[None, None, None, :], k0, v, do, c


def test_round_storage_ties_to_even():
    x = np.array([1 + 2.0**-8, 1 + 3 * 2.0**-8, -(1 + 2.0**-8), 3.0])
    assert np.array_equal(qa.round_storage(x, "bf16"), [1.0, 1 + 2.0**-6, -1.0, 3.0])
    y = np.array([1 + 2.0**-11, 1 + 3 * 2.0**-11])
    assert np.array_equal(qa.round_storage(y, "fp16"), [1.0, 1 + 2.0**-9])


def test_key_mean_is_over_batch_heads_and_tokens():
    k = np.zeros((2, 2, 4, 3))
    k[0, 0] += 1.0
    k[0, 1] += 3.0
    k[1, 0] += 2.0
    k[1, 1] += 6.0
    assert np.array_equal(qa.smooth_key_mean(k, "bf16"), [3.0, 3.0, 3.0])
    assert np.array_equal(qa.smooth_keys(k[0, 1], qa.smooth_key_mean(k, "bf16"), "bf16"), np.zeros((4, 3)))


@pytest.mark.parametrize("p_quant", [False, True])
@pytest.mark.parametrize("causal", [False, True])
def test_smoothing_is_a_score_shift(p_quant, causal):
    q, k, k0, v, do, c = _shift_inputs(3)
    sm = 0.25
    assert np.array_equal(qa.smooth_key_mean(k, "bf16"), c)
    kw = dict(causal=causal, p_quant=p_quant, dtype="bf16")
    O, Oh, lse = qa.attention_forward(q, k, v, sm, **kw)
    Os, Ohs, lses = qa.attention_forward(q, k, v, sm, smooth_k=True, **kw)
    assert np.allclose(Os, O, rtol=1e-12, atol=1e-13)
    assert np.allclose(Ohs, Oh, rtol=1e-12, atol=1e-13)
    assert np.allclose(lses, lse - sm * np.einsum("bhnd,d->bhn", q, c), rtol=0, atol=1e-12)
    g = qa.attention_backward(q, k, v, do, sm, **kw)
    gs = qa.attention_backward(q, k, v, do, sm, smooth_k=True, **kw)
    for a, b in zip(gs, g):   # dQ (with the rowsum(dS) k_mean term), dK, dV
        assert np.allclose(a, b, rtol=1e-10, atol=1e-12)


def test_smoothing_precedes_qkv_quant():
    """With Q/K/V quantization the smoothed K is what gets quantized: the same
    as quantizing the pre-shifted K0 = K - c (lse shifted by q . c)."""
    q, k, k0, v, do, c = _shift_inputs(5, N=32, D=32)
    sm = 0.2
    O, Oh, lse = qa.attention_forward(q, k, v, sm, qkv_quant=True, smooth_k=True, dtype="bf16")
    O0, Oh0, lse0 = qa.attention_forward(q, k0, v, sm, qkv_quant=True, dtype="bf16")
    assert np.array_equal(O, O0) and np.array_equal(Oh, Oh0)
    assert np.array_equal(lse, lse0)   # the same quantized K0 on both sides
    dq, dk, dv = qa.attention_backward(q, k, v, do, sm, qkv_quant=True, smooth_k=True, dtype="bf16")
    dq0, dk0, dv0 = qa.attention_backward(q, k0, v, do, sm, qkv_quant=True, dtype="bf16")
    assert np.array_equal(dk, dk0) and np.array_equal(dv, dv0)
    assert np.allclose(dq, dq0, rtol=1e-10, atol=1e-12)   # + rowsum(dS) k_mean, zero up to rounding
