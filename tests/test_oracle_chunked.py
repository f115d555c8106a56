"""Pins of the oracle's chunked-KV mode (the local half of ring attention on
the "usp: differentiable operators for training" page): forward results of
KV chunks merged by log-sum-exp equal the unchunked forward, the quantized O
included when chunk boundaries are multiples of the 64-key P group (and not
otherwise); each chunk's backward with the merged lse and O_hp gives that
chunk's dK, dV, and the chunks' dQ add up to dQ."""
import numpy as np
import pytest

from oracle import qat_attention as qa


def _inputs(seed, Nq=40, Nkv=192, D=16, H=2):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((1, H, Nq, D))
    k = rng.standard_normal((1, H, Nkv, D)) * 1.5
    v = rng.standard_normal((1, H, Nkv, D))
    do = rng.standard_normal((1, H, Nq, D))
    return q, k, v, do


def _chunked_forward(q, k, v, sm, bounds, **kw):
    parts = [qa.attention_forward(q, k[:, :, a:b], v[:, :, a:b], sm, **kw) for a, b in bounds]
    return qa.merge_chunks([p[0] for p in parts], [p[1] for p in parts], [p[2] for p in parts])


@pytest.mark.parametrize("bounds", [[(0, 64), (64, 128), (128, 192)], [(0, 128), (128, 192)]])
def test_chunked_forward_equals_unchunked(bounds):
    q, k, v, _ = _inputs(1)
    sm = 0.25
    O, Oh, lse = qa.attention_forward(q, k, v, sm)
    Oc, Ohc, lsec = _chunked_forward(q, k, v, sm, bounds)
    # FQ quantizes the fp32-rounded chunk probabilities: the per-group scale
    # invariance holds up to that rounding
    assert np.linalg.norm(Oc - O) <= 1e-6 * np.linalg.norm(O)
    assert np.allclose(Ohc, Oh, rtol=1e-12, atol=1e-13)
    assert np.allclose(lsec, lse, rtol=0, atol=1e-12)


def test_misaligned_chunks_change_only_the_quantized_output():
    q, k, v, _ = _inputs(2)
    sm = 0.25
    O, Oh, lse = qa.attention_forward(q, k, v, sm)
    Oc, Ohc, lsec = _chunked_forward(q, k, v, sm, [(0, 96), (96, 192)])   # splits the group [64, 128)
    assert np.allclose(Ohc, Oh, rtol=1e-12, atol=1e-13) and np.allclose(lsec, lse, atol=1e-12)
    assert np.linalg.norm(Oc - O) > 1e-4 * np.linalg.norm(O)


def test_merge_of_masked_rows():
    """A chunk whose row is fully masked (lse -inf) takes no weight; a row
    masked in every chunk merges to lse -inf and zeros."""
    o = [np.ones((1, 1, 2, 4)), 2 * np.ones((1, 1, 2, 4))]
    lse = [np.array([[[-np.inf, -np.inf]]]), np.array([[[0.5, -np.inf]]])]
    O, Oh, L = qa.merge_chunks(o, o, lse)
    assert np.array_equal(O[0, 0, 0], [2.0] * 4) and np.array_equal(O[0, 0, 1], [0.0] * 4)
    assert L[0, 0, 0] == 0.5 and L[0, 0, 1] == -np.inf


def test_chunked_backward_equals_unchunked():
    q, k, v, do = _inputs(3)
    sm = 0.25
    bounds = [(0, 64), (64, 192)]
    O, Oh, lse = qa.attention_forward(q, k, v, sm)
    dq, dk, dv = qa.attention_backward(q, k, v, do, sm)
    dq_sum = np.zeros_like(dq)
    for a, b in bounds:
        dqc, dkc, dvc = qa.attention_backward(q, k[:, :, a:b], v[:, :, a:b], do, sm, lse=lse, o_hp=Oh)
        assert np.allclose(dkc, dk[:, :, a:b], rtol=1e-10, atol=1e-12)
        assert np.allclose(dvc, dv[:, :, a:b], rtol=1e-10, atol=1e-12)
        dq_sum += dqc
    assert np.allclose(dq_sum, dq, rtol=1e-10, atol=1e-12)
