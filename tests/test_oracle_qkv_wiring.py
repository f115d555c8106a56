"""Pins of the oracle's Q/K/V fake-quant wiring (FastVideo attn_qat_train.py,
_attention.forward: the fake_quantize_q / fake_quantize_kv pre-pass ahead of
_attn_fwd, and the straight-through return of the gradients).

The reading pinned here: each of Q, K and V is fake-quantized per token (one
absmax scale per (b, h, n) row over D) on the e4m3 grid, and the gradients
are those of attention at the quantized point.  The expected quantized
tensors are written by hand, not produced by the oracle:

* two of the three tensors are fixed points of that quantizer: every row holds
  e4m3 grid values times 2^k_row and one element of magnitude 448 * 2^k_row,
  so its scale is exactly 2^k_row, x * r lands on the grid and FQ(x) = x;
* the third tensor has one row (the last) with absmax 448 * 2^-8 and three off-grid
  values whose e4m3 results are derived by hand below (one of them a tie).

qkv_quant=True on those inputs must then equal the plain attention on the
hand-quantized tensors, forward and backward, bit for bit.  A quantizer left
off one tensor, an e5m2 grid, or one scale per channel instead of per token
all break the equality (tests/test_oracle_mutations.py plants each of them).
"""
import numpy as np
import pytest

from oracle import fp8
from oracle import qat_attention as qa

N, D = 12, 16
SCALE_EXP = range(-12, -7)   # row absmax 448 * 2^k: values of order 0.1 .. 1


def _grid_values(rng, size):
    """Random finite e4m3 values (any code but the two NaN patterns)."""
    codes = rng.integers(0, 256, size=size).astype(np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x7E
    return fp8.decode(codes, "e4m3")


def _fixed_point_tensor(seed):
    """[1, 1, N, D] with rows e4m3 grid values * 2^k_row and one element
    +/-448 * 2^k_row (at a row-dependent column), so that per-token e4m3
    fake quant returns every value unchanged."""
    rng = np.random.default_rng(seed)
    x = np.empty((N, D))
    for n in range(N):
        k = int(rng.choice(list(SCALE_EXP)))
        row = _grid_values(rng, D)
        row[n % D] = 448.0 * (1 if rng.random() < 0.5 else -1)
        x[n] = row * 2.0 ** k
    return x[None, None]


# hand-derived e4m3 results in a row of absmax 448 * 2^-8 (s = 2^-8, r = 2^8):
#   134.4 -> grid step 16 in [128, 256): nearest 128
#   100.0 -> grid step 8 in [64, 128): halfway between 96 (mantissa 4, even)
#            and 104 (mantissa 5): ties to even give 96
#   -0.3  -> grid step 1/32 in [0.25, 0.5): 0.3 * 32 = 9.6 -> 10, i.e. -0.3125
OFF_GRID = [(1, 134.4, 128.0), (2, 100.0, 96.0), (3, -0.3, -0.3125)]


def _off_grid_pair(seed):
    """(tensor, its hand-quantized copy): a fixed-point tensor whose last row
    (a query row that sees every key under the causal mask too) is replaced by
    absmax 448 * 2^-8 plus the three off-grid values above."""
    x = _fixed_point_tensor(seed)
    xq = x.copy()
    rng = np.random.default_rng(seed + 100)
    row = _grid_values(rng, D) * 2.0 ** -8            # grid values at scale 2^-8: unchanged by FQ
    row[0] = 448.0 * 2.0 ** -8
    rowq = row.copy()
    for col, val, qval in OFF_GRID:
        row[col] = val * 2.0 ** -8
        rowq[col] = qval * 2.0 ** -8
    x[0, 0, N - 1], xq[0, 0, N - 1] = row, rowq
    assert not np.array_equal(x, xq)
    return x, xq


def _case(which, seed):
    """Inputs (q, k, v), their hand-quantized copies and dO; ``which`` names
    the tensor that carries the off-grid row."""
    plain = {}
    hand = {}
    for i, name in enumerate("qkv"):
        if name == which:
            plain[name], hand[name] = _off_grid_pair(seed + i)
        else:
            plain[name] = _fixed_point_tensor(seed + i)
            hand[name] = plain[name]
    do = np.random.default_rng(seed + 9).standard_normal((1, 1, N, D))
    return plain, hand, do


@pytest.mark.parametrize("which", ["q", "k", "v"])
@pytest.mark.parametrize("causal", [False, True])
def test_qkv_quant_equals_attention_on_hand_quantized_inputs(which, causal):
    plain, hand, do = _case(which, 50 + 3 * "qkv".index(which) + (7 if causal else 0))
    sc = 1.0
    fwd_q = qa.attention_forward(plain["q"], plain["k"], plain["v"], sc, causal=causal, qkv_quant=True)
    fwd_h = qa.attention_forward(hand["q"], hand["k"], hand["v"], sc, causal=causal, qkv_quant=False)
    for a, b, n in zip(fwd_q, fwd_h, ("O", "O_hp", "lse")):
        assert np.array_equal(a, b), n
    bwd_q = qa.attention_backward(plain["q"], plain["k"], plain["v"], do, sc, causal=causal, qkv_quant=True)
    bwd_h = qa.attention_backward(hand["q"], hand["k"], hand["v"], do, sc, causal=causal, qkv_quant=False)
    for a, b, n in zip(bwd_q, bwd_h, ("dQ", "dK", "dV")):
        assert np.array_equal(a, b), n
    # the case has teeth: without the quantization the off-grid row moves the outputs
    fwd_p = qa.attention_forward(plain["q"], plain["k"], plain["v"], sc, causal=causal, qkv_quant=False)
    assert not np.allclose(fwd_p[1], fwd_h[1], rtol=0, atol=1e-9)


@pytest.mark.parametrize("seed", [61, 62])
def test_fixed_point_tensors_are_fixed(seed):
    """The premise of the pin, checked against the hand argument (scale 2^k,
    grid values): per-token e4m3 FQ leaves the tensor unchanged, while an
    e5m2 grid or per-channel scales do not."""
    x = _fixed_point_tensor(seed)
    codes, scales, xh = qa.quantize_token_rows(x, "e4m3")
    assert np.array_equal(xh.astype(np.float64), x)
    assert np.all(np.log2(scales) == np.round(np.log2(scales)))        # powers of two
    assert not np.array_equal(qa.quantize_token_rows(x, "e5m2")[2].astype(np.float64), x)
    per_channel = qa.quantize_token_rows(np.swapaxes(x, 2, 3), "e4m3")[2]
    assert not np.array_equal(np.swapaxes(per_channel, 2, 3).astype(np.float64), x)
