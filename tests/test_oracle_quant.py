"""Pins of the oracle's fake quantizer FQ.

The quantizer module is not printed on the pages, so FQ follows the reading
"absmax scale, round to the fp8 grid, dequantize" made exact in fp32.  What
pins it here is independent of its code: a worked example derived by hand,
the absmax element landing exactly on +-FMAX, exact power-of-two scale
equivariance, code idempotence, the format's rounding error bound, group
independence and the zero / underflow special cases.
"""
import numpy as np
import pytest

from oracle import fp8
from oracle import qat_attention as qa


def test_worked_example_e4m3():
    # a = 1, so r = 448 exactly and s = fp32(1/448) = fp32(1/7) * 2^-6.
    # v = x * r: 448, 224, fp32(0.3)*448 = 134.40000534 -> fp32 134.40001, 0, 28, 119.
    # e4m3 spacing is 16 in [128, 256), 8 in [64, 128), 2 in [16, 32):
    #   134.4 -> 128, 119 -> 120, 28 -> 28.
    x = np.array([[1.0, 0.5, 0.3, 0.0, 0.0625, 0.265625]])
    codes, s, xh = qa.fake_quant_groups(x, "e4m3", 64)
    assert list(fp8.decode(codes[0], "e4m3")) == [448, 224, 128, 0, 28, 120]
    assert list(codes[0]) == [0x7E, 0x76, 0x70, 0x00, 0x5E, 0x6F]
    # fp32(1/7) = 0x3E124925
    s_expect = np.float32(np.uint32(0x3E124925).view(np.float32) * np.float32(2.0 ** -6))
    assert s[0, 0] == s_expect
    # x^_0 = fp32(448 * s) = fp32(7 * fp32(1/7)) = fp32(1.0000000447) = 1.0
    assert xh[0, 0] == np.float32(1.0)
    assert xh[0, 3] == 0.0
    # x^_4 = fp32(28 * s): 28 = 4 * 7 -> 4 * 2^-6 * 7 * fp32(1/7) rounds to 0.0625
    assert xh[0, 4] == np.float32(0.0625)


def test_worked_example_e5m2():
    # a = 2, r = fp32(57344 / 2) = 28672, s = 2 / 57344 = 2^-11 * (1/14)...
    # v = [57344, -28672, 7168 + 0.25*... ] : x = [2, -1, 0.25+2^-12]
    # 0.25 * 28672 = 7168 (exact grid point 1.75 * 2^12);
    # (0.25 + 2^-12) * 28672 = 7175 -> spacing 1024 in [4096, 8192) -> 7168.
    x = np.array([[2.0, -1.0, 0.25 + 2.0 ** -12]])
    codes, s, xh = qa.fake_quant_groups(x, "e5m2", 8)
    assert list(fp8.decode(codes[0], "e5m2")) == [57344.0, -28672.0, 7168.0]


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_absmax_element_maps_to_fmax(fmt):
    rng = np.random.default_rng(1)
    x = rng.standard_normal((500, 64)) * np.exp2(rng.integers(-30, 30, (500, 1)))
    codes, s, _ = qa.fake_quant_groups(x, fmt, 64)
    vals = np.abs(fp8.decode(codes, fmt))
    arg = np.argmax(np.abs(x.astype(np.float32)), axis=1)
    assert np.all(vals[np.arange(500), arg] == fp8.fmax(fmt))
    assert np.all(vals <= fp8.fmax(fmt))


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_power_of_two_equivariance_and_idempotence(fmt):
    rng = np.random.default_rng(2)
    x = rng.standard_normal((300, 40)).astype(np.float32)
    c1, s1, xh1 = qa.fake_quant_groups(x, fmt, 16)
    for k in (-20, -3, 5, 17):
        c2, s2, xh2 = qa.fake_quant_groups(x * np.float32(2.0 ** k), fmt, 16)
        assert np.array_equal(c1, c2)
        assert np.array_equal(xh2, xh1 * np.float32(2.0 ** k))
    # quantizing the quantized values again gives the same codes
    c3, _, _ = qa.fake_quant_groups(xh1, fmt, 16)
    assert np.array_equal(c3, c1)


@pytest.mark.parametrize("fmt,mbits", [("e4m3", 3), ("e5m2", 2)])
def test_error_bound(fmt, mbits):
    # the rounding error of the format: at most half a grid spacing, i.e.
    # 2^-(mbits+1) relative for normals, plus at most a few fp32 ulps from s.
    rng = np.random.default_rng(3)
    x = rng.standard_normal((400, 64))
    _, s, xh = qa.fake_quant_groups(x, fmt, 64)
    x32 = x.astype(np.float32).astype(np.float64)
    a = np.max(np.abs(x32), axis=1, keepdims=True)
    err = np.abs(xh.astype(np.float64) - x32)
    sub_floor = a / fp8.fmax(fmt) * 2.0 ** (1 - fp8.FORMATS[fmt][2] - mbits)
    bound = np.maximum(np.abs(x32) * 2.0 ** -(mbits + 1), sub_floor / 2) * (1 + 1e-6) + a * 2.0 ** -22
    assert np.all(err <= bound)


def test_groups_are_independent_and_absolute():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((10, 150))
    c, s, xh = qa.fake_quant_groups(x, "e4m3", 64)
    assert s.shape == (10, 3)
    y = x.copy()
    y[:, 64:128] *= 1000.0        # only the middle group changes
    c2, s2, xh2 = qa.fake_quant_groups(y, "e4m3", 64)
    assert np.array_equal(c[:, :64], c2[:, :64]) and np.array_equal(c[:, 128:], c2[:, 128:])
    assert np.array_equal(xh[:, :64], xh2[:, :64])
    # the tail group [128, 150) is its own group: its absmax maps to 448
    tail = np.abs(fp8.decode(c[:, 128:], "e4m3"))
    assert np.all(tail.max(axis=1) == 448.0)
    # rows are independent
    z = x.copy()
    z[3] *= -7.0
    c4, _, _ = qa.fake_quant_groups(z, "e4m3", 64)
    assert np.array_equal(np.delete(c4, 3, 0), np.delete(c, 3, 0))


def test_zero_and_underflow_groups():
    x = np.zeros((3, 8))
    x[1, 2] = 1e-37          # FMAX / a overflows fp32: the group flushes to zero
    x[2, 5] = -3.0
    c, s, xh = qa.fake_quant_groups(x, "e4m3", 8)
    assert np.all(c[0] == 0) and s[0, 0] == 0 and np.all(xh[0] == 0)
    assert np.all(c[1] == 0) and s[1, 0] == 0 and np.all(xh[1] == 0)
    assert c[2, 5] == 0xFE and xh[2, 5] == np.float32(-3.0)


def test_token_and_channel_helpers():
    rng = np.random.default_rng(6)
    x = rng.standard_normal((2, 3, 20, 16))
    codes, scales, xhat = qa.quantize_token_rows(x)
    assert codes.shape == x.shape and scales.shape == (2, 3, 20)
    # per-token: the absmax of every token row is +-448
    assert np.all(np.abs(fp8.decode(codes, "e4m3")).max(axis=-1) == 448.0)
    vc, vs = qa.quantize_v_channels(x)
    assert vc.shape == x.shape and vs.shape == (2, 3, 16)
    # per-channel: the absmax over tokens of every channel is +-57344
    assert np.all(np.abs(fp8.decode(vc, "e5m2")).max(axis=2) == 57344.0)
    vh = qa.dequant_v_channels(vc, vs)
    assert np.max(np.abs(vh - x) / np.abs(x).max(axis=2, keepdims=True)) < 2.0 ** -3
