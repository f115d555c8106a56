"""Pins of the oracle's fp8 codec against things other than itself.

* every code's value against torch's own float8 dtypes (a library decoder);
* rounding against a brute-force nearest-grid-point search with the
  ties-to-even rule, on every fp32 value within a few ulps of every grid point
  and of every midpoint between grid points (the only places where rounding
  decisions change), plus a strided sweep of all fp32 values in range;
* rounding against torch's CPU float8 casts inside the finite range.
"""
import numpy as np
import pytest
import torch

from oracle import fp8

TORCH_DT = {"e4m3": torch.float8_e4m3fn, "e5m2": torch.float8_e5m2}


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_decode_matches_torch_float8(fmt):
    codes = np.arange(256, dtype=np.uint8)
    ours = fp8.decode(codes, fmt)
    ref = torch.from_numpy(codes.copy()).view(TORCH_DT[fmt]).to(torch.float64).numpy()
    both_nan = np.isnan(ours) & np.isnan(ref)
    assert np.array_equal(np.where(both_nan, 0, ours), np.where(both_nan, 0, ref))


def test_grid_shape():
    g4, g5 = fp8.grid("e4m3"), fp8.grid("e5m2")
    assert len(g4) == 127 and g4[-1] == 448.0 and g4[1] == 2.0 ** -9
    assert len(g5) == 124 and g5[-1] == 57344.0 and g5[1] == 2.0 ** -16


def _brute_force(v, fmt):
    """Nearest finite grid value; ties go to the code with an even mantissa."""
    g = fp8.grid(fmt)
    codes = fp8.encode(g, fmt)
    a = np.abs(v.astype(np.float64))
    vmax = g[-1]
    a_c = np.minimum(a, vmax)
    hi = np.searchsorted(g, a_c, side="left")
    hi = np.clip(hi, 0, len(g) - 1)
    lo = np.clip(hi - 1, 0, len(g) - 1)
    dlo = a_c - g[lo]
    dhi = g[hi] - a_c
    pick_hi = (dhi < dlo) | ((dhi == dlo) & ((codes[hi] & 1) == 0))
    pick = np.where(pick_hi, hi, lo)
    exact = g[hi] == a_c
    pick = np.where(exact, hi, pick)
    return np.copysign(g[pick], v)


def _boundary_values(fmt):
    g = fp8.grid(fmt)
    mids = (g[:-1] + g[1:]) / 2
    pts = np.concatenate([g, mids, [g[-1] * (1 + 2.0 ** -23), g[-1] * 1.01, 2.0 ** -30]])
    f = pts.astype(np.float32)
    out = [f]
    for k in range(1, 5):
        out.append(np.nextafter(f, np.float32(np.inf)))
        out.append(np.nextafter(f, np.float32(0)))
        f2 = out[-2]
        for _ in range(k - 1):
            f2 = np.nextafter(f2, np.float32(np.inf))
        out.append(f2)
    v = np.concatenate(out)
    v = v[np.isfinite(v)]
    return np.concatenate([v, -v])


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_rounding_vs_brute_force_at_boundaries(fmt):
    v = _boundary_values(fmt)
    vals, codes = fp8.round_rne_sat(v, fmt)
    ref = _brute_force(v, fmt)
    assert np.array_equal(vals, ref)
    assert np.array_equal(fp8.decode(codes, fmt), vals)


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_rounding_vs_brute_force_strided_sweep(fmt):
    # every 97th fp32 bit pattern between 0 and FMAX*(1+2^-23)
    top = np.float32(fp8.fmax(fmt) * (1 + 2.0 ** -23)).view(np.uint32)
    bits = np.arange(0, int(top) + 1, 97, dtype=np.uint32)
    v = bits.view(np.float32)
    vals, _ = fp8.round_rne_sat(v, fmt)
    assert np.array_equal(vals, _brute_force(v, fmt))


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_rounding_vs_torch_cast_in_range(fmt):
    rng = np.random.default_rng(5)
    fm = fp8.fmax(fmt)
    v = np.concatenate([
        rng.uniform(-fm, fm, 200000),
        np.exp2(rng.uniform(-20, np.log2(fm), 200000)) * rng.choice([-1, 1], 200000),
        _boundary_values(fmt),
    ]).astype(np.float32)
    v = v[np.abs(v) <= fm]
    vals, _ = fp8.round_rne_sat(v, fmt)
    ref = torch.from_numpy(v).to(TORCH_DT[fmt]).to(torch.float64).numpy()
    assert np.array_equal(vals, ref)


def test_saturation_and_signed_zero():
    vals, codes = fp8.round_rne_sat(np.array([448.0 * (1 + 2.0 ** -23), -500.0, -0.0, 0.0]), "e4m3")
    assert list(vals[:2]) == [448.0, -448.0]
    assert codes[0] == 0x7E and codes[1] == 0xFE
    assert codes[2] == 0x80 and codes[3] == 0x00
    vals, codes = fp8.round_rne_sat(np.array([1e6, 57344.0]), "e5m2")
    assert list(vals) == [57344.0, 57344.0] and codes[0] == 0x7B


def test_ties_to_even_examples():
    # e4m3 around 1: spacing 1/8.  1.0625 is the midpoint of 1 (mantissa 000)
    # and 1.125 (mantissa 001): goes to 1.  1.1875 lies between 1.125 (001)
    # and 1.25 (010): goes to 1.25.  Subnormal: 1.5 * 2^-9 -> 2^-8.
    vals, _ = fp8.round_rne_sat(np.array([1.0625, 1.1875, 1.5 * 2.0 ** -9, 0.5 * 2.0 ** -9]), "e4m3")
    assert list(vals) == [1.0, 1.25, 2.0 ** -8, 0.0]
    # e5m2 around 1: spacing 1/4.  1.125 -> 1.0, 1.375 -> 1.5
    vals, _ = fp8.round_rne_sat(np.array([1.125, 1.375]), "e5m2")
    assert list(vals) == [1.0, 1.5]
