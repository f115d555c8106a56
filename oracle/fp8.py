"""FP8 grids of the OCP 8-bit formats, written from the format definitions.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import this module;
only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` use it.

The pages name the target formats only by the quantizer call of the FastVideo
``attn_qat_train.py`` source (``fake_quantize(..., dst_dtype=...)`` inside
``_attn_fwd_inner`` and the backward inner loops) and by the e5m2 value path
(``FP8_OUTPUT``, ``tl.float8e5``) of ``_attn_fwd``.  The grids themselves are
the OCP 8-bit floating-point definitions:

* e4m3fn: 1 sign, 4 exponent (bias 7), 3 mantissa bits; no infinities; the
  all-ones pattern S.1111.111 is NaN, so the largest finite value is
  1.75 * 2**8 = 448; smallest subnormal 2**-9.
* e5m2: 1 sign, 5 exponent (bias 15), 2 mantissa bits; IEEE-like, exponent
  field 31 holds Inf/NaN, so the largest finite value is 1.75 * 2**15 = 57344;
  smallest subnormal 2**-16.

Everything here is float64 arithmetic on exactly representable values, so the
results are exact.
"""
from __future__ import annotations

import numpy as np

# name -> (exponent bits, mantissa bits, bias, largest finite value)
FORMATS = {
    "e4m3": (4, 3, 7, 448.0),
    "e5m2": (5, 2, 15, 57344.0),
}


def fmt_params(fmt: str):
    if fmt not in FORMATS:
        raise ValueError(f"unknown fp8 format {fmt!r}")
    return FORMATS[fmt]


def fmax(fmt: str) -> float:
    return fmt_params(fmt)[3]


def decode(codes, fmt: str) -> np.ndarray:
    """Value of each 8-bit code, straight from the bit-field definition.

    NaN/Inf encodings decode to NaN/Inf; the quantizer never produces them.
    """
    ebits, mbits, bias, _ = fmt_params(fmt)
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where((c >> 7) & 1, -1.0, 1.0)
    e = (c >> mbits) & ((1 << ebits) - 1)
    m = c & ((1 << mbits) - 1)
    sub = m.astype(np.float64) * 2.0 ** (1 - bias - mbits)
    nrm = (1.0 + m.astype(np.float64) / (1 << mbits)) * np.exp2(e.astype(np.float64) - bias)
    val = np.where(e == 0, sub, nrm)
    emax_field = (1 << ebits) - 1
    if fmt == "e4m3":
        val = np.where((e == emax_field) & (m == (1 << mbits) - 1), np.nan, val)
    else:
        val = np.where(e == emax_field, np.where(m == 0, np.inf, np.nan), val)
    return sign * val


def grid(fmt: str) -> np.ndarray:
    """All finite non-negative values of the format, ascending."""
    v = decode(np.arange(128, dtype=np.uint8), fmt)
    return np.unique(v[np.isfinite(v)])


def round_rne_sat(v, fmt: str):
    """Round float values onto the format's grid: nearest, ties to even, saturating.

    Returns ``(values, codes)``: ``values`` as float64 (exactly on the grid, with
    the sign of the input kept on zero) and ``codes`` as uint8.

    Definition used: for |v| with binary exponent e = floor(log2|v|), clamped
    below at the smallest normal exponent 1 - bias, the spacing of the grid
    around |v| is 2**(e - mbits); |v| is divided by that spacing, rounded to
    the nearest integer with ties to even (the last kept mantissa bit is the
    parity of that integer), multiplied back and clamped to the largest finite
    value.
    """
    ebits, mbits, bias, vmax = fmt_params(fmt)
    x = np.asarray(v, dtype=np.float64)
    if np.isnan(x).any():
        raise ValueError("NaN input has no fp8 rounding here")
    a = np.abs(x)
    emin = 1 - bias
    with np.errstate(divide="ignore"):
        _, ex = np.frexp(a)          # a = f * 2**ex, f in [0.5, 1)
    e = np.maximum(ex - 1, emin)     # floor(log2 a), clamped to the normal range
    e = np.where(a == 0, emin, e)
    quantum = np.ldexp(1.0, (e - mbits).astype(np.int64))
    n = np.rint(a / quantum)         # np.rint: round half to even
    mag = np.minimum(n * quantum, vmax)
    vals = np.copysign(mag, x)
    return vals, encode(vals, fmt)


def encode(vals, fmt: str) -> np.ndarray:
    """8-bit code of values that lie exactly on the grid (sign of zero kept)."""
    ebits, mbits, bias, vmax = fmt_params(fmt)
    x = np.asarray(vals, dtype=np.float64)
    a = np.abs(x)
    if (a > vmax).any():
        raise ValueError("value beyond the largest finite fp8 value")
    sign = np.signbit(x).astype(np.int64) << 7
    emin = 1 - bias
    with np.errstate(divide="ignore"):
        _, ex = np.frexp(a)
    e = ex - 1
    normal = (a >= 2.0 ** emin)
    sub_m = np.where(normal, 0, np.rint(a / 2.0 ** (emin - mbits))).astype(np.int64)
    nrm_m = np.where(normal, np.rint(a / np.exp2(np.where(normal, e, 0).astype(np.float64)) * (1 << mbits)) - (1 << mbits), 0).astype(np.int64)
    e_field = np.where(normal, e + bias, 0).astype(np.int64)
    m_field = np.where(normal, nrm_m, sub_m)
    codes = sign | (e_field << mbits) | m_field
    back = decode(codes.astype(np.uint8), fmt)
    if not np.array_equal(np.abs(back), a):
        raise ValueError("value is not on the fp8 grid")
    return codes.astype(np.uint8)
