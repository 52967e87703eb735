"""Storage-format codecs for the oracle (test infrastructure only).

The oracle reads the exact stored bytes of every input, so that input
quantisation is never counted as error.  These codecs are written from the
format definitions, not from any library:

* bfloat16: the upper 16 bits of an IEEE-754 binary32 value (1 sign bit,
  8 exponent bits with bias 127, 7 fraction bits).
* OCP FP8 E4M3FN: 1 sign bit, 4 exponent bits with bias 7, 3 fraction bits;
  exponent field 0 is subnormal (value = f/8 * 2**-6); the pattern S.1111.111
  is NaN; there is no infinity; the largest finite magnitude is 448.

Tests pin these decoders against torch's own dtype conversions for every code.
"""

import numpy as np


def bf16_bits_to_f64(bits):
    """Decode bfloat16 bit patterns (uint16/int16 array) to float64, exactly."""
    b = np.asarray(bits).astype(np.uint16).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):
        return b.view(np.float32).astype(np.float64)


def f64_to_bf16_bits(x):
    """Round float64 values to the nearest bfloat16 (ties to even); return bits.

    Rounding is done once, directly from float64 (no detour through binary32
    that could round twice).  The significand of a bfloat16 has 8 bits, so the
    spacing of representable values around |x| in [2**e, 2**(e+1)) is
    2**(e-7); below the smallest normal (2**-126) the spacing is fixed at
    2**-133.  Magnitudes that round to 2**128 or above become infinity.
    """
    x = np.asarray(x, dtype=np.float64)
    out = np.empty(x.shape, dtype=np.float64)
    a = np.abs(x)
    finite = np.isfinite(a) & (a > 0)
    _, e = np.frexp(np.where(finite, a, 1.0))  # a = mant * 2**e, mant in [0.5, 1)
    # exponent of the leading bit is e-1; spacing 2**(e-1-7), floored at 2**-133
    spacing_exp = np.maximum(e - 8, -133)
    q = np.ldexp(1.0, spacing_exp)
    r = np.rint(a / q) * q  # np.rint rounds half to even; a/q is exact
    r = np.where(r >= 2.0 ** 128, np.inf, r)
    out = np.where(finite, np.copysign(r, x), x)  # zeros, infs and nans pass
    f32 = out.astype(np.float32)  # exact: every r is a bfloat16 value
    bits = (f32.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(x)
    if np.any(nan):
        bits = np.where(nan, np.uint16(0x7FC0), bits)
    return bits


def round_to_bf16(x):
    """Float64 value of the bfloat16 nearest to x (ties to even)."""
    return bf16_bits_to_f64(f64_to_bf16_bits(x))


def e4m3fn_to_f64(codes):
    """Decode OCP FP8 E4M3FN codes (uint8 array) to float64, exactly."""
    c = np.asarray(codes).astype(np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    exp = (c >> 3) & 0xF
    frac = (c & 0x7).astype(np.float64)
    normal = np.ldexp(1.0 + frac / 8.0, exp - 7)
    subnormal = np.ldexp(frac / 8.0, -6)
    mag = np.where(exp == 0, subnormal, normal)
    mag = np.where((exp == 0xF) & ((c & 0x7) == 0x7), np.nan, mag)
    return sign * mag


def f32_to_f64(x):
    return np.asarray(x, dtype=np.float32).astype(np.float64)


class Stored:
    """A stored tensor as the oracle sees it: raw values plus their format.

    ``kind`` is ``"f32"`` (float32 array), ``"bf16"`` (uint16 bit patterns) or
    ``"e4m3"`` (uint8 codes with one float32 scale per row held in ``scale``,
    value = decode(code) * scale).  ``rows(idx)`` decodes only the requested
    rows along axis 0 to float64, so a 1 GiB cache is never expanded whole.
    """

    def __init__(self, data, kind, scale=None):
        if kind not in ("f32", "bf16", "e4m3"):
            raise ValueError(kind)
        if kind == "e4m3" and scale is None:
            raise ValueError("e4m3 needs per-row scales")
        self.data = data
        self.kind = kind
        self.scale = scale

    def __len__(self):
        return self.data.shape[0]

    @property
    def shape(self):
        return self.data.shape

    def rows(self, idx=None):
        d = self.data if idx is None else self.data[idx]
        if self.kind == "f32":
            return f32_to_f64(d)
        if self.kind == "bf16":
            return bf16_bits_to_f64(d)
        s = self.scale if idx is None else self.scale[idx]
        v = e4m3fn_to_f64(d)
        s = np.asarray(s, dtype=np.float32).astype(np.float64)
        return v * s.reshape(s.shape + (1,) * (v.ndim - s.ndim))

    def all(self):
        return self.rows(None)
