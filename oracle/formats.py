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

    ``kind`` is ``"f32"`` (float32 array), ``"bf16"`` (uint16 bit patterns),
    ``"e4m3"`` (uint8 codes with one float32 scale per row held in ``scale``,
    value = decode(code) * scale), ``"mxfp4"`` (packed E2M1 bytes, n/2 per
    row, with E8M0 block scales [n/32] per row in ``scale``) or ``"fp8bf16"``
    (576-byte rows: 448 e4m3 codes then 64 bf16, one float32 scale per row).  ``rows(idx)`` decodes only the requested
    rows along axis 0 to float64, so a 1 GiB cache is never expanded whole.
    """

    def __init__(self, data, kind, scale=None):
        if kind not in ("f32", "bf16", "e4m3", "mxfp4", "fp8bf16"):
            raise ValueError(kind)
        if kind in ("e4m3", "mxfp4", "fp8bf16") and scale is None:
            raise ValueError(f"{kind} needs its scales")
        self.data = data
        self.kind = kind
        self.scale = scale

    def __len__(self):
        return self.data.shape[0]

    @property
    def shape(self):
        return self.data.shape

    @property
    def width(self):
        """Length of a decoded row (two E2M1 values per byte for mxfp4; 448 +
        64 values in 576 bytes for fp8bf16)."""
        if self.kind == "mxfp4":
            return 2 * self.data.shape[-1]
        if self.kind == "fp8bf16":
            return FP8_DIMS + BF16_DIMS
        return self.data.shape[-1]

    def rows(self, idx=None):
        d = self.data if idx is None else self.data[idx]
        if self.kind == "f32":
            return f32_to_f64(d)
        if self.kind == "bf16":
            return bf16_bits_to_f64(d)
        s = self.scale if idx is None else self.scale[idx]
        if self.kind == "mxfp4":
            return mxfp4_decode(d, s)
        if self.kind == "fp8bf16":
            return fp8bf16_decode(d, s)
        v = e4m3fn_to_f64(d)
        s = np.asarray(s, dtype=np.float32).astype(np.float64)
        return v * s.reshape(s.shape + (1,) * (v.ndim - s.ndim))

    def all(self):
        return self.rows(None)


# ---------------------------------------------------------------------------
# OCP MX FP4: E2M1 elements in blocks of 32 sharing one E8M0 scale
# ("DeepSeek-V4" book ch. 16 "The two main FP4 targets", "Why use
# fine-grained scales?": 1 x 32 tiles; ch. 8: a 128-dim FP4 key is 64 bytes
# plus four one-byte scales for groups of 32)
# ---------------------------------------------------------------------------

MX_BLOCK = 32


def e2m1_to_f64(codes):
    """Decode 4-bit E2M1 codes (1 sign, 2 exponent bits with bias 1, 1
    fraction bit; exponent 0 is subnormal: value = f/2)."""
    c = np.asarray(codes).astype(np.int64) & 0xF
    sign = np.where(c & 8, -1.0, 1.0)
    e = (c >> 1) & 3
    f = (c & 1).astype(np.float64)
    mag = np.where(e == 0, f * 0.5, np.ldexp(1.0 + f * 0.5, e - 1))
    return sign * mag


def e8m0_to_f64(codes):
    """Decode E8M0 scales: 2**(code - 127); code 255 is NaN."""
    c = np.asarray(codes).astype(np.int64)
    return np.where(c == 255, np.nan, np.ldexp(1.0, c - 127))


def mxfp4_unpack(packed):
    """[..., n/2] bytes -> [..., n] E2M1 codes; element 2j sits in the low
    nibble of byte j, element 2j+1 in the high nibble."""
    p = np.asarray(packed).astype(np.uint8)
    out = np.empty(p.shape[:-1] + (2 * p.shape[-1],), np.uint8)
    out[..., 0::2] = p & 0xF
    out[..., 1::2] = p >> 4
    return out


def mxfp4_pack(codes):
    c = np.asarray(codes).astype(np.uint8)
    return (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8)


def mxfp4_decode(packed, scales):
    """Values of MXFP4 vectors: packed [..., n/2] bytes, scales [..., n/32]
    E8M0 codes."""
    v = e2m1_to_f64(mxfp4_unpack(packed))
    s = e8m0_to_f64(scales)
    return (v.reshape(v.shape[:-1] + (-1, MX_BLOCK)) * s[..., None]).reshape(v.shape)


_E2M1_VALUES = e2m1_to_f64(np.arange(8))  # 0, 0.5, 1, 1.5, 2, 3, 4, 6


def _round_e2m1(y):
    """Nearest E2M1 magnitude code of |y|, ties to the even code, values
    beyond the largest (6) saturating to it."""
    a = np.abs(np.asarray(y, np.float64))
    spacing = np.where(a < 2.0, 0.5, np.where(a < 4.0, 1.0, 2.0))
    r = np.minimum(np.rint(a / spacing) * spacing, 6.0)  # rint: half to even on the multiple
    return np.searchsorted(_E2M1_VALUES, r).astype(np.uint8)


def mxfp4_quantize(x):
    """OCP MX quantisation of float64 vectors (length a multiple of 32): per
    block of 32 the shared exponent is floor(log2(max |v|)) minus the
    element format's largest exponent (2 for E2M1), the scale is 2 to that
    power (E8M0, clamped to its range; an all-zero block takes the smallest
    scale), and every element is v / scale rounded to E2M1, nearest-even,
    saturating.  Returns (packed bytes, scale codes, the float64 values they
    encode)."""
    x = np.asarray(x, np.float64)
    blk = x.reshape(x.shape[:-1] + (-1, MX_BLOCK))
    amax = np.abs(blk).max(axis=-1)
    _, e = np.frexp(np.where(amax > 0, amax, 1.0))  # amax = f 2**e, f in [0.5, 1)
    shared = np.where(amax > 0, (e - 1) - 2, -127)
    code = np.clip(shared + 127, 0, 254).astype(np.uint8)
    scale = np.ldexp(1.0, code.astype(np.int64) - 127)
    y = blk / scale[..., None]
    mag = _round_e2m1(y)
    codes = np.where((np.signbit(y)) & (mag > 0), mag | 8, mag).astype(np.uint8).reshape(x.shape)
    packed = mxfp4_pack(codes)
    return packed, code, mxfp4_decode(packed, code)


# ---------------------------------------------------------------------------
# the main compressed entry: 448 FP8 dims and 64 BF16 rotary dims, 576 bytes
# ("DeepSeek-V4" book ch. 8 "The main compressed-entry payload"; ch. 7: RoPE
# on the last 64 coordinates).  The FP8 part is OCP e4m3fn with one float32
# scale per entry (max |v| / 448, so nothing saturates); the BF16 part is
# rounded to nearest-even.
# ---------------------------------------------------------------------------

FP8_DIMS, BF16_DIMS = 448, 64


def fp8bf16_decode(row_bytes, scale):
    """Rows of [448 e4m3 codes][64 bf16 little-endian] (576 bytes), with
    their float32 scales, to float64 [..., 512]."""
    b = np.asarray(row_bytes).astype(np.uint8)
    codes = b[..., :FP8_DIMS]
    bits = b[..., FP8_DIMS:].reshape(b.shape[:-1] + (BF16_DIMS, 2))
    u16 = bits[..., 0].astype(np.uint16) | (bits[..., 1].astype(np.uint16) << 8)
    s = np.asarray(scale, np.float32).astype(np.float64)
    return np.concatenate([e4m3fn_to_f64(codes) * s[..., None], bf16_bits_to_f64(u16)], axis=-1)
