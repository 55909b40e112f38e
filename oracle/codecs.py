"""Storage codecs used by the latent cache, written from the formats' definitions.

Test infrastructure only (see the package docstring).

The pages say a cache's size "depends on the cache precision" and that engines
may keep an FP8 cache ("Multi-head Latent Attention (MLA) și arhitectura
DeepSeekMoE", "Exemplul 1" and "Greșeli frecvente"). They fix no format, so the
reading taken here is:

* fp32: IEEE binary32.
* bf16: the top 16 bits of binary32 (1 sign, 8 exponent, 7 mantissa bits);
  encoding rounds to nearest, ties to even.
* fp8:  OCP E4M3FN (1 sign, 4 exponent bits with bias 7, 3 mantissa bits, no
  infinities, NaN only at 0x7F / 0xFF, largest finite 448). Encoding rounds
  to nearest, ties to even, then clamps to +-448.

Decoding is exact: every stored value is representable in fp64.
"""

import numpy as np

F8_MAX = 448.0


# ---------------------------------------------------------------- fp32
def f32_decode(x):
    """fp32 array (or raw uint32 bits) -> exact fp64."""
    x = np.asarray(x)
    if x.dtype == np.uint32:
        x = x.view(np.float32)
    return x.astype(np.float64)


def f32_encode(x):
    """fp64 -> fp32, IEEE round-to-nearest-even (NumPy's cast)."""
    return np.asarray(x, dtype=np.float64).astype(np.float32)


# ---------------------------------------------------------------- bf16
def bf16_decode(bits):
    """bf16 bit patterns (uint16 / int16) -> exact fp64: the value is the fp32
    whose upper half is ``bits`` and whose lower half is zero."""
    b = np.asarray(bits).view(np.uint16).astype(np.uint32) << 16
    with np.errstate(invalid="ignore"):  # NaN patterns stay NaN
        return b.view(np.float32).astype(np.float64)


def _round_to_grid(x, mant_bits, min_exp):
    """Round fp64 ``x`` to the nearest value with ``mant_bits`` fraction bits
    and exponent >= ``min_exp`` (below it the spacing stays 2**(min_exp -
    mant_bits): gradual underflow). Ties go to the even neighbour because
    ``np.rint`` rounds half to even and ``x / ulp`` is exact (power-of-two
    scaling)."""
    x = np.asarray(x, dtype=np.float64)
    ax = np.abs(x)
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(ax > 0, ax, 1.0)))
    # log2 in floating point can land one off near powers of two; fix up so
    # that 2**e <= ax < 2**(e+1) holds exactly.
    e = np.where(np.exp2(e) > ax, e - 1, e)
    e = np.where(np.exp2(e + 1) <= ax, e + 1, e)
    e = np.maximum(e, min_exp)
    ulp = np.exp2(e - mant_bits)
    return np.rint(x / ulp) * ulp


def bf16_round(x):
    """fp64 -> nearest bf16 value (as fp64), ties to even; beyond the largest
    finite bf16 the result is +-inf, as an IEEE cast would give."""
    r = _round_to_grid(x, 7, -126)
    bf16_max = float(np.uint32(0x7F7F0000).view(np.float32))
    return np.where(np.abs(r) > bf16_max, np.copysign(np.inf, r), r)


def bf16_encode(x):
    """fp64 -> bf16 bit patterns (uint16), round to nearest even."""
    r = bf16_round(x).astype(np.float32)  # exact: r is on the bf16 grid
    return (r.view(np.uint32) >> 16).astype(np.uint16)


# ---------------------------------------------------------------- fp8 e4m3fn
def e4m3_value(code):
    """Value of one E4M3FN byte from the format definition (NaN for 0x7F/0xFF)."""
    code = int(code) & 0xFF
    sign = -1.0 if code & 0x80 else 1.0
    exp = (code >> 3) & 0xF
    man = code & 0x7
    if exp == 0xF and man == 0x7:
        return float("nan")
    if exp == 0:
        return sign * (man / 8.0) * 2.0 ** (1 - 7)
    return sign * (1.0 + man / 8.0) * 2.0 ** (exp - 7)


E4M3_TABLE = np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)


def e4m3_decode(codes):
    """uint8 E4M3FN codes -> exact fp64 via the 256-entry table."""
    return E4M3_TABLE[np.asarray(codes).view(np.uint8)]


def e4m3_round(x):
    """fp64 -> nearest E4M3FN value (as fp64), ties to even, clamped to +-448
    (saturating: the format has no infinity)."""
    r = _round_to_grid(x, 3, -6)
    return np.clip(r, -F8_MAX, F8_MAX)


_POS_VALUES = E4M3_TABLE[:0x7F]  # codes 0x00..0x7E: the finite values >= 0, ascending


def e4m3_encode(x):
    """fp64 -> E4M3FN codes (uint8), round to nearest even, saturating. After
    rounding every magnitude is exactly one of the table's finite values, so
    its code is that value's index; the sign goes to bit 7."""
    r = e4m3_round(x)
    mag = np.abs(r)
    idx = np.searchsorted(_POS_VALUES, mag)
    assert np.array_equal(_POS_VALUES[idx], mag), "value off the e4m3 grid"
    sign = np.where(np.signbit(r), 0x80, 0)
    return (idx | sign).astype(np.uint8)


def e4m3_token_scale(c_row):
    """Per-token scale of an fp8 latent row: the largest magnitude maps to the
    largest finite code, s = amax / 448 rounded to fp32; an all-zero row gets
    s = 1 so that decoding stays finite."""
    amax = float(np.max(np.abs(np.asarray(c_row, dtype=np.float64))))
    if amax == 0.0:
        return np.float32(1.0)
    return np.float32(amax / F8_MAX)
