"""Exact decoders for the storage formats the attention inputs arrive in.

TEST INFRASTRUCTURE ONLY (see the package docstring).

* bf16: the top 16 bits of an IEEE-754 binary32 value. Decoding is exact.
* fp8 e4m3fn (OCP 8-bit floating point specification, E4M3 encoding): one sign
  bit, four exponent bits with bias 7, three mantissa bits; exponent field 0
  encodes subnormals; there are no infinities; the two codes with all exponent
  and mantissa bits set (0x7F, 0xFF) are NaN; the largest finite magnitude is
  1.75 * 2**8 = 448. The pages only say "FP8 KV cache" ("Attention kernels",
  section "Paged KV and kernels"); the OCP e4m3fn flavour is the reading taken.
"""

import numpy as np

E4M3FN_MAX = 448.0
_E4M3_BIAS = 7


def decode_bf16_bits(bits) -> np.ndarray:
    """uint16 bf16 bit patterns (any shape) -> float64, exactly."""
    b = np.asarray(bits)
    if b.dtype not in (np.uint16, np.int16):
        raise TypeError(f"bf16 bit patterns must be 16-bit integers, got {b.dtype}")
    u32 = b.astype(np.uint16).astype(np.uint32) << np.uint32(16)
    return u32.view(np.float32).astype(np.float64)


def decode_e4m3fn(codes) -> np.ndarray:
    """uint8 OCP e4m3fn codes (any shape) -> float64, from the bit-field definition."""
    c = np.asarray(codes)
    if c.dtype != np.uint8:
        raise TypeError(f"fp8 codes must be uint8, got {c.dtype}")
    c = c.astype(np.int64)
    sign = np.where((c >> 7) & 1, -1.0, 1.0)
    exp_field = (c >> 3) & 0xF
    mant = (c & 0x7).astype(np.float64)
    normal = sign * np.ldexp(1.0 + mant / 8.0, exp_field - _E4M3_BIAS)
    subnormal = sign * np.ldexp(mant / 8.0, 1 - _E4M3_BIAS)
    value = np.where(exp_field == 0, subnormal, normal)
    is_nan = (exp_field == 0xF) & ((c & 0x7) == 0x7)
    return np.where(is_nan, np.nan, value)


def encode_e4m3fn(x) -> np.ndarray:
    """Finite floats (any shape) -> uint8 OCP e4m3fn codes: the nearest representable value,
    ties to the code with an even mantissa, magnitudes beyond 448 saturated to 448.

    Written from the definition: the 127 non-negative finite codes are decoded (they increase
    with the code), the magnitude is placed between its two neighbours, and the nearer one is
    taken (on a tie, the one whose last mantissa bit is 0). The sign bit is copied (so -0.0
    gives 0x80). The caller computes x in the precision its quantiser uses.
    """
    a = np.asarray(x, dtype=np.float64)
    if not np.all(np.isfinite(a)):
        raise ValueError("encode_e4m3fn takes finite values only")
    codes = np.arange(0x7F, dtype=np.uint8)                  # 0x00 .. 0x7E: +0 .. 448
    values = decode_e4m3fn(codes)
    mag = np.minimum(np.abs(a), E4M3FN_MAX)
    hi = np.searchsorted(values, mag, side="left")          # first value >= mag
    hi = np.minimum(hi, len(values) - 1)
    lo = np.maximum(hi - 1, 0)
    d_lo = mag - values[lo]
    d_hi = values[hi] - mag
    take_hi = (d_hi < d_lo) | ((d_hi == d_lo) & ((codes[hi] & 1) == 0))
    code = np.where(take_hi, codes[hi], codes[lo]).astype(np.uint8)
    code = np.where(mag == values[hi], codes[hi], code).astype(np.uint8)   # exact hits
    sign = np.signbit(a)
    return np.where(sign, code | np.uint8(0x80), code).astype(np.uint8)
