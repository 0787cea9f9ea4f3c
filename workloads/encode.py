"""Bit-exact encoders/decoders for the storage formats the kernel reads.

bfloat16: the upper 16 bits of an IEEE float32, rounded to nearest, ties to even.
OCP e4m3fn ("FN" = finite, NaN only): 1 sign bit, 4 exponent bits (bias 7), 3
mantissa bits; largest finite value 448 = 1.75 * 2**8, smallest normal 2**-6,
subnormal step 2**-9, no infinities, 0x7f/0xff are NaN.  Encoding rounds to
nearest-even and saturates magnitudes above 448 to 448.
"""

import numpy as np

E4M3FN_MAX = 448.0


def bf16_bits_from_f32(x):
    """float32 array -> uint16 bfloat16 bit patterns (round to nearest even)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    rounded = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        rounded[nan] = (((u[nan] >> 16) & 0x8000) | 0x7FC0).astype(np.uint16)
    return rounded


def bf16_bits_to_f64(bits):
    """uint16 bfloat16 bit patterns -> float64 values (exact)."""
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    with np.errstate(invalid="ignore"):            # signalling-NaN patterns stay NaN
        return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def e4m3fn_bits_from_f32(x):
    """float32 (or float64) array -> uint8 e4m3fn bits, RNE with saturation at +-448."""
    x = np.asarray(x)
    a = np.abs(x.astype(np.float64))
    sign = np.signbit(x).astype(np.uint8) << 7
    nan = np.isnan(a)
    a = np.where(nan, 0.0, np.minimum(a, E4M3FN_MAX))
    _, ex = np.frexp(a)                      # a = f * 2**ex, f in [0.5, 1)
    e = np.maximum(ex - 1, -6)               # binade exponent; subnormals share 2**-6's quantum
    quantum_exp = e - 3                      # 3 mantissa bits
    steps = np.rint(np.ldexp(a, -quantum_exp))   # exact scaling by a power of two, RNE
    q = np.ldexp(steps, quantum_exp)
    q = np.minimum(q, E4M3FN_MAX)
    # encode the rounded magnitude
    _, qe = np.frexp(q)
    eq = qe - 1
    normal = (q > 0) & (eq >= -6)
    exp_field = np.where(normal, eq + 7, 0)
    mant = np.where(normal, np.ldexp(q, -(eq - 3)) - 8, np.ldexp(q, 9))
    bits = (exp_field.astype(np.int64) << 3) | mant.astype(np.int64)
    bits = bits.astype(np.uint8) | sign
    bits = np.where(nan, sign | 0x7F, bits).astype(np.uint8)
    return bits


def e4m3fn_bits_to_f64(bits):
    """uint8 e4m3fn bits -> float64 values (exact); 0x7f/0xff -> NaN."""
    b = np.asarray(bits, dtype=np.uint8).astype(np.int64)
    s = np.where(b & 0x80, -1.0, 1.0)
    e = (b >> 3) & 0xF
    m = b & 0x7
    val = np.where(e == 0, np.ldexp(m.astype(np.float64), -9),
                   np.ldexp((8 + m).astype(np.float64), e - 10))
    val = np.where((b & 0x7F) == 0x7F, np.nan, val)
    return s * val
