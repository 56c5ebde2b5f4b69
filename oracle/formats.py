"""Number formats the cache stores, written from their published definitions.

bfloat16: 1 sign, 8 exponent (bias 127), 7 stored mantissa bits; rounding to
nearest, ties to even.  OCP 8-bit floating point, E4M3 ("fn") variant: 1 sign,
4 exponent (bias 7), 3 mantissa bits, no infinities, NaN = S.1111.111, largest
finite 448, smallest subnormal 2^-9.  Conversion here rounds to nearest even
and saturates to +-448 (the pages require a K/V scale of 1 for the fused
materialisation path, CSDN article, fused_kv_materialize enabling conditions).

Rounding is done on the exact (fp64) value, never via an intermediate fp32.
"""
import numpy as np


def _round_to_spacing(x, mant_bits, min_exp):
    """Nearest multiple of 2^(E - mant_bits), E = max(floor(log2|x|), min_exp), ties to even."""
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)                      # x = m * 2^e, 0.5 <= |m| < 1
    E = np.maximum(e - 1, min_exp)          # exponent of the leading bit, clamped to normals
    q = np.ldexp(np.rint(np.ldexp(x, -(E - mant_bits))), E - mant_bits)  # np.rint: ties to even
    return np.where(x == 0, x, q)       # keeps the sign of zero


def round_bf16(x):
    """fp64 -> nearest bfloat16 value (as fp64)."""
    return _round_to_spacing(x, 7, -126)


def round_e4m3(x):
    """fp64 -> nearest E4M3 value (as fp64), saturating at +-448."""
    q = _round_to_spacing(x, 3, -6)
    return np.clip(q, -448.0, 448.0)


def e4m3_decode(codes):
    """uint8 E4M3 codes -> fp64 values (NaN for S.1111.111)."""
    c = np.asarray(codes, dtype=np.int64)
    s = np.where(c >> 7, -1.0, 1.0)
    e = (c >> 3) & 15
    m = c & 7
    val = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    val = np.where((e == 15) & (m == 7), np.nan, val)
    return s * val


def e4m3_encode(x):
    """fp64 -> uint8 E4M3 codes (round to nearest even, saturate)."""
    v = round_e4m3(x)
    a = np.abs(v)
    sign = np.where(np.signbit(v), 128, 0)
    mm, ee = np.frexp(a)
    E = ee - 1
    normal = a >= 2.0 ** -6
    e_field = np.where(normal, E + 7, 0)
    m_field = np.where(normal, np.rint((a / np.exp2(E) - 1.0) * 8.0), np.rint(a * 2.0 ** 9))
    code = np.where(a == 0, 0, e_field * 8 + m_field)
    return (sign + code).astype(np.uint8)


def round_kv(x, kv_dtype: str):
    """The storage rounding Q_kv applied when K/V enter the cache."""
    if kv_dtype == "f32":
        return np.asarray(x, np.float64).astype(np.float32).astype(np.float64)
    if kv_dtype == "bf16":
        return round_bf16(x)
    if kv_dtype == "fp8_e4m3":
        return round_e4m3(x)
    raise ValueError(kv_dtype)
