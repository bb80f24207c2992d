"""Number formats of block-scaled low-bit attention, written from their definitions.

TEST INFRASTRUCTURE. This module is part of the CPU oracle: only the tests,
the smoke check and the benchmark's CPU-baseline leg may import it. It shares
no code with the GPU path.

Sources (pages of the reference set):
  * "General notes on quantization" (zdszero, quantization.html), format table:
    bf16 = 1-8-7, fp16 = 1-5-10, e4m3 = 1-4-3, e5m2 = 1-5-2, e2m1 = 1-2-1
    sign-exponent-mantissa bits; E8M0 is listed there with a sign bit, which is
    an error of that table: a pure exponent byte has none (read as 0-8-0).
  * "MXFP vs NVFP4" (tqpw.cn news 81738), sections 2.1-2.2: MXFP4 = E2M1
    elements, 32-element blocks, E8M0 block scale; NVFP4 = E2M1 elements,
    16-element blocks, E4M3 block scale, an FP32 tensor scale.

Every encoder here rounds to nearest with ties to the even code (the code whose
mantissa LSB is 0). For both E2M1 and E4M3 the non-negative codes are ordered
by value, so "nearest value, ties to even code" is computed by locating the
input between two neighbouring codes of the value table.

Readings taken where the pages are silent (listed with the others in the
design notes): the sign of a code is the sign bit of the input (so -0 and tiny
negatives give the negative-zero code); values beyond the largest finite
magnitude saturate to it; E4M3 is the OCP "fn" variant (no infinities, 0x7F
and 0xFF are NaN and are never produced); 4-bit codes are packed two per byte
with element 2i in bits 3:0 and element 2i+1 in bits 7:4.
"""
import numpy as np

__all__ = [
    "E2M1_MAG", "E4M3_MAG", "E4M3_MAX", "E2M1_MAX",
    "e2m1_decode", "e2m1_encode", "e4m3_decode", "e4m3_encode",
    "e8m0_decode", "bf16_round", "fp32", "pack_nibbles", "unpack_nibbles",
]


def _minifloat_magnitudes(exp_bits, man_bits, bias, n_codes):
    """Value of each non-negative code of a sign/exponent/mantissa minifloat.

    Exponent field 0 is subnormal: m * 2^(1-bias-man_bits); otherwise the value
    is 2^(e-bias) * (1 + m / 2^man_bits).
    """
    vals = []
    for c in range(n_codes):
        e = c >> man_bits
        m = c & ((1 << man_bits) - 1)
        if e == 0:
            v = m * 2.0 ** (1 - bias - man_bits)
        else:
            v = 2.0 ** (e - bias) * (1.0 + m / 2.0 ** man_bits)
        vals.append(v)
    return np.array(vals, dtype=np.float64)


# E2M1: 1 sign, 2 exponent (bias 1), 1 mantissa bit -> 8 magnitudes.
E2M1_MAG = _minifloat_magnitudes(2, 1, 1, 8)
E2M1_MAX = float(E2M1_MAG[-1])
# E4M3 (OCP fn): 1 sign, 4 exponent (bias 7), 3 mantissa bits; magnitude code
# 0x7F is NaN, so the finite magnitudes are codes 0..126 and the largest is 448.
E4M3_MAG = _minifloat_magnitudes(4, 3, 7, 127)
E4M3_MAX = float(E4M3_MAG[-1])


def fp32(x):
    """Round a float64 array to float32 (IEEE round to nearest even)."""
    return np.asarray(x, dtype=np.float64).astype(np.float32)


def _round_to_table(a, table):
    """Index of the nearest table entry to a >= 0, ties to the even index.

    `table` is strictly increasing and starts at 0; inputs above the last entry
    saturate to it.
    """
    a = np.asarray(a, dtype=np.float64)
    hi = np.searchsorted(table, a, side="left")          # first index with table[hi] >= a
    hi = np.minimum(hi, len(table) - 1)
    lo = np.maximum(hi - 1, 0)
    d_lo = a - table[lo]
    d_hi = table[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    idx = np.where(pick_hi, hi, lo)
    idx = np.where(a >= table[-1], len(table) - 1, idx)   # saturation
    return idx.astype(np.int64)


def _sign_bit(x):
    return np.signbit(np.asarray(x)).astype(np.int64)


def e2m1_decode(code):
    """4-bit code -> value: bit 3 is the sign, bits 2:0 index E2M1_MAG."""
    code = np.asarray(code, dtype=np.int64)
    mag = E2M1_MAG[code & 7]
    return np.where(code & 8, -mag, mag)


def e2m1_encode(x):
    """Round each value to the nearest E2M1 code (ties to even, saturating at +-6)."""
    x = np.asarray(x, dtype=np.float64)
    return (_sign_bit(x) << 3) | _round_to_table(np.abs(x), E2M1_MAG)


def e4m3_decode(code):
    """8-bit OCP E4M3 code -> value (NaN for 0x7F / 0xFF)."""
    code = np.asarray(code, dtype=np.int64)
    mag_code = code & 0x7F
    mag = np.where(mag_code == 0x7F, np.nan, E4M3_MAG[np.minimum(mag_code, 126)])
    return np.where(code & 0x80, -mag, mag)


def e4m3_encode(x):
    """Round each value to the nearest E4M3 code (ties to even, saturating at +-448)."""
    x = np.asarray(x, dtype=np.float64)
    return (_sign_bit(x) << 7) | _round_to_table(np.abs(x), E4M3_MAG)


def e8m0_decode(code):
    """E8M0 scale byte -> 2^(code-127) (code 255 is NaN and never produced here)."""
    code = np.asarray(code, dtype=np.int64)
    return np.ldexp(1.0, code - 127)


def bf16_round(x):
    """Round values to bfloat16 (8 significant bits, float32's exponent range), nearest-even.

    With x = f * 2^E, f in [0.5, 1), the bf16 grid near x has spacing
    2^(E-8) (the exponent is floored at the float32/bf16 minimum, which makes
    the subnormal spacing 2^-133); the result is rint(x / spacing) * spacing,
    and numpy's rint rounds halves to even. Returned as float64.
    """
    x = np.asarray(x, dtype=np.float64)
    _, E = np.frexp(x)
    E = np.maximum(E, -125)
    q = np.ldexp(1.0, E - 8)
    return np.rint(x / q) * q


def pack_nibbles(codes):
    """[..., 2n] 4-bit codes -> [..., n] bytes; element 2i in the low nibble."""
    codes = np.asarray(codes, dtype=np.int64)
    return (codes[..., 0::2] | (codes[..., 1::2] << 4)).astype(np.uint8)


def unpack_nibbles(packed):
    """[..., n] bytes -> [..., 2n] 4-bit codes (inverse of pack_nibbles)."""
    p = np.asarray(packed, dtype=np.int64)
    out = np.empty(p.shape[:-1] + (2 * p.shape[-1],), dtype=np.int64)
    out[..., 0::2] = p & 0xF
    out[..., 1::2] = p >> 4
    return out
