"""Block-scaled quantizers of the oracle (MXFP4, NVFP4, FP8 per token, dual residual, Hadamard).

TEST INFRASTRUCTURE: only the tests, the smoke check and the benchmark's
CPU-baseline leg may use this module. Shares no code with the GPU path.

All arithmetic is float64 except at the rounding points named in each
function, where a value is rounded to float32 (numpy float32 operations are
IEEE round-to-nearest-even, division included).

Sources:
  * "General notes on quantization" (zdszero), the general model: a tensor is
    approximated as X ~ s_X * Q_X with per-tensor, per-token or per-group
    scales (granularity table).
  * "MXFP vs NVFP4" (tqpw.cn 81738) sections 2.1-2.2: MXFP4 blocks of 32 with
    an E8M0 scale; NVFP4 blocks of 16 with an E4M3 scale plus an FP32 tensor
    scale (the three-level element / block / tensor hierarchy).
  * "BitDecoding-FP4" (sns.style digest): dual-residual query quantization
    (q ~ Q1 + Q2, Q2 carries Q1's residual) and a Hadamard rotation of keys
    before quantization.
  * "MpFA QK4V8" (hotelren.com 6111405) section 5.1: a zero block maximum must
    not produce a zero scale (no division by zero).

Readings taken where the pages leave the step open: MXFP4's scale is the
smallest power of two 2^e with 6*2^e >= amax (scale = amax/6 rounded up to a
power of two, so nothing saturates); NVFP4's tensor scale is amax/(6*448) so
that the largest block scale lands at 448, and the block scale is the E4M3
rounding of amax_b / (6*s_t); FP8 V uses one float32 scale amax/448 per token;
zero maxima give the neutral scales listed per function.
"""
import numpy as np

from .formats import (E2M1_MAX, E4M3_MAX, e2m1_decode, e2m1_encode, e4m3_decode,
                      e4m3_encode, fp32, pack_nibbles, unpack_nibbles)

MX_BLOCK = 32
NV_BLOCK = 16


# ----------------------------------------------------------------------------- MXFP4

def mx_scale_exponent(amax):
    """Smallest integer e with 6 * 2^e >= amax, clamped to [-127, 127]; -127 for amax == 0.

    Closed form: write amax = f * 2^E with f in [0.5, 1). Then 6*2^e >= amax
    holds for e >= E - 3 + log2(8f/6); with 8f in [4, 8) this is e = E-3 when
    f <= 0.75 and e = E-2 otherwise. (The tests check this against the
    definition by direct search.)
    """
    amax = np.asarray(amax, dtype=np.float64)
    f, E = np.frexp(amax)
    e = np.where(f <= 0.75, E - 3, E - 2)
    e = np.where(amax == 0, -127, e)
    return np.clip(e, -127, 127).astype(np.int64)


def mxfp4_quantize(x):
    """MXFP4-quantize the last axis of x (length a multiple of 32).

    Returns (codes [..., d/2] uint8 packed, scales [..., d/32] uint8 E8M0).
    Per block: amax = max |x|; e = mx_scale_exponent(amax); element code =
    E2M1(x * 2^-e) (the multiply by a power of two is exact).
    """
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    assert d % MX_BLOCK == 0
    blocks = x.reshape(x.shape[:-1] + (d // MX_BLOCK, MX_BLOCK))
    amax = np.max(np.abs(blocks), axis=-1)
    e = mx_scale_exponent(amax)
    scaled = blocks * np.ldexp(1.0, -e)[..., None]
    codes = e2m1_encode(scaled).reshape(x.shape)
    return pack_nibbles(codes), (e + 127).astype(np.uint8)


def mxfp4_dequantize(codes, scales):
    """Inverse map: value = E2M1(code) * 2^(scale-127), float64."""
    c = unpack_nibbles(codes)
    d = c.shape[-1]
    v = e2m1_decode(c).reshape(c.shape[:-1] + (d // MX_BLOCK, MX_BLOCK))
    s = np.ldexp(1.0, np.asarray(scales, dtype=np.int64) - 127)
    return (v * s[..., None]).reshape(c.shape)


# ----------------------------------------------------------------------------- MXFP8

def mx8_scale_exponent(amax):
    """Smallest integer e with 448 * 2^e >= amax, clamped to [-127, 127]; -127 for amax == 0.

    Closed form: with amax = f * 2^E, f in [0.5, 1), 448 * 2^e >= amax holds for
    e >= E + log2(f / 448); 448 = 0.875 * 2^9, so e = E - 9 when f <= 0.875 and
    e = E - 8 otherwise. (The tests check it against the definition by search.)
    """
    amax = np.asarray(amax, dtype=np.float64)
    f, E = np.frexp(amax)
    e = np.where(f <= 0.875, E - 9, E - 8)
    e = np.where(amax == 0, -127, e)
    return np.clip(e, -127, 127).astype(np.int64)


def mxfp8_quantize(x):
    """MXFP8 (E4M3 elements) of the last axis of x (length a multiple of 32).

    "MXFP vs NVFP4" (tqpw.cn 81738) section 2.1 (the MX family: 32-element blocks with an E8M0
    scale, FP8 E4M3 elements) and section 4.2 (Q and K in MXFP8). Reading, as for MXFP4: the scale is
    the smallest power of two 2^e with 448 * 2^e >= amax (nothing saturates); codes = E4M3(x * 2^-e)
    (the scaling is exact), round to nearest even.
    Returns (codes [..., d] uint8, scales [..., d/32] uint8 E8M0).
    """
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    assert d % MX_BLOCK == 0
    blocks = x.reshape(x.shape[:-1] + (d // MX_BLOCK, MX_BLOCK))
    e = mx8_scale_exponent(np.max(np.abs(blocks), axis=-1))
    codes = e4m3_encode(blocks * np.ldexp(1.0, -e)[..., None]).reshape(x.shape)
    return codes.astype(np.uint8), (e + 127).astype(np.uint8)


def mxfp8_dequantize(codes, scales):
    """value = E4M3(code) * 2^(scale-127), float64."""
    c = np.asarray(codes)
    d = c.shape[-1]
    v = e4m3_decode(c).reshape(c.shape[:-1] + (d // MX_BLOCK, MX_BLOCK))
    s = np.ldexp(1.0, np.asarray(scales, dtype=np.int64) - 127)
    return (v * s[..., None]).reshape(c.shape)


def mxfp4_keys_quantize(v):
    """4-bit V for prefill: MXFP4 of v [..., L, d] with its 32-element blocks along L (the key axis),
    i.e. MXFP4 of the transposed rows v^T [..., d, L]. Returns (codes [..., d, L/2], E8M0 scales
    [..., d, L/32]); element 2i of a code row in the low nibble, as for any MXFP4 row."""
    return mxfp4_quantize(np.swapaxes(np.asarray(v, dtype=np.float64), -1, -2))


def mxfp4_keys_dequantize(codes, scales):
    """Values [..., L, d] of mxfp4_keys_quantize's output (exact)."""
    return np.swapaxes(mxfp4_dequantize(codes, scales), -1, -2)


# ----------------------------------------------------------------------------- NVFP4

def nvfp4_quantize(x):
    """NVFP4-quantize x of shape [G, R, d]: one tensor scale per group g.

    Steps (float32 rounding points marked fl32):
      1. amax_t = max |x| over the group; s_t = fl32(amax_t / 2688), 2688 = 6*448;
         s_t = 1 when that is zero (amax_t == 0, or so small that the quotient underflows: the
         tensor then quantizes like an all-zero one, every block scale rounding to zero).
      2. per block of 16 along d: r = fl32(amax_b / fl32(6 * s_t)); block scale
         s_b = E4M3(r) (nearest-even, saturating at 448).
      3. denom = fl32(E4M3value(s_b) * s_t); element code = E2M1(fl32(x / denom)),
         saturating at +-6. A block whose scale rounds to zero keeps only the
         signs (codes are signed zeros).
    Returns (codes [G,R,d/2] uint8, block_scales [G,R,d/16] uint8, tensor_scales [G] float32).
    """
    x = np.asarray(x, dtype=np.float64)
    G, R, d = x.shape
    assert d % NV_BLOCK == 0
    x32 = fp32(x)
    amax_t = np.max(np.abs(x32).reshape(G, -1), axis=1).astype(np.float32) if R > 0 else np.zeros(G, np.float32)
    s_t = (amax_t / np.float32(6.0 * E4M3_MAX)).astype(np.float32)
    s_t = np.where(s_t == 0, np.float32(1.0), s_t).astype(np.float32)
    blocks = x32.reshape(G, R, d // NV_BLOCK, NV_BLOCK)
    amax_b = np.max(np.abs(blocks), axis=-1).astype(np.float32)
    six_st = (np.float32(6.0) * s_t).astype(np.float32)
    r = (amax_b / six_st[:, None, None]).astype(np.float32)
    s_b = e4m3_encode(r).astype(np.uint8)
    denom = (e4m3_decode(s_b).astype(np.float32) * s_t[:, None, None]).astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        q = (blocks / denom[..., None]).astype(np.float32)
    codes = e2m1_encode(q)
    zero_blk = (s_b == 0)[..., None]
    codes = np.where(zero_blk, np.signbit(blocks).astype(np.int64) << 3, codes)
    return pack_nibbles(codes.reshape(G, R, d)), s_b, s_t


def nvfp4_dequantize(codes, block_scales, tensor_scales):
    """value = E2M1(code) * E4M3(s_b) * s_t, exact in float64 (6 x 24 significant bits)."""
    c = unpack_nibbles(codes)
    G, R, d = c.shape
    v = e2m1_decode(c).reshape(G, R, d // NV_BLOCK, NV_BLOCK)
    sb = e4m3_decode(block_scales)
    st = np.asarray(tensor_scales, dtype=np.float64)
    return (v * sb[..., None] * st[:, None, None, None]).reshape(G, R, d)


def dual_residual_quantize(q):
    """q ~ Q1 + Q2 with both NVFP4: Q1 = NVFP4(q), r = fl32(q - dequant(Q1)), Q2 = NVFP4(r).

    Each residual has its own tensor scale (per group). The subtraction is done
    in float64 (exact here) and rounded once to float32.
    Returns ((codes1, sb1, st1), (codes2, sb2, st2)).
    """
    q32 = fp32(q).astype(np.float64)
    c1, sb1, st1 = nvfp4_quantize(q32)
    r = fp32(q32 - nvfp4_dequantize(c1, sb1, st1)).astype(np.float64)
    c2, sb2, st2 = nvfp4_quantize(r)
    return (c1, sb1, st1), (c2, sb2, st2)


def dual_residual_quantize_mx(q):
    """q ~ Q1 + Q2 with both MXFP4: Q1 = MXFP4(q), r = fl32(q - dequant(Q1)), Q2 = MXFP4(r).

    The query of an MXFP4 KV cache ("BitDecoding-FP4": the query is split into two FP4 tensors of
    the cache's format, the second carrying the first one's residual). No tensor scales.
    Returns ((codes1, scales1), (codes2, scales2)).
    """
    q32 = fp32(q).astype(np.float64)
    c1, s1 = mxfp4_quantize(q32)
    r = fp32(q32 - mxfp4_dequantize(c1, s1)).astype(np.float64)
    c2, s2 = mxfp4_quantize(r)
    return (c1, s1), (c2, s2)


# ----------------------------------------------------------------------------- FP8 V per token

def fp8_per_token_quantize(v):
    """V -> E4M3 codes with one float32 scale per token (row).

    s_v = fl32(amax_row / 448) (1 when amax_row == 0); code = E4M3(fl32(v / s_v)).
    Returns (codes [..., d] uint8, s_v [...] float32).
    """
    v32 = fp32(v)
    amax = np.max(np.abs(v32), axis=-1).astype(np.float32)
    s_v = np.where(amax == 0, np.float32(1.0), amax / np.float32(E4M3_MAX)).astype(np.float32)
    q = (v32 / s_v[..., None]).astype(np.float32)
    return e4m3_encode(q).astype(np.uint8), s_v


def fp8_per_token_dequantize(codes, s_v):
    return e4m3_decode(codes) * np.asarray(s_v, dtype=np.float64)[..., None]


# ----------------------------------------------------------------------------- Hadamard

def sylvester_hadamard(n):
    """Sylvester construction: H_1 = [1], H_2k = [[H, H], [H, -H]] (symmetric, entries +-1)."""
    H = np.ones((1, 1), dtype=np.float64)
    while H.shape[0] < n:
        H = np.block([[H, H], [H, -H]])
    assert H.shape[0] == n
    return H


def hadamard_rotate(x, n=128):
    """x' = fl32((x @ H_n) * (1/sqrt(n))) on the last axis, products and sums in float64.

    The rotation is orthonormal, so dot products between rotated rows equal
    those of the originals; it spreads a large channel over all channels
    before quantization (outlier-aware key quantization).
    """
    x = np.asarray(x, dtype=np.float64)
    assert x.shape[-1] == n
    y = x @ sylvester_hadamard(n)
    return fp32(y * (1.0 / np.sqrt(np.float64(n)))).astype(np.float64)


# ----------------------------------------------------------------------------- row norms

def row_norm2(x):
    """Squared L2 norm of each row, float64, summed as a balanced binary tree over d, rounded to float32.

    Level 0 adds the squares of elements (2i, 2i+1), each next level adds
    neighbouring partial sums, until one sum is left (d is a power of two).
    The squares of float32/bf16 inputs are exact in float64; fixing the tree
    makes the rounded result one defined number.
    """
    x = fp32(x).astype(np.float64)
    s = x * x
    while s.shape[-1] > 1:
        s = s[..., 0::2] + s[..., 1::2]
    return fp32(s[..., 0])
