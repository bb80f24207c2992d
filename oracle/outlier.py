"""Outlier-aware key quantization of the oracle: static per-channel smoothing and per-block scale search.

TEST INFRASTRUCTURE: only the tests, the smoke check and the benchmark's
CPU-baseline leg may use this module. Shares no code with the GPU path.

Source: "BitDecoding-FP4" (sns.style digest), outlier-aware key quantization:
static smoothing and the Hadamard rotation spread an outlier channel's energy,
and a scale search picks a better scale for each group. The page names these
parts but not their formulas; the readings taken here:

  * Smoothing factors, per (key head, channel c), from calibration maxima
    amax_K[c] (over the calibration tokens of the key head) and amax_Q[c] (over
    the tokens and the query heads of its group): with e = floor(log2 amax)
    (the binary exponent), k = floor((e_K - e_Q + 1) / 2), i.e. the square root
    of the ratio rounded to a power of two through exponents only, clamped to
    [-20, 20]; k = 0 when either maximum is zero. Keys are multiplied by 2^-k,
    queries by 2^k: both products are exact and QK^T is unchanged.
  * Scale search, per block: candidates around the round-to-nearest scale,
    each scored by the block's squared reconstruction error sum (x - x^)^2 in
    float64, summed as a balanced binary tree over the block's elements in
    index order; the first candidate in the listed order with the smallest
    error wins (so ties keep the round-to-nearest scale).
      MXFP4: exponents e_rtn, e_rtn - 1 (the smaller one clips the largest
             values at 6 * 2^(e-1) and refines the rest).
      NVFP4: E4M3 block-scale codes c_rtn, c_rtn - 1, c_rtn + 1, c_rtn - 2,
             those within [1, 126]; a zero round-to-nearest scale (an all-zero
             block relative to the tensor scale) is kept as is.
"""
import numpy as np

from .formats import e2m1_decode, e2m1_encode, e4m3_decode, e4m3_encode, fp32, pack_nibbles
from .quant import MX_BLOCK, NV_BLOCK, mx_scale_exponent

SMOOTH_CLAMP = 20


def _exponent(a):
    """floor(log2 a) for a > 0 (frexp: a = f 2^E, f in [0.5, 1) -> E - 1)."""
    return np.frexp(np.asarray(a, dtype=np.float64))[1] - 1


def smoothing_exponents(amax_q, amax_k, group):
    """k [Hkv, d] from amax_q [Hq, d] and amax_k [Hkv, d] (float32 maxima); group = Hq // Hkv."""
    amax_q = np.asarray(amax_q, dtype=np.float64)
    amax_k = np.asarray(amax_k, dtype=np.float64)
    Hkv, d = amax_k.shape
    aq = amax_q.reshape(Hkv, group, d).max(axis=1)
    ok = (aq > 0) & (amax_k > 0)
    eq = np.where(ok, _exponent(np.where(ok, aq, 1.0)), 0)
    ek = np.where(ok, _exponent(np.where(ok, amax_k, 1.0)), 0)
    k = np.floor_divide(ek - eq + 1, 2)
    return np.where(ok, np.clip(k, -SMOOTH_CLAMP, SMOOTH_CLAMP), 0).astype(np.int64)


def smoothing_factors(q_calib, k_calib):
    """(q_scale [Hq, d], k_scale [Hkv, d]) float32 from calibration tensors q [B, Hq, L, d] and
    k [B, Hkv, L, d]: channel maxima over batch and tokens, then 2^k and 2^-k."""
    q = fp32(q_calib).astype(np.float64)
    k = fp32(k_calib).astype(np.float64)
    Hq, Hkv = q.shape[1], k.shape[1]
    amax_q = np.abs(q).max(axis=(0, 2))
    amax_k = np.abs(k).max(axis=(0, 2))
    e = smoothing_exponents(amax_q, amax_k, Hq // Hkv)
    k_scale = np.ldexp(1.0, -e).astype(np.float32)
    q_scale = np.repeat(np.ldexp(1.0, e), Hq // Hkv, axis=0).astype(np.float32)
    return q_scale, k_scale


def tree_sum(t):
    """Balanced binary-tree sum over the last axis (length a power of two), in index order."""
    t = np.asarray(t, dtype=np.float64)
    while t.shape[-1] > 1:
        t = t[..., 0::2] + t[..., 1::2]
    return t[..., 0]


def _sse(x, xh):
    d = np.asarray(x, dtype=np.float64) - np.asarray(xh, dtype=np.float64)
    return tree_sum(d * d)


def mxfp4_quantize_search(x):
    """MXFP4 with the per-block scale search (see the module notes). x [..., d] (float32 values).
    Returns (codes [..., d/2], E8M0 scales [..., d/32])."""
    x = fp32(x).astype(np.float64)
    d = x.shape[-1]
    blocks = x.reshape(x.shape[:-1] + (d // MX_BLOCK, MX_BLOCK))
    e0 = mx_scale_exponent(np.max(np.abs(blocks), axis=-1))
    best_e = e0.copy()
    best_c = e2m1_encode(blocks * np.ldexp(1.0, -e0)[..., None])
    best_err = _sse(blocks, e2m1_decode(best_c) * np.ldexp(1.0, e0)[..., None])
    e1 = e0 - 1
    valid = e1 >= -127
    e1 = np.where(valid, e1, e0)
    c1 = e2m1_encode(blocks * np.ldexp(1.0, -e1)[..., None])
    err1 = _sse(blocks, e2m1_decode(c1) * np.ldexp(1.0, e1)[..., None])
    take = valid & (err1 < best_err)
    best_e = np.where(take, e1, best_e)
    best_c = np.where(take[..., None], c1, best_c)
    return pack_nibbles(best_c.reshape(x.shape)), (best_e + 127).astype(np.uint8)


def nvfp4_quantize_search(x):
    """NVFP4 with the per-block scale search. x [G, R, d]. The tensor scale is the round-to-nearest
    one, fl32(amax / 2688), or 1 when that quotient is zero (an all-zero group, or one whose maximum
    is so small that the quotient underflows: every block scale is then zero). Returns (codes, block
    scales, tensor scales) as nvfp4_quantize."""
    x = np.asarray(x, dtype=np.float64)
    G, R, d = x.shape
    x32 = fp32(x)
    amax_t = np.max(np.abs(x32).reshape(G, -1), axis=1).astype(np.float32) if R > 0 else np.zeros(G, np.float32)
    # the round-to-nearest tensor scale, with its zero rule: 1 when fl32(amax / 2688) is zero (amax == 0,
    # or a maximum so small that the quotient underflows), as in quant.nvfp4_quantize
    s_t = (amax_t / np.float32(6.0 * 448.0)).astype(np.float32)
    s_t = np.where(s_t == 0, np.float32(1.0), s_t).astype(np.float32)
    blocks = x32.reshape(G, R, d // NV_BLOCK, NV_BLOCK)
    amax_b = np.max(np.abs(blocks), axis=-1).astype(np.float32)
    six_st = (np.float32(6.0) * s_t).astype(np.float32)
    c0 = e4m3_encode((amax_b / six_st[:, None, None]).astype(np.float32)).astype(np.int64)
    stb = s_t[:, None, None]

    def attempt(c):
        denom = (e4m3_decode(c).astype(np.float32) * stb).astype(np.float32)
        with np.errstate(divide="ignore", invalid="ignore"):
            q = (blocks / denom[..., None]).astype(np.float32)
        codes = e2m1_encode(q)
        xh = e2m1_decode(codes) * e4m3_decode(c)[..., None] * stb[..., None].astype(np.float64)
        return codes, _sse(blocks, xh)

    best_s = c0.copy()
    best_c, best_err = attempt(np.maximum(c0, 1))
    for dc in (-1, 1, -2):
        c = c0 + dc
        valid = (c0 > 0) & (c >= 1) & (c <= 126)
        codes, err = attempt(np.clip(c, 1, 126))
        take = valid & (err < best_err)
        best_s = np.where(take, c, best_s)
        best_c = np.where(take[..., None], codes, best_c)
        best_err = np.where(take, err, best_err)
    zero_blk = (c0 == 0)[..., None]
    best_c = np.where(zero_blk, np.signbit(blocks).astype(np.int64) << 3, best_c)
    return pack_nibbles(best_c.reshape(G, R, d)), best_s.astype(np.uint8), s_t
