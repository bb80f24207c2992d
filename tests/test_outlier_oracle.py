"""Pins of the oracle's outlier-aware key quantization (static smoothing, per-block scale search).

The scale search is checked against an exact-arithmetic brute force (Python fractions over every
candidate scale) and against its defining invariant (never worse than round-to-nearest); the
smoothing against its exponent definition and the exactness of QK^T.
"""
import math
from fractions import Fraction

import numpy as np

import bruteforce as bf
import workloads as W
from oracle import formats as F
from oracle import outlier as O
from oracle import quant as Q


def _bf_mx_block(vals):
    """Best exponent for one 32-element block by exact errors over the candidates {e_rtn, e_rtn - 1}."""
    e0 = bf.mx_exponent(max(abs(v) for v in vals))
    best = None
    for e in (e0, e0 - 1):
        if e < -127:
            continue
        err = sum((Fraction(v) - Fraction(bf.e2m1_value(bf.e2m1_encode(v * 2.0 ** -e))) * Fraction(2) ** e) ** 2
                  for v in vals)
        if best is None or err < best[1]:
            best = (e, err)
    return best[0]


def _bf_nv_block(vals, st):
    """Best E4M3 block-scale code for one 16-element block by exact errors over the candidates."""
    six_st = bf.f32(6.0 * st)
    c0 = bf.e4m3_encode(bf.f32(max(abs(v) for v in vals) / six_st))
    if c0 == 0:
        return 0
    best = None
    for c in (c0, c0 - 1, c0 + 1, c0 - 2):
        if not 1 <= c <= 126:
            continue
        denom = bf.f32(bf.e4m3_value(c) * st)
        err = Fraction(0)
        for v in vals:
            code = bf.e2m1_encode(bf.f32(v / denom))
            err += (Fraction(v) - Fraction(bf.e2m1_value(code)) * Fraction(bf.e4m3_value(c)) * Fraction(st)) ** 2
        if best is None or err < best[1]:
            best = (c, err)
    return best[0]


def _rows(seed, n, outliers=True):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((n, 128)).astype(np.float32)
    if outliers:
        x[:, rng.permutation(128)[:4]] *= 20.0
    x[0, :32] = 0.0                                          # an all-zero MX block
    x[1, :32] = np.float32([0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0, -6.0] * 4)   # exactly on the grid
    return x


def test_mx_search_matches_exact_bruteforce():
    x = _rows(0, 24)
    codes, scales = O.mxfp4_quantize_search(x)
    for r in range(x.shape[0]):
        for b in range(4):
            vals = [float(v) for v in x[r, 32 * b:32 * b + 32]]
            assert int(scales[r, b]) - 127 == _bf_mx_block(vals), (r, b)
    # codes follow from the chosen scales
    un = F.unpack_nibbles(codes)
    for r in range(4):
        for i in range(128):
            e = int(scales[r, i // 32]) - 127
            assert un[r, i] == bf.e2m1_encode(float(x[r, i]) * 2.0 ** -e)
    assert scales[0, 0] == 0 and scales[1, 0] == Q.mxfp4_quantize(x[1:2])[1][0, 0]


def test_nv_search_matches_exact_bruteforce():
    x = _rows(1, 12)[None]
    codes, sb, st = O.nvfp4_quantize_search(x)
    _, sb0, st0 = Q.nvfp4_quantize(x)
    assert np.array_equal(st, st0)                               # the tensor scale is not searched
    for r in range(x.shape[1]):
        for b in range(8):
            vals = [float(v) for v in x[0, r, 16 * b:16 * b + 16]]
            assert sb[0, r, b] == _bf_nv_block(vals, float(st[0])), (r, b)
    assert sb[0, 0, 0] == 0 and sb[0, 0, 1] == 0                 # zero blocks keep the zero scale


def test_search_never_worse_than_round_to_nearest():
    cfg = W.C4.scaled(Hq=2, Hkv=2, Lq=128, Lk=256)
    _, k, _ = W.prefill_inputs(cfg)
    x = k.float().numpy().reshape(2, 256, 128).astype(np.float64)
    xr = Q.hadamard_rotate(x)
    for data in (x, xr):
        c, s, t = O.nvfp4_quantize_search(data)
        c0, s0, t0 = Q.nvfp4_quantize(data)
        e = (Q.nvfp4_dequantize(c, s, t) - data) ** 2
        e0 = (Q.nvfp4_dequantize(c0, s0, t0) - data) ** 2
        assert np.all(e.reshape(2, 256, 8, 16).sum(-1) <= e0.reshape(2, 256, 8, 16).sum(-1) * (1 + 1e-12))
        assert e.sum() < e0.sum()
        cm, sm = O.mxfp4_quantize_search(data)
        cm0, sm0 = Q.mxfp4_quantize(data)
        em = (Q.mxfp4_dequantize(cm, sm) - data) ** 2
        em0 = (Q.mxfp4_dequantize(cm0, sm0) - data) ** 2
        assert np.all(em.reshape(2, 256, 4, 32).sum(-1) <= em0.reshape(2, 256, 4, 32).sum(-1) * (1 + 1e-12))


def test_smoothing_exponents_definition():
    rng = np.random.default_rng(2)
    aq = (np.abs(rng.standard_normal((8, 128))) * np.exp2(rng.integers(-30, 30, (8, 128)))).astype(np.float32)
    ak = (np.abs(rng.standard_normal((2, 128))) * np.exp2(rng.integers(-30, 30, (2, 128)))).astype(np.float32)
    aq[0, 0] = 0.0
    ak[1, 5] = 0.0
    k = O.smoothing_exponents(aq, ak, 4)
    for h in range(2):
        for c in range(128):
            q = max(float(aq[4 * h + j, c]) for j in range(4))
            kk = float(ak[h, c])
            if q == 0 or kk == 0:
                assert k[h, c] == 0
                continue
            eq, ek = math.frexp(q)[1] - 1, math.frexp(kk)[1] - 1
            want = max(-20, min(20, (ek - eq + 1) // 2))
            assert k[h, c] == want
            # 2^k is within a factor 2^(3/4)... of sqrt(kk / q): the exponents bound both maxima within 2x
            assert abs(2 * k[h, c] - math.log2(kk / q)) <= 3.0 or abs(k[h, c]) == 20


def test_smoothing_keeps_qk_exact_and_cuts_logit_error():
    """Powers of two keep QK^T exact; on keys with x20 outlier channels, smoothing (with the Hadamard
    rotation off) lowers the NVFP4 logit error, and the scale search lowers it further."""
    cfg = W.C4.scaled(Hq=4, Hkv=1, Lq=256, Lk=512)
    q, k, _ = W.prefill_inputs(cfg)
    qf = q.float().numpy().astype(np.float64)
    kf = k.float().numpy().astype(np.float64)
    qs, ks = O.smoothing_factors(qf[:, :, :128], kf[:, :, :256])        # static: from a calibration prefix
    assert np.all(np.log2(qs) == np.round(np.log2(qs))) and np.array_equal(qs[0], 1.0 / ks[0])
    q2 = qf * qs[None, :, None, :]
    k2 = kf * np.repeat(ks, 4, axis=0)[None, :1, None, :]
    ref = qf[0] @ kf[0, 0].T
    assert np.array_equal(q2[0] @ k2[0, 0].T, ref)
    def logit_err(qx, kx, quant):
        cq, sq, tq = quant(qx.reshape(4, 256, 128))
        ck, sk, tk = quant(kx.reshape(1, 512, 128))
        got = Q.nvfp4_dequantize(cq, sq, tq) @ Q.nvfp4_dequantize(ck, sk, tk)[0].T
        return np.linalg.norm(got - ref) / np.linalg.norm(ref)
    e_rtn = logit_err(qf, kf, Q.nvfp4_quantize)
    e_smooth = logit_err(q2, k2, Q.nvfp4_quantize)
    e_both = logit_err(q2, k2, O.nvfp4_quantize_search)
    assert e_smooth < 0.9 * e_rtn and e_both < e_smooth


def _tiny_groups():
    """Groups whose tensor maximum is subnormal: 1e-42 (fl32(amax / 2688) underflows to zero) and
    1e-39, 3e-40 (the quotient is a representable subnormal), plus one normal group."""
    rng = np.random.default_rng(11)
    g = []
    for amax in (1e-42, 1e-39, 3e-40, 1e-30):
        x = rng.standard_normal((6, 128))
        x = x / np.abs(x).max() * amax
        g.append(x.astype(np.float32))
    return np.stack(g).astype(np.float64)


def test_nv_search_tensor_scale_zero_rule():
    """The search path takes the tensor scale of nvfp4_quantize: 1 when fl32(amax / 2688) is zero.
    With a maximum of 1e-42 the quotient underflows, so the group quantizes as an all-zero one (zero
    block scales, signed-zero codes) instead of dividing by a zero scale; the other groups keep
    their round-to-nearest tensor scale and match the exact brute force block by block."""
    x = _tiny_groups()
    assert np.float32(1e-42) / np.float32(2688) == 0 and np.float32(1e-39) / np.float32(2688) > 0
    codes, sb, st = O.nvfp4_quantize_search(x)
    _, _, st0 = Q.nvfp4_quantize(x)
    assert np.array_equal(st, st0) and st[0] == 1.0 and np.all(st[1:] < 1e-30)
    assert np.all(sb[0] == 0)
    u = F.unpack_nibbles(codes)[0]
    assert np.array_equal(u, np.signbit(x[0]).astype(np.int64) << 3)
    for g in range(x.shape[0]):
        _, _, bst = bf.nvfp4_group([[float(v) for v in r] for r in x[g]])
        assert bf.f32(bst) == float(st[g])
        for r in range(x.shape[1]):
            for b in range(8):
                vals = [float(v) for v in x[g, r, 16 * b:16 * b + 16]]
                assert sb[g, r, b] == _bf_nv_block(vals, float(st[g])), (g, r, b)
    assert not np.any((sb & 0x7F) == 0x7F)
    assert np.all(np.isfinite(Q.nvfp4_dequantize(codes, sb, st)))
