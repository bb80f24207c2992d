"""Pins of the oracle's quantizers: closed forms vs definitions, round-trip bounds, brute force, invariants."""
import math
import os

import numpy as np
import torch

import bruteforce as bf
from oracle import formats as F
from oracle import quant as Q

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _blocks():
    out = {}
    for line in open(os.path.join(GOLDEN, "block_sizes.txt")):
        line = line.strip()
        if line and not line.startswith("#"):
            name, n, sfmt, tfmt = line.split()
            out[name] = (int(n), sfmt, tfmt)
    return out


def test_block_sizes_match_pages():
    b = _blocks()
    assert b["mxfp4"][0] == Q.MX_BLOCK and b["nvfp4"][0] == Q.NV_BLOCK


def test_mx_exponent_closed_form_vs_definition():
    """e(amax) == the smallest e with 6 * 2^e >= amax, over every float32 exponent and many mantissas."""
    rng = np.random.default_rng(0)
    amax = []
    for E in range(-149, 128):
        for m in list(rng.integers(0, 1 << 23, 64)) + [0, 1, (1 << 22), (1 << 23) - 1, 0x400000, 0x3FFFFF]:
            v = np.ldexp(1.0 + m / 2.0 ** 23, E) if E >= -126 else np.ldexp(float(m), -149)
            if 0 < v < 3.4e38:
                amax.append(v)
    amax = np.array(amax, dtype=np.float32).astype(np.float64)
    got = Q.mx_scale_exponent(amax)
    ref = np.array([bf.mx_exponent(float(a)) for a in amax])
    assert np.array_equal(got, ref)
    # exactly at 6 * 2^e the power e itself is chosen; just above it, e + 1
    for e in range(-100, 100):
        assert Q.mx_scale_exponent(6.0 * 2.0 ** e) == e
        assert Q.mx_scale_exponent(np.nextafter(np.float32(6.0 * 2.0 ** e), np.float32(np.inf))) == e + 1
    assert Q.mx_scale_exponent(0.0) == -127


def test_mx_scale_puts_block_max_in_3_to_6():
    rng = np.random.default_rng(1)
    x = (rng.standard_normal((4000, 32)) * np.exp2(rng.uniform(-20, 20, (4000, 1)))).astype(np.float32)
    codes, scales = Q.mxfp4_quantize(x)
    amax = np.abs(x).max(axis=1)
    e = scales[:, 0].astype(np.int64) - 127
    r = amax * np.exp2(-e.astype(np.float64))
    assert np.all(r > 3) and np.all(r <= 6)
    top = np.abs(F.e2m1_decode(F.unpack_nibbles(codes))).max(axis=1)
    assert set(np.unique(top).tolist()) <= {3.0, 4.0, 6.0}


def test_mxfp4_round_trip_bound():
    """|x - x^| <= 2^e * {0.25, 0.5, 1} in the bands |x 2^-e| <= 2, <= 4, <= 6 (X ~ s Q)."""
    rng = np.random.default_rng(2)
    x = (rng.standard_normal((2000, 128)) * np.exp2(rng.uniform(-8, 8, (2000, 1)))).astype(np.float32).astype(np.float64)
    codes, scales = Q.mxfp4_quantize(x)
    xh = Q.mxfp4_dequantize(codes, scales)
    s = np.repeat(np.exp2(scales.astype(np.int64) - 127.0), 32, axis=1)
    a = np.abs(x) / s
    bound = np.where(a <= 2, 0.25, np.where(a <= 4, 0.5, 1.0)) * s
    assert np.all(np.abs(x - xh) <= bound)


def test_mxfp4_vs_bruteforce():
    rng = np.random.default_rng(3)
    x = (rng.standard_normal((6, 64)) * np.array([1, 1e-3, 40, 0, 1e-39, 7])[:, None]).astype(np.float32)
    x[3] = 0.0
    x[5, :32] = -0.0
    codes, scales = Q.mxfp4_quantize(x)
    cu = F.unpack_nibbles(codes)
    for r in range(x.shape[0]):
        c, s = bf.mxfp4_row([float(v) for v in x[r]])
        assert cu[r].tolist() == c
        assert scales[r].tolist() == s


def test_nvfp4_vs_bruteforce_and_invariants():
    rng = np.random.default_rng(4)
    x = (rng.standard_normal((3, 5, 64)) * np.exp2(rng.uniform(-6, 6, (3, 5, 1)))).astype(np.float32)
    x[1, 2, 16:32] = 0.0
    x[2] *= 0.0
    codes, sb, st = Q.nvfp4_quantize(x)
    for g in range(3):
        c, s, t = bf.nvfp4_group([[float(v) for v in row] for row in x[g]])
        assert np.float32(t) == st[g]
        assert F.unpack_nibbles(codes[g]).tolist() == c
        assert sb[g].tolist() == s
    assert st[2] == 1.0 and np.all((F.unpack_nibbles(codes[2]) & 7) == 0)
    # the block holding the tensor maximum gets the largest scale code (448 = 0x7E) up to one step
    for g in range(2):
        top = sb[g].max()
        assert top in (0x7D, 0x7E)
    # reconstruction error is bounded by half a grid step at the block's scale, plus float32 slack
    xh = Q.nvfp4_dequantize(codes, sb, st)
    scale = (F.e4m3_decode(sb) * st[:, None, None]).repeat(16, axis=2)
    a = np.abs(x) / np.where(scale > 0, scale, 1)
    half = np.where(a <= 2, 0.25, np.where(a <= 4, 0.5, 1.0))
    over = np.maximum(a - 6, 0)                        # values above 6 * scale saturate
    ok = np.abs(x - xh) <= (half + over) * scale * (1 + 1e-6) + 1e-30
    assert np.all(ok | (scale == 0))


def test_nvfp4_idempotent():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((2, 4, 32)).astype(np.float32)
    c, sb, st = Q.nvfp4_quantize(x)
    xh = Q.nvfp4_dequantize(c, sb, st)
    c2, sb2, st2 = Q.nvfp4_quantize(xh)
    assert np.array_equal(Q.nvfp4_dequantize(c2, sb2, st2), xh)


def test_dual_residual_reduces_error():
    rng = np.random.default_rng(6)
    q = torch.randn(64, 1, 128, generator=torch.Generator().manual_seed(0)).to(torch.bfloat16).float().numpy()
    (c1, s1, t1), (c2, s2, t2) = Q.dual_residual_quantize(q)
    x1 = Q.nvfp4_dequantize(c1, s1, t1)
    x2 = Q.nvfp4_dequantize(c2, s2, t2)
    e1 = np.linalg.norm(q - x1, axis=-1)
    e2 = np.linalg.norm(q - x1 - x2, axis=-1)
    assert np.all(e2 <= e1)
    assert np.median(e2 / e1) < 0.25
    # query-logit error against random keys drops as well
    k = rng.standard_normal((1000, 128))
    l0 = q[:, 0] @ k.T
    r1 = np.linalg.norm(x1[:, 0] @ k.T - l0) / np.linalg.norm(l0)
    r2 = np.linalg.norm((x1 + x2)[:, 0] @ k.T - l0) / np.linalg.norm(l0)
    assert r2 < 0.25 * r1


def test_fp8_token_vs_torch():
    rng = np.random.default_rng(7)
    v = (rng.standard_normal((500, 128)) * np.exp2(rng.uniform(-10, 10, (500, 1)))).astype(np.float32)
    v[3] = 0.0
    codes, sv = Q.fp8_per_token_quantize(v)
    q = (v / sv[:, None]).astype(np.float32)
    ref = torch.from_numpy(q).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(codes, ref)
    assert sv[3] == 1.0 and np.all(codes[3] == 0)
    for r in range(4):
        c, s = bf.fp8_token([float(x) for x in v[r]])
        assert np.float32(s) == sv[r] and codes[r].tolist() == c
    # the largest element of every nonzero row maps to 448 (code 0x7E), possibly one step below
    top = codes[np.arange(500) != 3].astype(np.int64) & 0x7F
    assert set(np.unique(top.max(axis=1)).tolist()) <= {0x7D, 0x7E}


def test_hadamard_orthogonal_and_norm_preserving():
    H = Q.sylvester_hadamard(128)
    assert np.array_equal(H @ H.T, 128 * np.eye(128))
    assert np.array_equal(H, H.T)
    # recursive definition checked entry-wise: H[i, j] = (-1)^popcount(i & j)
    i = np.arange(128)
    assert np.array_equal(H, (-1.0) ** np.array([[bin(a & b).count("1") for b in i] for a in i]))
    rng = np.random.default_rng(8)
    x = torch.from_numpy(rng.standard_normal((50, 128)).astype(np.float32)).to(torch.bfloat16).double().numpy()
    y = Q.hadamard_rotate(x)
    assert np.allclose(np.linalg.norm(y, axis=1), np.linalg.norm(x, axis=1), rtol=1e-6)
    yy = x @ H / math.sqrt(128)
    assert np.allclose(yy @ yy.T, x @ x.T, rtol=1e-12, atol=1e-9)
    assert np.array_equal(y, yy.astype(np.float32).astype(np.float64))


def test_row_norm2_vs_exact_sum():
    rng = np.random.default_rng(9)
    x = torch.from_numpy((rng.standard_normal((3000, 128)) * 3).astype(np.float32)).to(torch.bfloat16).float().numpy()
    n = Q.row_norm2(x)
    exact = np.array([math.fsum(float(v) ** 2 for v in row) for row in x])
    assert np.array_equal(n, exact.astype(np.float32))


def test_zero_and_tiny_blocks_are_defined():
    x = np.zeros((1, 2, 64), dtype=np.float32)
    x[0, 1, :] = -0.0
    c, s = Q.mxfp4_quantize(x)
    assert np.all(s == 0) and np.all(F.unpack_nibbles(c)[0, 0] == 0) and np.all(F.unpack_nibbles(c)[0, 1] == 8)
    c, sb, st = Q.nvfp4_quantize(x)
    assert st[0] == 1.0 and np.all(sb == 0)
    v = np.full((1, 64), 1e-42, dtype=np.float32)
    c, s = Q.mxfp4_quantize(v)
    assert not np.any(np.isnan(Q.mxfp4_dequantize(c, s)))


def test_nvfp4_tensor_scale_underflow_is_a_zero_tensor():
    """When fl32(amax/2688) underflows to zero the tensor quantizes as an all-zero one: s_t = 1, every
    block scale 0, signed-zero codes. Across tiny magnitudes no block scale is ever an E4M3 NaN code
    (0x7F / 0xFF) and every dequantized value is finite."""
    x = np.zeros((1, 1, 32), dtype=np.float32)
    x[0, 0, :16] = np.float32(1e-42)
    x[0, 0, 16:] = np.float32(-1e-42)
    assert np.float32(1e-42) / np.float32(2688) == 0                 # the quotient underflows
    c, sb, st = Q.nvfp4_quantize(x)
    assert st[0] == 1.0 and np.all(sb == 0)
    u = F.unpack_nibbles(c)[0, 0]
    assert np.all(u[:16] == 0) and np.all(u[16:] == 8)
    rng = np.random.default_rng(3)
    for e in range(-160, -118, 2):
        t = (rng.standard_normal((4, 3, 32)) * 2.0 ** e).astype(np.float32)
        c, sb, st = Q.nvfp4_quantize(t)
        assert np.all(st > 0) and not np.any((sb & 0x7F) == 0x7F)
        assert np.all(np.isfinite(Q.nvfp4_dequantize(c, sb, st)))


def test_mx8_exponent_closed_form_vs_definition():
    """e(amax) == the smallest e with 448 * 2^e >= amax, over every float32 exponent and many mantissas."""
    rng = np.random.default_rng(1)
    amax = []
    for E in range(-149, 128):
        for m in list(rng.integers(0, 1 << 23, 32)) + [0, 1, 0x600000, 0x5FFFFF, 0x600001, (1 << 23) - 1]:
            v = np.ldexp(1.0 + m / 2.0 ** 23, E) if E >= -126 else np.ldexp(float(m), -149)
            if 0 < v < 3.4e38:
                amax.append(v)
    amax = np.array(amax, dtype=np.float32).astype(np.float64)
    got = Q.mx8_scale_exponent(amax)
    for a, e in zip(amax[::7], got[::7]):
        want = -127
        while 448.0 * 2.0 ** want < a and want < 127:
            want += 1
        assert e == want, (a, e, want)
    assert Q.mx8_scale_exponent(np.array([0.0]))[0] == -127


def test_mxfp8_codes_are_torch_e4m3_of_the_scaled_block():
    """Codes equal torch's float8_e4m3fn cast of x * 2^-e (a library routine, RNE), and every block's
    largest magnitude lands in (224, 448] (the top binade), so nothing saturates."""
    rng = np.random.default_rng(2)
    x = (rng.standard_normal((64, 128)) * np.exp2(rng.integers(-40, 40, (64, 4)).repeat(32, 1))).astype(np.float32)
    x[0, :32] = 0.0
    codes, scales = Q.mxfp8_quantize(x)
    e = scales.astype(np.int64) - 127
    scaled = x.astype(np.float64) * np.ldexp(1.0, -e).repeat(32, axis=1)
    ref = torch.from_numpy(scaled.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(codes, ref)
    am = np.abs(scaled).reshape(64, 4, 32).max(-1)
    assert np.all((am[am > 0] > 224) & (am[am > 0] <= 448)) and scales[0, 0] == 0
    back = Q.mxfp8_dequantize(codes, scales)
    rel = np.abs(back - x) / np.maximum(np.abs(x), 1e-300)
    assert np.all(rel[np.abs(x) >= np.ldexp(1.0, -6 + e.repeat(32, axis=1))] <= 2.0 ** -4)


def test_dual_residual_vs_bruteforce():
    """NVFP4 dual residual re-derived by the brute-force loops: Q1 = the group's NVFP4 by search over
    every code, x1 its exact value (Python doubles), r = fl32(q - x1) rounded once, Q2 = NVFP4(r) with
    its own tensor scale. Codes, block scales and tensor scales must equal the oracle's. Groups of
    several rows and of one row, bf16-valued and float32 inputs, and a row of special values."""
    rng = np.random.default_rng(21)
    q = rng.standard_normal((3, 4, 64)).astype(np.float32)
    q[1] = q[1].astype(np.float32) * np.float32(2.0 ** -20)
    q[2, 0, :16] = np.float32([0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0, -6.0, 0.25, 0.75, 1.25, -1.75, 2.5, 3.5, 5.0, 0.0])
    q[2, 1] = 0.0
    q[0] = torch.from_numpy(q[0]).to(torch.bfloat16).float().numpy()
    for groups in (q, q.reshape(12, 1, 64)):
        (c1, s1, t1), (c2, s2, t2) = Q.dual_residual_quantize(groups.astype(np.float64))
        u1, u2 = F.unpack_nibbles(c1), F.unpack_nibbles(c2)
        for g in range(groups.shape[0]):
            rows = [[float(v) for v in r] for r in groups[g]]
            bc1, bs1, bt1 = bf.nvfp4_group(rows)
            assert bf.f32(bt1) == float(t1[g]) and bs1 == s1[g].tolist() and bc1 == u1[g].tolist()
            x1 = bf.nvfp4_values(bc1, bs1, bt1)
            res = [[bf.f32(a - b) for a, b in zip(r, xr)] for r, xr in zip(rows, x1)]
            bc2, bs2, bt2 = bf.nvfp4_group(res)
            assert bf.f32(bt2) == float(t2[g]) and bs2 == s2[g].tolist() and bc2 == u2[g].tolist()
