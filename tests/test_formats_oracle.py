"""Pins of the oracle's number formats against the pages' bit tables, torch's casts and brute force."""
import os

import numpy as np
import pytest
import torch

import bruteforce as bf
from oracle import formats as F

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden_rows(name):
    rows = []
    for line in open(os.path.join(GOLDEN, name)):
        line = line.strip()
        if line and not line.startswith("#"):
            rows.append(line.split())
    return rows


def test_bit_table_matches_code_tables():
    """The page's sign/exponent/mantissa table fixes the code counts and largest values."""
    bits = {r[0]: tuple(int(v) for v in r[1:]) for r in _golden_rows("format_bits.txt")}
    s, e, m = bits["e2m1"]
    assert (s, e, m) == (1, 2, 1)
    assert len(F.E2M1_MAG) == 2 ** (e + m)
    # bias 2^(e-1)-1 = 1; largest = 2^(3-1) * (1 + 1/2) = 6 (E2M1 has no Inf/NaN codes)
    assert F.E2M1_MAX == 2.0 ** ((2 ** e - 1) - (2 ** (e - 1) - 1)) * (1 + (2 ** m - 1) / 2 ** m)
    s, e, m = bits["e4m3"]
    assert (s, e, m) == (1, 4, 3)
    # OCP E4M3: only the all-ones pattern is NaN, so the top binade keeps mantissas 0..6: 2^8 * 1.75
    assert F.E4M3_MAX == 448.0 and len(F.E4M3_MAG) == 2 ** (e + m) - 1
    assert bits["e8m0"] == (0, 8, 0)


def test_e2m1_grid_is_the_published_value_set():
    """The 16 codes decode to {0, +-0.5, +-1, +-1.5, +-2, +-3, +-4, +-6}."""
    vals = sorted(set(F.e2m1_decode(np.arange(16)).tolist()))
    assert vals == [-6, -4, -3, -2, -1.5, -1, -0.5, 0, 0.5, 1, 1.5, 2, 3, 4, 6]
    assert np.signbit(F.e2m1_decode(8)) and not np.signbit(F.e2m1_decode(0))
    for c in range(16):
        assert F.e2m1_decode(c) == bf.e2m1_value(c)


def test_e2m1_encode_vs_bruteforce():
    rng = np.random.default_rng(0)
    grid = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6], dtype=np.float64)
    mids = (grid[1:] + grid[:-1]) / 2
    pts = [0.0, -0.0, 7.0, -100.0, 1e-30, -1e-30]
    for m in mids:
        m32 = np.float32(m)
        for k in range(-4, 5):
            pts.append(float(np.nextafter(m32, np.float32(np.inf * np.sign(k))) if k else m32) if k in (-1, 1)
                       else float(m32 + np.float32(k) * np.float32(1e-6)))
            pts.append(-pts[-1])
        pts.append(float(m))
    pts += rng.uniform(-7, 7, 20000).astype(np.float32).tolist()
    pts = np.array(pts, dtype=np.float64)
    got = F.e2m1_encode(pts)
    ref = np.array([bf.e2m1_encode(float(x)) for x in pts])
    assert np.array_equal(got, ref)
    # ties: 0.25->0, 0.75->1, 1.25->1, 1.75->2, 2.5->2, 3.5->4, 5->4
    ties = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
    assert F.E2M1_MAG[F.e2m1_encode(ties)].tolist() == [0, 1, 1, 2, 2, 4, 4]


def test_e2m1_idempotent():
    for e in range(-10, 10):
        for c in range(16):
            v = F.e2m1_decode(c) * 2.0 ** e
            assert F.e2m1_encode(v * 2.0 ** -e) == c or (c in (0, 8) and F.e2m1_encode(v * 2.0 ** -e) in (0, 8))


def test_e4m3_decode_vs_torch():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    t = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(F.e4m3_decode(codes), t)
    assert np.isnan(F.e4m3_decode(0x7F)) and np.isnan(F.e4m3_decode(0xFF))


def test_e4m3_encode_vs_torch_cast():
    """Below 464 torch's float8_e4m3fn cast is round-to-nearest-even; it must agree code for code."""
    rng = np.random.default_rng(1)
    mags = np.concatenate([
        rng.uniform(0, 464, 200000),
        np.exp2(rng.uniform(-14, 8.8, 200000)),
        (F.E4M3_MAG[1:] + F.E4M3_MAG[:-1]) / 2,            # exact ties
        F.E4M3_MAG,
    ]).astype(np.float32)
    mags = mags[mags < 464]
    x = np.concatenate([mags, -mags]).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = F.e4m3_encode(x.astype(np.float64))
    assert np.array_equal(got.astype(np.uint8), ref)
    for v, c in [(449.0, 0x7E), (464.0, 0x7E), (232.0, 0x76), (1.0625, 0x38), (1.1875, 0x3A),
                 (-0.0, 0x80), (0.0, 0x00)]:
        assert int(F.e4m3_encode(v)) == c
        assert bf.e4m3_encode(v) == c


def test_e4m3_saturates():
    for v in [480.0, 1e6, 3.4e38]:
        assert int(F.e4m3_encode(v)) == 0x7E and int(F.e4m3_encode(-v)) == 0xFE


def test_e4m3_encode_vs_bruteforce():
    rng = np.random.default_rng(2)
    x = np.exp2(rng.uniform(-12, 9.2, 3000)) * rng.choice([-1, 1], 3000)
    got = F.e4m3_encode(x)
    ref = np.array([bf.e4m3_encode(float(v)) for v in x])
    assert np.array_equal(got, ref)


def test_e8m0_vs_torch_on_powers_of_two():
    e = np.arange(-127, 128)
    x = torch.from_numpy(np.ldexp(1.0, e).astype(np.float32))
    codes = x.to(torch.float8_e8m0fnu).view(torch.uint8).numpy().astype(np.int64)
    assert np.array_equal(codes, e + 127)
    assert np.array_equal(F.e8m0_decode(codes), np.ldexp(1.0, e))


def test_bf16_round_vs_torch():
    rng = np.random.default_rng(3)
    x = np.concatenate([rng.standard_normal(100000), np.exp2(rng.uniform(-130, 100, 100000)),
                        rng.uniform(0, 1, 100000)]).astype(np.float32)
    # exact ties between bf16 neighbours
    ties = ((x.view(np.uint32) & 0xFFFF0000) | 0x8000).view(np.float32)
    x = np.concatenate([x, ties, -x])
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(F.bf16_round(x.astype(np.float64)), ref)
    for v in x[:2000]:
        assert bf.bf16(float(v)) == F.bf16_round(float(v))


def test_nibble_packing_roundtrip():
    rng = np.random.default_rng(4)
    c = rng.integers(0, 16, (3, 64))
    p = F.pack_nibbles(c)
    assert p.shape == (3, 32)
    assert int(p[0, 0]) == int(c[0, 0]) | (int(c[0, 1]) << 4)
    assert np.array_equal(F.unpack_nibbles(p), c)
