"""GPU prefill path (quantize -> select -> fused attention) vs the oracle.

Codes, scales, norms and tile bitmaps are compared bit for bit; O within relative L2 <= 1e-3 and
max-abs <= 2e-3 max|O|; LSE within 1e-4 absolute. Small shapes are compared in full (several tiles,
causal diagonal, GQA, chunk offset); the full-size workloads on sampled rows of sampled heads.
"""
import numpy as np
import pytest
import torch

import workloads as W
from oracle import attention as A
from oracle_cases import assert_parity, prefill_reference, rel_errors

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fa4():
    import fp8_quantized_attention_amd as m
    return m


def _run(fa4, cfg, seed=0, select=None):
    q, k, v = W.prefill_inputs(cfg, seed)
    fmt = {"mxfp4": fa4.FA4_MXFP4, "nvfp4": fa4.FA4_NVFP4, "mxfp8": fa4.FA4_MXFP8}[cfg.qk_fmt]
    vf = fa4.FA4_MXFP4_KEYS if cfg.v_fmt == "mxfp4k" else fa4.FA4_FP8_TOKEN
    res = fa4.prefill(q.cuda(), k.cuda(), v.cuda(), cfg.causal, fmt=fmt, hadamard=cfg.hadamard, select=select,
                      v_fmt=vf)
    torch.cuda.synchronize()
    return (q, k, v), res


def _check_full(fa4, cfg, seed=0, select=None, lse=True):
    (q, k, v), res = _run(fa4, cfg, seed, select)
    heads = [(b, h) for b in range(cfg.B) for h in range(cfg.Hq)]
    rows = np.arange(cfg.Lq)
    O, L, bms = prefill_reference(cfg, seed, heads, rows, select, q, k, v)
    got = res["o"].cpu().numpy().reshape(-1, cfg.Lq, cfg.d)
    rel, mx = assert_parity(got, O, cfg.name)
    if lse:
        assert np.abs(res["lse"].cpu().numpy().reshape(-1, cfg.Lq) - L).max() < 1e-4
    if select is not None:
        gb = res["bitmap"].cpu().numpy()
        for (b, h), bm in bms.items():
            assert np.array_equal(gb[b, h], bm), (b, h)
    return rel, mx, res, (q, k, v)


def test_tiny_noncausal_d64(fa4):
    for seed in (0, 1, 2):
        _check_full(fa4, W.C0, seed)


def test_causal_small_mxfp4(fa4):
    _check_full(fa4, W.C1.scaled(Hq=2, Hkv=2, Lq=512, Lk=512))


def test_causal_small_gqa_offset_mxfp4(fa4):
    _check_full(fa4, W.C1.scaled(Hq=4, Hkv=2, Lq=256, Lk=768))


@pytest.mark.parametrize("frac", [(5, 100), (30, 100)])
def test_selection_small(fa4, frac):
    cfg = W.C2.scaled(Hq=2, Hkv=2, Lq=1024, Lk=1024)
    rel, mx, res, _ = _check_full(fa4, cfg, select=frac)
    assert int(res["bitmap"].sum()) == int(res["counts"].sum())


def test_all_tiles_bf16_is_ordinary_attention(fa4):
    """num/den = 1: every valid tile runs in bf16; O matches unquantized attention up to bf16(P)."""
    cfg = W.C2.scaled(Hq=2, Hkv=2, Lq=512, Lk=512)
    rel, mx, res, (q, k, v) = _check_full(fa4, cfg, select=(100, 100))
    ref = A.attention_reference(q.double().numpy(), k.double().numpy(), v.double().numpy(), True)
    r2, _ = rel_errors(res["o"].cpu().numpy(), ref)
    assert r2 < 5e-3


def test_zero_fraction_equals_no_selection(fa4):
    cfg = W.C2.scaled(Hq=2, Hkv=2, Lq=512, Lk=512)
    (_, _, _), r0 = _run(fa4, cfg, select=(0, 100))
    (_, _, _), r1 = _run(fa4, cfg, select=None)
    assert int(r0["bitmap"].sum()) == 0
    assert torch.equal(r0["o"], r1["o"])


def test_nvfp4_hadamard_gqa_offset_selection_small(fa4):
    _check_full(fa4, W.C4.scaled(Hq=8, Hkv=2, Lq=256, Lk=1024), select=(5, 100))
    _check_full(fa4, W.C4.scaled(Hq=8, Hkv=2, Lq=256, Lk=1024), select=(25, 100))


def test_deterministic(fa4):
    cfg = W.C2.scaled(Hq=2, Hkv=2, Lq=1024, Lk=1024)
    _, a = _run(fa4, cfg, select=(5, 100))
    _, b = _run(fa4, cfg, select=(5, 100))
    assert torch.equal(a["o"], b["o"]) and torch.equal(a["lse"], b["lse"]) and torch.equal(a["bitmap"], b["bitmap"])


# ---- Q and K in MXFP8 (E4M3 elements, E8M0 per 32): K expanded to exact bf16, QK^T on bf16 MFMAs
def test_mxfp8_tiny_noncausal_f32(fa4):
    _check_full(fa4, W.C0.scaled(qk_fmt="mxfp8", d=128))


def test_mxfp8_causal_small_gqa_offset(fa4):
    _check_full(fa4, W.C1_MX8.scaled(Hq=4, Hkv=2, Lq=256, Lk=768))


def test_mxfp8_selection_small(fa4):
    _check_full(fa4, W.C1_MX8.scaled(Hq=2, Hkv=2, Lq=1024, Lk=1024, select=True), select=(5, 100))


def _sampled(fa4, cfg, heads, nrows, select=None, seed=0):
    (q, k, v), res = _run(fa4, cfg, seed, select)
    rng = np.random.default_rng(7)
    rows = np.sort(np.concatenate([[0, cfg.Lq - 1], rng.choice(cfg.Lq, nrows, replace=False)]))
    rows = np.unique(rows)
    O, L, bms = prefill_reference(cfg, seed, heads, rows, select, q, k, v)
    o = res["o"].cpu().numpy()
    got = np.stack([o[b, h, rows] for (b, h) in heads])
    assert_parity(got, O, cfg.name)
    lse = res["lse"].cpu().numpy()
    assert np.abs(np.stack([lse[b, h, rows] for (b, h) in heads]) - L).max() < 1e-4
    if select is not None:
        gb = res["bitmap"].cpu().numpy()
        for (b, h), bm in bms.items():
            assert np.array_equal(gb[b, h], bm)
    return res


def test_full_size_prefill_4k(fa4):
    _sampled(fa4, W.C1, heads=[(0, 0), (0, 13), (0, 31)], nrows=96)


def test_full_size_prefill_32k_selection(fa4):
    _sampled(fa4, W.C2, heads=[(0, 5), (0, 30)], nrows=24, select=(5, 100))


def test_full_size_chunked_prefill_128k(fa4):
    _sampled(fa4, W.C4, heads=[(0, 0), (0, 7), (0, 29)], nrows=24, select=(5, 100))


def test_full_size_prefill_4k_mxfp8(fa4):
    _sampled(fa4, W.C1_MX8, heads=[(0, 0), (0, 17)], nrows=96)



# ---- 4-bit V (MXFP4 along the keys; FP4 V^T x FP8 P^T in one block-scaled MFMA)

def test_v4_causal_small(fa4):
    _check_full(fa4, W.C1_V4.scaled(Hq=2, Hkv=2, Lq=512, Lk=512))


def test_v4_noncausal_gqa_offset(fa4):
    _check_full(fa4, W.C1_V4.scaled(Hq=4, Hkv=2, Lq=256, Lk=768, causal=False))
    _check_full(fa4, W.C1_V4.scaled(Hq=4, Hkv=2, Lq=256, Lk=768), seed=1)


def test_full_size_prefill_4k_v4(fa4):
    _sampled(fa4, W.C1_V4, heads=[(0, 0), (0, 21)], nrows=96)
