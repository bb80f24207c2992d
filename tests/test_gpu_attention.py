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
    pf = fa4.FA4_P_MXFP4 if cfg.p_fmt == "mxfp4" else fa4.FA4_P_FP8
    res = fa4.prefill(q.cuda(), k.cuda(), v.cuda(), cfg.causal, fmt=fmt, hadamard=cfg.hadamard, select=select,
                      v_fmt=vf, p_fmt=pf)
    torch.cuda.synchronize()
    return (q, k, v), res


def _check_full(fa4, cfg, seed=0, select=None, lse=True):
    (q, k, v), res = _run(fa4, cfg, seed, select)
    heads = [(b, h) for b in range(cfg.B) for h in range(cfg.Hq)]
    rows = np.arange(cfg.Lq)
    O, L, bms, slack = prefill_reference(cfg, seed, heads, rows, select, q, k, v, slack=True)
    got = res["o"].cpu().numpy().reshape(-1, cfg.Lq, cfg.d)
    rel, mx = assert_parity(got, O, cfg.name, slack)
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
def test_fp8_pv_one_large_many_small(fa4):
    """PV with one dominant probability per row in every 128-key tile and 127 others about 2^-8 of it, so
    that each 64-key FP8 MFMA step adds one large product next to many small ones, the case where the
    FP8 MFMA's accumulation is inexact: the result must stay within the parity bar."""
    cfg = W.C1.scaled(B=1, Hq=1, Hkv=1, Lq=128, Lk=512, causal=False)
    d = cfg.d
    q = torch.zeros(1, 1, cfg.Lq, d)
    k = torch.zeros(1, 1, cfg.Lk, d)
    rows = torch.arange(cfg.Lq)
    q[0, 0, rows, rows % d] = 64.0                       # exact in MXFP4 (code 4, scale 2^4)
    keys = torch.arange(cfg.Lk)
    k[0, 0, keys, keys % d] = 1.0                        # score 64 / sqrt(128) for keys r, r + 128, ..., else 0
    g = torch.Generator().manual_seed(11)
    v = torch.randn(1, 1, cfg.Lk, d, generator=g) * (1.0 + 4.0 * torch.rand(1, 1, cfg.Lk, 1, generator=g))
    q, k, v = (t.to(torch.bfloat16) for t in (q, k, v))
    res = fa4.prefill(q.cuda(), k.cuda(), v.cuda(), cfg.causal, fmt=fa4.FA4_MXFP4)
    torch.cuda.synchronize()
    O, L, _, slack = prefill_reference(cfg, 0, [(0, 0)], np.arange(cfg.Lq), None, q, k, v, slack=True)
    got = res["o"].cpu().numpy().reshape(-1, cfg.Lq, d)
    assert_parity(got, O, "one large product next to many small ones", slack)
    assert np.abs(res["lse"].cpu().numpy().reshape(-1, cfg.Lq) - L).max() < 1e-4


def test_mxfp8_tiny_noncausal_f32(fa4):
    _check_full(fa4, W.C0.scaled(qk_fmt="mxfp8", d=128))


def test_mxfp8_causal_small_gqa_offset(fa4):
    _check_full(fa4, W.C1_MX8.scaled(Hq=4, Hkv=2, Lq=256, Lk=768))


def test_mxfp8_selection_small(fa4):
    _check_full(fa4, W.C1_MX8.scaled(Hq=2, Hkv=2, Lq=1024, Lk=1024, select=True), select=(5, 100))


# ---- NVFP4 / MXFP8 over grouped key heads (one to four query heads per key head), with and without
# selection (the heads of a group select different tiles), in both work orders (key heads split evenly
# over the 8 XCDs, and not).

@pytest.mark.parametrize("causal", [True, False], ids=["causal", "noncausal"])
@pytest.mark.parametrize("select", [None, (5, 100), (25, 100)], ids=["nosel", "sel5", "sel25"])
def test_nvfp4_gqa(fa4, causal, select):
    _check_full(fa4, W.C4.scaled(Hq=4, Hkv=2, Lq=256, Lk=768, causal=causal), select=select)


@pytest.mark.parametrize("frac", [0, 90, 100])
def test_nvfp4_gqa_selection_extremes(fa4, frac):
    # 100%: no quantized tile at all; 90%: runs of one or two quantized tiles between selected ones
    _check_full(fa4, W.C4.scaled(Hq=4, Hkv=2, Lq=512, Lk=1024), select=(frac, 100))


def test_nvfp4_gqa_xcd_order(fa4):
    # 8 key heads (the work order that keeps all query heads of a key head on one XCD), 4 per key head
    _check_full(fa4, W.C4.scaled(Hq=32, Hkv=8, Lq=256, Lk=512), select=(5, 100))


@pytest.mark.parametrize("hkv", [2, 4], ids=["fallback_order", "xcd_order"])
def test_nvfp4_gqa_two_batches(fa4, hkv):
    # B = 2: batch and key head ordered without (2 x 2 key heads) and with (2 x 4 = 8) the XCD grouping
    _check_full(fa4, W.C4.scaled(B=2, Hq=2 * hkv, Hkv=hkv, Lq=256, Lk=512), select=(10, 100))


@pytest.mark.parametrize("hq", [2, 6], ids=["mha", "group3"])
def test_nvfp4_odd_groups(fa4, hq):
    _check_full(fa4, W.C4.scaled(Hq=hq, Hkv=2, Lq=256, Lk=768), select=(5, 100))


def test_mxfp8_gqa_selection(fa4):
    _check_full(fa4, W.C1_MX8.scaled(Hq=4, Hkv=2, Lq=512, Lk=512, select=True), select=(10, 100))


def _sampled(fa4, cfg, heads, nrows, select=None, seed=0):
    (q, k, v), res = _run(fa4, cfg, seed, select)
    rng = np.random.default_rng(7)
    rows = np.sort(np.concatenate([[0, cfg.Lq - 1], rng.choice(cfg.Lq, nrows, replace=False)]))
    rows = np.unique(rows)
    O, L, bms, slack = prefill_reference(cfg, seed, heads, rows, select, q, k, v, slack=True)
    o = res["o"].cpu().numpy()
    got = np.stack([o[b, h, rows] for (b, h) in heads])
    assert_parity(got, O, cfg.name, slack)
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


@pytest.mark.parametrize("select", [(5, 100), (25, 100), (100, 100)], ids=["sel5", "sel25", "all"])
def test_v4_with_selection(fa4, select):
    # quantized tiles through 4-bit V (their P^ carries 448), selected tiles through bf16 V (no 448)
    _check_full(fa4, W.C1_V4.scaled(Hq=2, Hkv=2, Lq=512, Lk=512), select=select)


@pytest.mark.parametrize("causal", [True, False], ids=["causal", "noncausal"])
def test_v4_with_selection_gqa_offset(fa4, causal):
    _check_full(fa4, W.C1_V4.scaled(Hq=4, Hkv=2, Lq=256, Lk=768, causal=causal), select=(10, 100))


def test_full_size_prefill_4k_v4_selection(fa4):
    _sampled(fa4, W.C1_V4, heads=[(0, 3), (0, 30)], nrows=64, select=(5, 100))


def test_full_size_prefill_4k_v4(fa4):
    _sampled(fa4, W.C1_V4, heads=[(0, 0), (0, 21)], nrows=96)


# ---- 4K causal at the other two seeds (small shape in full, full size on sampled rows)

@pytest.mark.parametrize("seed", [1, 2])
def test_causal_small_mxfp4_seeds(fa4, seed):
    _check_full(fa4, W.C1.scaled(Hq=2, Hkv=2, Lq=512, Lk=512), seed)


@pytest.mark.parametrize("seed", [1, 2])
def test_full_size_prefill_4k_seeds(fa4, seed):
    _sampled(fa4, W.C1, heads=[(0, 3), (0, 26)], nrows=64, seed=seed)


# ---- the online softmax's reference jumps: keys of some tiles scaled so that a tile's row maximum rises
# far above the running reference (the accumulator and the pending half-tile are rescaled), and so far that
# earlier tiles fall below the smallest representable weight

def _jump_inputs(causal, factors, seed=31):
    g = torch.Generator().manual_seed(seed)
    L, d = 128 * len(factors), 128
    q = torch.randn(1, 2, L, d, generator=g).to(torch.bfloat16)
    k = torch.randn(1, 2, L, d, generator=g)
    for j, f in enumerate(factors):
        k[:, :, 128 * j:128 * (j + 1)] *= f
    k = k.to(torch.bfloat16)
    v = torch.randn(1, 2, L, d, generator=g).to(torch.bfloat16)
    return q, k, v


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("factors", [(1, 1, 1, 8, 1, 1, 1, 1), (1, 2, 40, 1, 1, 1, 160, 1)],
                         ids=["raise_once", "raise_past_smallest_weight"])
@pytest.mark.parametrize("select", [None, (25, 100)])
@pytest.mark.parametrize("p4", [False, True], ids=["p8", "p4"])
@pytest.mark.parametrize("v4", [False, True], ids=["v8", "v4"])
def test_reference_jumps(fa4, causal, factors, select, p4, v4):
    # p4: MXFP4 probabilities, whose per-block E8M0 scale carries the tile weight (and the pending half's
    # weight follows a raised reference); v4: 4-bit V (its 448 and its division with FP8 probabilities)
    from oracle import quant as Q
    from oracle import selection as S
    q, k, v = _jump_inputs(causal, factors)
    L = q.shape[2]
    pf = "mxfp4" if p4 else "fp8"
    res = fa4.prefill(q.cuda(), k.cuda(), v.cuda(), causal, fmt=fa4.FA4_MXFP4, select=select,
                      p_fmt=fa4.FA4_P_MXFP4 if p4 else fa4.FA4_P_FP8,
                      v_fmt=fa4.FA4_MXFP4_KEYS if v4 else fa4.FA4_FP8_TOKEN)
    torch.cuda.synchronize()
    qd, kd, vd = (t.double().numpy() for t in (q, k, v))
    qq = Q.mxfp4_dequantize(*Q.mxfp4_quantize(qd))
    kk = Q.mxfp4_dequantize(*Q.mxfp4_quantize(kd))
    if v4:
        vc, sv = None, None
        v_deq = Q.mxfp4_keys_dequantize(*Q.mxfp4_keys_quantize(vd))
    else:
        (vc, sv), v_deq = Q.fp8_per_token_quantize(vd), None
    bm = None
    if select is not None:
        bm, _ = S.select_tiles(Q.row_norm2(qd), Q.row_norm2(kd), L, L, causal, *select)
        assert np.array_equal(res["bitmap"].cpu().numpy(), bm)
    O, lse = A.attention_prefill(qq, kk, vc, sv, causal, q_orig=qd, k_orig=kd, v_orig=vd, bitmap=bm, p_fmt=pf,
                                 v_deq=v_deq)
    # Conditioning of this input: scores reach ~230 in log2 units, where the float32 rounding of the
    # exponent's argument (2^-24 relative) already flips bf16 and E4M3 probability codes of rows that one
    # key dominates. The oracle itself, with its softmax scale moved by one float32 ulp, differs by
    # delta; the max-abs bound is max(2e-3, 2 delta), the relative-L2 bound stays 1e-3.
    O1, _ = A.attention_prefill(qq, kk, vc, sv, causal, scale=(1.0 + 2.0 ** -23) / np.sqrt(128), q_orig=qd,
                                k_orig=kd, v_orig=vd, bitmap=bm, p_fmt=pf, v_deq=v_deq)
    _, delta = rel_errors(O1, O)
    rel, mx = rel_errors(res["o"].cpu().numpy(), O)
    what = f"jumps {factors} causal={causal} select={select} p={pf} v4={v4}"
    assert rel <= 1e-3 and mx <= max(2e-3, 2 * delta), f"{what}: rel-L2 {rel:.3e} max-abs/max {mx:.3e} (delta {delta:.2e})"
    # LSE: the scores themselves are float32 sums of 128 products here reaching ~1e4, so their rounding
    # (about 2^-23 of sum |q_i k_i| per score, in units of the softmax scale) bounds the LSE agreement
    eps_s = 2.0 ** -23 * (np.abs(qq) @ np.abs(np.swapaxes(kk, -1, -2))).max() / np.sqrt(128)
    assert np.abs(res["lse"].cpu().numpy() - lse).max() < 1e-4 + 4 * eps_s


def test_few_quantized_tiles_between_selected(fa4):
    """90% of the tiles in bf16: the quantized pipeline runs over one or two tiles per row of tiles."""
    _check_full(fa4, W.C2.scaled(Hq=2, Hkv=2, Lq=1024, Lk=1024), select=(90, 100))


# ---- MXFP4 probabilities (FP8 V^T x FP4 P^T, the block scale and the tile weight as P^T's E8M0 scale)

def test_p4_causal_small(fa4):
    rel, mx, res, _ = _check_full(fa4, W.C1_P4.scaled(Hq=2, Hkv=2, Lq=512, Lk=512))
    # the probabilities are rounded to FP4 (the result differs from the FP8-probability path)
    (q, k, v), r8 = _run(fa4, W.C1.scaled(Hq=2, Hkv=2, Lq=512, Lk=512))
    assert rel_errors(res["o"].cpu().numpy(), r8["o"].cpu().numpy())[0] > 1e-3


@pytest.mark.parametrize("causal", [True, False], ids=["causal", "noncausal"])
def test_p4_gqa_offset(fa4, causal):
    _check_full(fa4, W.C1_P4.scaled(Hq=4, Hkv=2, Lq=256, Lk=768, causal=causal))
    _check_full(fa4, W.C1_P4.scaled(Hq=4, Hkv=2, Lq=256, Lk=768, causal=causal), seed=1)


@pytest.mark.parametrize("select", [(5, 100), (25, 100), (100, 100)], ids=["sel5", "sel25", "all"])
def test_p4_with_selection(fa4, select):
    _check_full(fa4, W.C1_P4.scaled(Hq=2, Hkv=2, Lq=512, Lk=512), select=select)


def test_full_size_prefill_4k_p4(fa4):
    _sampled(fa4, W.C1_P4, heads=[(0, 2), (0, 27)], nrows=96)


def test_full_size_prefill_32k_p4_selection(fa4):
    _sampled(fa4, W.C2.scaled(p_fmt="mxfp4"), heads=[(0, 9)], nrows=16, select=(5, 100))


# ---- 4-bit V with MXFP4 probabilities (FP4 V^T x FP4 P^T, both block scales inside the product)

def test_v4p4_causal_small(fa4):
    _check_full(fa4, W.C1_V4P4.scaled(Hq=2, Hkv=2, Lq=512, Lk=512))


@pytest.mark.parametrize("causal", [True, False], ids=["causal", "noncausal"])
def test_v4p4_gqa_offset(fa4, causal):
    _check_full(fa4, W.C1_V4P4.scaled(Hq=4, Hkv=2, Lq=256, Lk=768, causal=causal), seed=1)


@pytest.mark.parametrize("select", [(5, 100), (100, 100)], ids=["sel5", "all"])
def test_v4p4_with_selection(fa4, select):
    _check_full(fa4, W.C1_V4P4.scaled(Hq=2, Hkv=2, Lq=512, Lk=512), select=select)


def test_full_size_prefill_4k_v4p4(fa4):
    _sampled(fa4, W.C1_V4P4, heads=[(0, 4), (0, 30)], nrows=96, select=None)


@pytest.mark.parametrize("cfg", [W.C1_P4, W.C1_V4P4], ids=["p4", "v4p4"])
def test_p4_deterministic(fa4, cfg):
    """The MXFP4-probability kernels give bitwise the same output on a rerun (no atomics or order-dependent
    sums in the attention kernel)."""
    c = cfg.scaled(Hq=4, Hkv=2, Lq=1024, Lk=1024)
    (_, _, _), r1 = _run(fa4, c, select=(5, 100))
    (_, _, _), r2 = _run(fa4, c, select=(5, 100))
    assert torch.equal(r1["o"], r2["o"]) and torch.equal(r1["lse"], r2["lse"])
