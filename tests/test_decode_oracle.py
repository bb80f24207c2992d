"""Pins of the oracle's paged decode: paging, split and GQA invariances, SDPA limit, brute force."""
import numpy as np
import pytest
import torch

import bruteforce as bf
import workloads as W
from oracle import decode as Dd
from oracle import quant as Q

SMALL = W.C3.scaled(B=3, Hq=8, Hkv=2, ctx_lo=200, ctx_hi=700)


def build_cache(cfg, seed=0, fmt="nvfp4"):
    """Quantize K and V per (sequence, key head) and scatter rows into pages through the page table."""
    lay = W.decode_layout(cfg, seed)
    d, ps = cfg.d, cfg.page_size
    P = lay.num_pages
    blk = 16 if fmt == "nvfp4" else 32
    kc = np.zeros((P, cfg.Hkv, ps, d // 2), np.uint8); ks = np.zeros((P, cfg.Hkv, ps, d // blk), np.uint8)
    vc = np.zeros_like(kc); vs = np.zeros_like(ks)
    kt = np.zeros((cfg.B, cfg.Hkv), np.float32); vt = np.zeros_like(kt)
    logical = {}
    for b in range(cfg.B):
        L = int(lay.ctx_len[b])
        c = np.arange(L)
        phys = lay.page_table[b].numpy()[c // ps]
        for h in range(cfg.Hkv):
            for tensor, (codes, scales, ts) in [(W.T_K, (kc, ks, kt)), (W.T_V, (vc, vs, vt))]:
                x = W.decode_kv_head(cfg, tensor, b, h, L, seed).double().numpy()
                if fmt == "nvfp4":
                    qc, qs, qt = Q.nvfp4_quantize(x[None])
                    codes[phys, h, c % ps] = qc[0]
                    scales[phys, h, c % ps] = qs[0]
                    ts[b, h] = qt[0]
                    logical[(tensor, b, h)] = (x, Q.nvfp4_dequantize(qc, qs, qt)[0])
                else:
                    qc, qs = Q.mxfp4_quantize(x)
                    codes[phys, h, c % ps] = qc
                    scales[phys, h, c % ps] = qs
                    logical[(tensor, b, h)] = (x, Q.mxfp4_dequantize(qc, qs))
    q = W.decode_query(cfg, seed).double().numpy()
    rows = q.reshape(cfg.B * cfg.Hq, 1, d)
    q1, q2 = Q.dual_residual_quantize(rows) if fmt == "nvfp4" else Q.dual_residual_quantize_mx(rows)
    return lay, (kc, ks), (vc, vs), kt, vt, q, q1, q2, logical


FMTS = pytest.mark.parametrize("fmt", ["nvfp4", "mxfp4"])


@FMTS
def test_paged_equals_contiguous_and_sdpa_limit(fmt):
    cfg = SMALL
    lay, kp, vp, kt, vt, q, q1, q2, logical = build_cache(cfg, fmt=fmt)
    O = Dd.decode_paged(q1, q2, kp, vp, kt, vt, lay.page_table.numpy(), lay.ctx_len.numpy(), cfg.Hq, cfg.Hkv,
                        fmt=fmt)
    On = Dd.decode_paged(q1, q2, kp, vp, kt, vt, lay.page_table.numpy(), lay.ctx_len.numpy(), cfg.Hq, cfg.Hkv,
                         round_p=False, fmt=fmt)
    qhat = Dd.dequant_query(q1, q2, fmt).reshape(cfg.B, cfg.Hq, cfg.d)
    g = cfg.Hq // cfg.Hkv
    for b in range(cfg.B):
        for h in range(cfg.Hq):
            kh = logical[(W.T_K, b, h // g)][1]
            vh = logical[(W.T_V, b, h // g)][1]
            # contiguous logical rows, same computation
            ref = Dd.decode_one(qhat[b, h], kh, vh, 1 / np.sqrt(cfg.d))
            assert np.abs(O[b, h] - ref).max() <= 1e-6 * np.abs(ref).max()
            # without P rounding: plain softmax attention over the dequantized cache
            sd = torch.nn.functional.scaled_dot_product_attention(
                torch.from_numpy(qhat[b, h][None, None]), torch.from_numpy(kh[None]), torch.from_numpy(vh[None]),
                scale=1 / np.sqrt(cfg.d)).numpy()[0, 0]
            assert np.abs(On[b, h] - sd).max() <= 1e-6 * np.abs(sd).max()


@FMTS
def test_split_merge_equals_single_pass(fmt):
    cfg = SMALL
    lay, kp, vp, kt, vt, q, q1, q2, logical = build_cache(cfg, fmt=fmt)
    qhat = Dd.dequant_query(q1, q2, fmt).reshape(cfg.B, cfg.Hq, cfg.d)
    kh = logical[(W.T_K, 1, 0)][1]; vh = logical[(W.T_V, 1, 0)][1]
    one = Dd.decode_one(qhat[1, 2], kh, vh, 0.1)
    for chunk in [128, 256, 384]:
        sp = Dd.decode_one(qhat[1, 2], kh, vh, 0.1, chunk=chunk)
        assert np.abs(sp - one).max() <= 1e-12 * np.abs(one).max()


def _bf_codes(packed_row):
    return [int(x) for pair in packed_row for x in (pair & 15, pair >> 4)]


def test_bruteforce_decode_mxfp4():
    """MXFP4 cache and query residuals re-derived by the brute-force loops, then attended by loops."""
    cfg = SMALL.scaled(B=1, ctx_lo=300, ctx_hi=300)
    lay, kp, vp, kt, vt, q, q1, q2, logical = build_cache(cfg, fmt="mxfp4")
    O = Dd.decode_paged(q1, q2, kp, vp, kt, vt, lay.page_table.numpy(), lay.ctx_len.numpy(), cfg.Hq, cfg.Hkv,
                        pairs=[(0, 1), (0, 6)], fmt="mxfp4")
    for h in [1, 6]:
        row = [float(v) for v in q[0, h]]
        c1, s1 = bf.mxfp4_row(row)
        assert c1 == _bf_codes(q1[0][h, 0]) and s1 == q1[1][h, 0].tolist()
        x1 = bf.mxfp4_row_values(c1, s1)
        r = [bf.f32(a - b) for a, b in zip(row, x1)]
        c2, s2 = bf.mxfp4_row(r)
        assert c2 == _bf_codes(q2[0][h, 0]) and s2 == q2[1][h, 0].tolist()
        qv = [a + b for a, b in zip(x1, bf.mxfp4_row_values(c2, s2))]
        kvh = h // 4
        K, V = [], []
        for tensor, dst in [(W.T_K, K), (W.T_V, V)]:
            x = logical[(tensor, 0, kvh)][0]
            for t in range(x.shape[0]):
                c, sc = bf.mxfp4_row([float(v) for v in x[t]])
                dst.append(bf.mxfp4_row_values(c, sc))
        ref = bf.decode_row(qv, K, V, 1 / np.sqrt(cfg.d))
        assert np.abs(O[0, h] - np.array(ref)).max() <= 1e-6 * np.abs(ref).max()


def test_bruteforce_decode():
    cfg = SMALL.scaled(B=1, ctx_lo=300, ctx_hi=300)
    lay, kp, vp, kt, vt, q, q1, q2, logical = build_cache(cfg)
    O = Dd.decode_paged(q1, q2, kp, vp, kt, vt, lay.page_table.numpy(), lay.ctx_len.numpy(), cfg.Hq, cfg.Hkv,
                        pairs=[(0, 0), (0, 5)])
    # brute force dequantizes the query from its own NVFP4 loops and attends by loops
    for h in [0, 5]:
        qv = np.zeros(cfg.d)
        for (c, s, t) in (q1, q2):
            codes = [[int(x) for pair in row for x in (pair & 15, pair >> 4)] for row in c[h]]
            qv += np.array(bf.nvfp4_values(codes, s[h].tolist(), float(t[h]))[0])
        K = logical[(W.T_K, 0, h // 4)][1].tolist()
        V = logical[(W.T_V, 0, h // 4)][1].tolist()
        ref = bf.decode_row(qv.tolist(), K, V, 1 / np.sqrt(cfg.d))
        assert np.abs(O[0, h] - np.array(ref)).max() <= 1e-6 * np.abs(ref).max()


@FMTS
def test_dual_residual_query_cuts_logit_error(fmt):
    cfg = SMALL
    lay, kp, vp, kt, vt, q, q1, q2, logical = build_cache(cfg, fmt=fmt)
    x1 = (Q.nvfp4_dequantize if fmt == "nvfp4" else Q.mxfp4_dequantize)(*q1).reshape(cfg.B, cfg.Hq, cfg.d)
    x12 = Dd.dequant_query(q1, q2, fmt).reshape(cfg.B, cfg.Hq, cfg.d)
    kh = logical[(W.T_K, 0, 0)][1]
    l0 = kh @ q[0, 0]
    e1 = np.linalg.norm(kh @ x1[0, 0] - l0) / np.linalg.norm(l0)
    e2 = np.linalg.norm(kh @ x12[0, 0] - l0) / np.linalg.norm(l0)
    assert e2 < 0.25 * e1


# ---- probabilities in NVFP4 (E2M1 codes, E4M3 scales per 16 keys), the underflow case

def _p_rows(seed=0):
    """Tile rows of probabilities in (0, 1] with the largest exactly 1: full, ragged, one block, one
    key, and blocks whose maxima fall by 2^-3 each down past the block-scale underflow point."""
    rng = np.random.default_rng(seed)
    rows = []
    for n in [128, 77, 16, 1, 128]:
        p = np.exp(-rng.exponential(6.0, n))
        p[rng.integers(n)] = 1.0
        rows.append(p)
    steps = np.concatenate([2.0 ** (-3 * k) * (0.5 + 0.5 * rng.random(16)) for k in range(8)])
    steps[0] = 1.0
    rows.append(steps)
    return rows


def test_p_nvfp4_equals_bruteforce():
    for p in _p_rows():
        got = Dd.quantize_p_nvfp4(p)
        codes, sbs, st = bf.nvfp4_group([[bf.f32(float(v)) for v in p]])
        assert st == bf.f32(1.0 / 2688.0)
        assert got.tolist() == bf.nvfp4_values(codes, sbs, st)[0]


def test_p_nvfp4_block_scales_do_not_underflow():
    """Normalizing each tile row to its maximum keeps E4M3 block scales off zero down to block maxima
    of 2^-10/448; a block scale taken straight from amax_b / 6 (no tensor scale) is zero below
    6 * 2^-10, which is the underflow the digest describes."""
    from oracle.formats import e4m3_decode, e4m3_encode
    p = _p_rows()[-1]
    ph = Dd.quantize_p_nvfp4(p).reshape(8, 16)
    for k, blk in enumerate(p.reshape(8, 16)):
        amax = blk.max()
        j = int(blk.argmax())
        assert (ph[k].max() == 0) == (amax < 2.0 ** -10 / 448)
        if amax >= 2.0 ** -6 / 448:               # E4M3-normal block scale: the block max keeps 2^-4
            assert abs(ph[k, j] - amax) <= (2.0 ** -4 + 1e-6) * amax
        naive = float(e4m3_decode(e4m3_encode(np.array([amax / 6.0])))[0])
        assert (naive == 0) == (amax < 6 * 2.0 ** -10)
    assert (ph.max(axis=1) > 0).sum() == 7 and ph[7].max() == 0   # 2^-21 < 2^-10/448 < 2^-18


def test_bruteforce_decode_p_nvfp4():
    cfg = SMALL.scaled(B=1, ctx_lo=300, ctx_hi=300)
    lay, kp, vp, kt, vt, q, q1, q2, logical = build_cache(cfg)
    O = Dd.decode_paged(q1, q2, kp, vp, kt, vt, lay.page_table.numpy(), lay.ctx_len.numpy(), cfg.Hq, cfg.Hkv,
                        pairs=[(0, 3)], p_fmt="nvfp4")
    qhat = Dd.dequant_query(q1, q2).reshape(cfg.B, cfg.Hq, cfg.d)
    K = logical[(W.T_K, 0, 0)][1].tolist()
    V = logical[(W.T_V, 0, 0)][1].tolist()
    ref = bf.decode_row(qhat[0, 3].tolist(), K, V, 1 / np.sqrt(cfg.d), p_fmt="nvfp4")
    assert np.abs(O[0, 3] - np.array(ref)).max() <= 1e-6 * np.abs(ref).max()
    fp8 = Dd.decode_paged(q1, q2, kp, vp, kt, vt, lay.page_table.numpy(), lay.ctx_len.numpy(), cfg.Hq, cfg.Hkv,
                          pairs=[(0, 3)])
    assert np.abs(O[0, 3] - fp8[0, 3]).max() > 1e-4 * np.abs(ref).max()   # the format is really used


@FMTS
def test_p_nvfp4_split_merge_and_error(fmt):
    cfg = SMALL
    lay, kp, vp, kt, vt, q, q1, q2, logical = build_cache(cfg, fmt=fmt)
    qhat = Dd.dequant_query(q1, q2, fmt).reshape(cfg.B, cfg.Hq, cfg.d)
    kh = logical[(W.T_K, 2, 1)][1]; vh = logical[(W.T_V, 2, 1)][1]
    one = Dd.decode_one(qhat[2, 5], kh, vh, 1 / np.sqrt(cfg.d), p_fmt="nvfp4")
    for chunk in [128, 256]:
        sp = Dd.decode_one(qhat[2, 5], kh, vh, 1 / np.sqrt(cfg.d), chunk=chunk, p_fmt="nvfp4")
        assert np.abs(sp - one).max() <= 1e-12 * np.abs(one).max()
    exact = Dd.decode_one(qhat[2, 5], kh, vh, 1 / np.sqrt(cfg.d), round_p=False)
    fp8 = Dd.decode_one(qhat[2, 5], kh, vh, 1 / np.sqrt(cfg.d))
    e4 = np.linalg.norm(one - exact) / np.linalg.norm(exact)
    e8 = np.linalg.norm(fp8 - exact) / np.linalg.norm(exact)
    assert e8 < e4 < 0.15          # FP4 probabilities: about 9% here, FP8 about 2%


@FMTS
def test_empty_context_is_zero_and_leaves_others(fmt):
    """A sequence with no cached token has an empty softmax; its output is defined as zero, and the
    other sequences' outputs do not change (their pages and query rows are untouched)."""
    cfg = SMALL
    lay, kp, vp, kt, vt, q, q1, q2, logical = build_cache(cfg, fmt=fmt)
    pt, ctx = lay.page_table.numpy(), lay.ctx_len.numpy()
    full = Dd.decode_paged(q1, q2, kp, vp, kt, vt, pt, ctx, cfg.Hq, cfg.Hkv, fmt=fmt)
    ctx0 = ctx.copy(); ctx0[1] = 0
    pt0 = pt.copy(); pt0[1] = -1
    some = Dd.decode_paged(q1, q2, kp, vp, kt, vt, pt0, ctx0, cfg.Hq, cfg.Hkv, fmt=fmt)
    assert not some[1].any()
    assert np.array_equal(some[[0, 2]], full[[0, 2]])
    assert not Dd.decode_one(np.ones(cfg.d), np.zeros((0, cfg.d)), np.zeros((0, cfg.d)), 0.1).any()
