"""Pins of the oracle's MLA-geometry decode: the column-sliced page layout, the plain-attention limit,
the absorbed-query identity with per-head attention, split invariance and the brute-force loops."""
import numpy as np
import torch

import bruteforce as bf
import workloads as W
from oracle import decode as Dd
from oracle import quant as Q
from oracle_cases import mla_cache, mla_query_quant

SMALL = W.C5_MLA.scaled(B=2, ctx_lo=150, ctx_hi=330)


def build_mla(cfg, seed=0):
    """Column-sliced MXFP4 latent pages and the dual-residual query per head (oracle_cases)."""
    lay = W.decode_layout(cfg, seed)
    codes, scales, rows = mla_cache(cfg, lay, seed)
    q, (q1, q2) = mla_query_quant(cfg, seed)
    return lay, codes, scales, rows, q, q1, q2


def test_sliced_pages_hold_the_rows():
    """Gathering a token's 9 slices gives its 576-wide MXFP4 row, which is also the MXFP4 of the row
    cut into 64-wide pieces (blocks of 32 never straddle a cut)."""
    cfg = SMALL
    lay, codes, scales, rows, *_ = build_mla(cfg)
    for b in range(cfg.B):
        x, qc, qs = rows[b]
        gc, gs = Dd.gather_mla_rows(codes, scales, lay.page_table[b].numpy(), len(x))
        assert np.array_equal(gc, qc) and np.array_equal(gs, qs)
        pc, ps = Q.mxfp4_quantize(x.reshape(-1, 64))
        assert np.array_equal(pc.reshape(len(x), -1), qc) and np.array_equal(ps.reshape(len(x), -1), qs)


def test_plain_attention_limit_and_splits():
    cfg = SMALL
    lay, codes, scales, rows, q, q1, q2 = build_mla(cfg)
    s = cfg.softmax_scale
    args = (q1, q2, codes, scales, lay.page_table.numpy(), lay.ctx_len.numpy(), cfg.Hq, cfg.d_v, s)
    O = Dd.decode_mla(*args)
    On = Dd.decode_mla(*args, round_p=False)
    qhat = (Q.mxfp4_dequantize(*q1) + Q.mxfp4_dequantize(*q2)).reshape(cfg.B, cfg.Hq, cfg.d)
    for b in range(cfg.B):
        kh = Q.mxfp4_dequantize(rows[b][1], rows[b][2])
        sd = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(qhat[b][None]), torch.from_numpy(kh[None]),
            torch.from_numpy(np.ascontiguousarray(kh[None, :, :cfg.d_v])), scale=s).numpy()[0]
        assert np.abs(On[b] - sd).max() <= 1e-6 * np.abs(sd).max()
        for h in (0, 7, 15):
            for chunk in (64, 128):
                sp = Dd.decode_one(qhat[b, h], kh, kh[:, :cfg.d_v], s, chunk=chunk, tile=64, pow2_ref=True)
                assert np.abs(sp - O[b, h]).max() <= 1e-6 * np.abs(O[b, h]).max()
    assert np.abs(O - On).max() > 1e-5 * np.abs(On).max()      # the FP8 probabilities are used
    # the power-of-two reference changes where P is rounded, not the plain attention it tends to
    ex = Dd.decode_one(qhat[0, 2], Q.mxfp4_dequantize(rows[0][1], rows[0][2]),
                       Q.mxfp4_dequantize(rows[0][1], rows[0][2])[:, :cfg.d_v], s, tile=64)
    assert np.abs(ex - O[0, 2]).max() > 0 and np.abs(ex - O[0, 2]).max() <= 0.05 * np.abs(On[0, 2]).max()


def test_absorbed_query_equals_per_head_attention():
    """With the latent row [c; k_r] as key, the absorbed query [W_UK_h^T q_nope_h; q_rope_h] and the
    latent c as value, the per-head up-projection W_UV_h of the output is ordinary attention with
    keys [W_UK_h c; k_r] and values W_UV_h c (the identity the MLA geometry rests on)."""
    rng = np.random.default_rng(5)
    L, H, dc, dr, dn = 300, 4, 512, 64, 128
    c = rng.standard_normal((L, dc)); kr = rng.standard_normal((L, dr))
    Wuk = rng.standard_normal((H, dn, dc)) / np.sqrt(dc); Wuv = rng.standard_normal((H, dn, dc)) / np.sqrt(dc)
    qn = rng.standard_normal((H, dn)); qr = rng.standard_normal((H, dr))
    s = (dn + dr) ** -0.5
    latent = np.concatenate([c, kr], axis=1)
    for h in range(H):
        qa = np.concatenate([Wuk[h].T @ qn[h], qr[h]])
        o_lat = Dd.decode_one(qa, latent, c, s, round_p=False, tile=64)
        kh = np.concatenate([c @ Wuk[h].T, kr], axis=1)
        vh = c @ Wuv[h].T
        w = np.exp(s * (kh @ np.concatenate([qn[h], qr[h]])))
        ref = (w / w.sum()) @ vh
        assert np.abs(Wuv[h] @ o_lat - ref).max() <= 1e-9 * np.abs(ref).max()


def test_bruteforce_mla_row():
    cfg = SMALL.scaled(B=1, ctx_lo=150, ctx_hi=150)
    lay, codes, scales, rows, q, q1, q2 = build_mla(cfg)
    O = Dd.decode_mla(q1, q2, codes, scales, lay.page_table.numpy(), lay.ctx_len.numpy(), cfg.Hq, cfg.d_v,
                      cfg.softmax_scale, pairs=[(0, 3)])
    row = [float(v) for v in q[0, 3]]
    c1, s1 = bf.mxfp4_row(row)
    x1 = bf.mxfp4_row_values(c1, s1)
    c2, s2 = bf.mxfp4_row([bf.f32(a - b) for a, b in zip(row, x1)])
    qv = [a + b for a, b in zip(x1, bf.mxfp4_row_values(c2, s2))]
    K = []
    for t in rows[0][0]:
        c, sc = bf.mxfp4_row([float(v) for v in t])
        K.append(bf.mxfp4_row_values(c, sc))
    V = [k[:cfg.d_v] for k in K]
    ref = bf.decode_row(qv, K, V, cfg.softmax_scale, tile=64, pow2_ref=True)
    assert np.abs(O[0, 3] - np.array(ref)).max() <= 1e-6 * np.abs(ref).max()


def test_empty_context_is_zero_and_leaves_others():
    cfg = SMALL
    lay, codes, scales, rows, q, q1, q2 = build_mla(cfg)
    pt, ctx = lay.page_table.numpy(), lay.ctx_len.numpy()
    full = Dd.decode_mla(q1, q2, codes, scales, pt, ctx, cfg.Hq, cfg.d_v, cfg.softmax_scale)
    ctx0 = ctx.copy(); ctx0[0] = 0
    pt0 = pt.copy(); pt0[0] = -1
    some = Dd.decode_mla(q1, q2, codes, scales, pt0, ctx0, cfg.Hq, cfg.d_v, cfg.softmax_scale)
    assert not some[0].any()
    assert np.array_equal(some[1], full[1])
