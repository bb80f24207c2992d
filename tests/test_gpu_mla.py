"""GPU decode in the MLA geometry (MXFP4 latent cache, column-sliced pages) vs the oracle."""
import numpy as np
import pytest
import torch

import workloads as W
from oracle import decode as Dd
from oracle_cases import assert_parity, mla_cache, mla_query_quant

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fa4():
    import fp8_quantized_attention_amd as m
    return m


def _padded(cfg, lay, seed=0):
    Lmax = int(lay.ctx_len.max())
    x = torch.zeros(cfg.B, Lmax, cfg.d, dtype=torch.bfloat16)
    for b in range(cfg.B):
        L = int(lay.ctx_len[b])
        x[b, :L] = W.decode_kv_head(cfg, W.T_K, b, 0, L, seed)
    return x.cuda()


def _gpu(fa4, cfg, lay, seed=0):
    ctx, pt = lay.ctx_len.cuda(), lay.page_table.cuda()
    cache = fa4.quantize_paged_mla(_padded(cfg, lay, seed), ctx, pt, lay.num_pages)
    q = W.decode_query(cfg, seed).cuda()
    o, qq = fa4.decode_mla(q, cache, pt, ctx, cfg.softmax_scale)
    torch.cuda.synchronize()
    return o.cpu().numpy(), cache, qq


def _check(fa4, cfg, pairs=None, seed=0, empty=()):
    lay = W.decode_layout(cfg, seed)
    if empty:                                            # emptied sequences: context 0, no pages
        ctx, pt = lay.ctx_len.clone(), lay.page_table.clone()
        ctx[list(empty)] = 0
        pt[list(empty)] = -1
        lay = W.DecodeLayout(ctx, pt, lay.num_pages, lay.max_pages)
    print(f"[mla] B={cfg.B} ctx={lay.ctx_len.tolist()[:8]}", flush=True)
    o, cache, qq = _gpu(fa4, cfg, lay, seed)
    seqs = sorted({b for b, _ in pairs}) if pairs else None
    codes, scales, rows = mla_cache(cfg, lay, seed, seqs)
    q, (q1, q2) = mla_query_quant(cfg, seed)
    # the cache and the query residuals, bit for bit, on every existing row
    gc, gs = cache["codes"].cpu().numpy(), cache["block_scales"].cpu().numpy()
    for b in rows:
        L = int(lay.ctx_len[b])
        c = np.arange(L)
        phys = lay.page_table[b].numpy()[c // 64]
        assert np.array_equal(gc[phys, :, c % 64], codes[phys, :, c % 64])
        assert np.array_equal(gs[phys, :, c % 64], scales[phys, :, c % 64])
    n = cfg.B * cfg.Hq
    assert np.array_equal(qq["codes"].cpu().numpy().reshape(n, -1), q1[0])
    assert np.array_equal(qq["block_scales"].cpu().numpy().reshape(n, -1), q1[1])
    assert np.array_equal(qq["codes2"].cpu().numpy().reshape(n, -1), q2[0])
    assert np.array_equal(qq["block_scales2"].cpu().numpy().reshape(n, -1), q2[1])
    pairs = pairs or [(b, h) for b in range(cfg.B) for h in range(cfg.Hq)]
    ref = Dd.decode_mla(q1, q2, codes, scales, lay.page_table.numpy(), lay.ctx_len.numpy(), cfg.Hq, cfg.d_v,
                        cfg.softmax_scale, pairs=pairs)
    assert_parity(np.stack([o[b, h] for b, h in pairs]), np.stack([ref[b, h] for b, h in pairs]),
                  f"mla B={cfg.B}")
    for b in empty:
        assert not o[b].any()


@pytest.mark.parametrize("ctx", [(150, 700), (1, 70), (64, 64), (2047, 2113)])
def test_mla_small_all_pairs(fa4, ctx):
    """Ragged last pages, one-key and one-page contexts, and contexts across the 32-page split."""
    _check(fa4, W.C5_MLA.scaled(B=4, ctx_lo=ctx[0], ctx_hi=ctx[1]))


def test_mla_empty_sequences(fa4):
    """Sequences with no cached token get O = 0; the others are unaffected."""
    _check(fa4, W.C5_MLA.scaled(B=4, ctx_lo=100, ctx_hi=2200), empty=(1, 2))


def test_mla_deterministic(fa4):
    cfg = W.C5_MLA.scaled(B=3, ctx_lo=3000, ctx_hi=5000)
    lay = W.decode_layout(cfg)
    a, _, _ = _gpu(fa4, cfg, lay)
    b, _, _ = _gpu(fa4, cfg, lay)
    assert np.array_equal(a, b)


def test_mla_full_size_sampled(fa4):
    cfg = W.C5_MLA
    rng = np.random.default_rng(4)
    bs = rng.choice(cfg.B, 3, replace=False)
    pairs = [(int(b), int(h)) for b in bs for h in rng.choice(cfg.Hq, 4, replace=False)]
    _check(fa4, cfg, pairs)
