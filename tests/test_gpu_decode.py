"""GPU paged decode (dual-residual query over an NVFP4 or MXFP4 page cache) vs the oracle."""
import numpy as np
import pytest
import torch

import workloads as W
from oracle_cases import assert_parity, decode_cache, decode_query_quant, decode_reference

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fa4():
    import fp8_quantized_attention_amd as m
    return m


def _gpu_decode(fa4, cfg, lay, seed=0, scale=None):
    ctx = lay.ctx_len.cuda()
    pt = lay.page_table.cuda()
    caches = []
    for tensor in (W.T_K, W.T_V):
        x = W.decode_kv_padded(cfg, lay, tensor, seed, device="cuda")
        fmt = fa4.FA4_NVFP4 if cfg.kv_fmt == "nvfp4" else fa4.FA4_MXFP4
        caches.append(fa4.quantize_paged(x, fmt, ctx, pt, lay.num_pages))
        del x
    q = W.decode_query(cfg, seed).cuda()
    pf = fa4.FA4_P_NVFP4 if cfg.p_fmt == "nvfp4" else fa4.FA4_P_FP8
    o, _ = fa4.decode(q, caches[0], caches[1], pt, ctx, cfg.Hkv, softmax_scale=scale, p_fmt=pf)
    torch.cuda.synchronize()
    return o.cpu().numpy(), caches


FMTS = pytest.mark.parametrize("base", [W.C3, W.C3_MX, W.C3_P4, W.C3_MX_P4],
                               ids=["nvfp4", "mxfp4", "nvfp4_p4", "mxfp4_p4"])


@FMTS
@pytest.mark.parametrize("ctx", [(200, 700), (1, 130), (128, 128), (511, 513)])
def test_decode_small_all_pairs(fa4, ctx, base):
    cfg = base.scaled(B=5, Hq=8, Hkv=2, ctx_lo=ctx[0], ctx_hi=ctx[1])
    lay = W.decode_layout(cfg)
    o, _ = _gpu_decode(fa4, cfg, lay)
    _, _, _, _, logical = decode_cache(cfg, lay, 0)
    q, (q1, q2) = decode_query_quant(cfg, 0)
    pairs = [(b, h) for b in range(cfg.B) for h in range(cfg.Hq)]
    ref = decode_reference(cfg, 0, lay, pairs, logical, q1, q2)
    assert_parity(np.stack([o[b, h] for b, h in pairs]), ref, f"decode ctx {ctx}")


@FMTS
@pytest.mark.parametrize("hq", [2, 4, 6, 16, 24], ids=["g1", "g2", "g3", "g8", "g12"])
def test_decode_query_groups(fa4, hq, base):
    """Query heads per key head other than 4: a workgroup serves a group of up to 4 of them (a smaller
    group repeats its last head in the spare matrix columns; more than 4 take several groups, each a
    pass over the key head's pages)."""
    cfg = base.scaled(B=3, Hq=hq, Hkv=2, ctx_lo=300, ctx_hi=2500)
    lay = W.decode_layout(cfg)
    o, _ = _gpu_decode(fa4, cfg, lay)
    _, _, _, _, logical = decode_cache(cfg, lay, 0)
    q, (q1, q2) = decode_query_quant(cfg, 0)
    pairs = [(b, h) for b in range(cfg.B) for h in range(cfg.Hq)]
    ref = decode_reference(cfg, 0, lay, pairs, logical, q1, q2)
    assert_parity(np.stack([o[b, h] for b, h in pairs]), ref, f"decode with {hq // 2} query heads per key head")


def with_empty(lay, seqs):
    """The layout with the listed sequences emptied (context 0, no pages)."""
    ctx, pt = lay.ctx_len.clone(), lay.page_table.clone()
    ctx[list(seqs)] = 0
    pt[list(seqs)] = -1
    return W.DecodeLayout(ctx, pt, lay.num_pages, lay.max_pages)


@FMTS
def test_decode_empty_sequences(fa4, base):
    """Sequences with no cached token get O = 0; the others are unaffected."""
    cfg = base.scaled(B=5, Hq=8, Hkv=2, ctx_lo=100, ctx_hi=900)
    lay = with_empty(W.decode_layout(cfg), [0, 3])
    o, _ = _gpu_decode(fa4, cfg, lay)
    assert not o[[0, 3]].any()
    _, _, _, _, logical = decode_cache(cfg, lay, 0)
    q, (q1, q2) = decode_query_quant(cfg, 0)
    pairs = [(b, h) for b in (1, 2, 4) for h in range(cfg.Hq)]
    ref = decode_reference(cfg, 0, lay, pairs, logical, q1, q2)
    assert_parity(np.stack([o[b, h] for b, h in pairs]), ref, "decode with empty sequences")


@FMTS
def test_decode_deterministic(fa4, base):
    cfg = base.scaled(B=4, Hq=8, Hkv=2, ctx_lo=1000, ctx_hi=3000)
    lay = W.decode_layout(cfg)
    a, _ = _gpu_decode(fa4, cfg, lay)
    b, _ = _gpu_decode(fa4, cfg, lay)
    assert np.array_equal(a, b)


@FMTS
def test_full_size_decode_sampled(fa4, base):
    cfg = base
    lay = W.decode_layout(cfg)
    o, _ = _gpu_decode(fa4, cfg, lay)
    rng = np.random.default_rng(3)
    bs = rng.choice(cfg.B, 4, replace=False)
    pairs = [(int(b), int(h)) for b in bs for h in rng.choice(cfg.Hq, 3, replace=False)]
    need = {(b, h // 4) for (b, h) in pairs}
    _, _, _, _, logical = decode_cache(cfg, lay, 0, pairs_only=need)
    q, (q1, q2) = decode_query_quant(cfg, 0)
    ref = decode_reference(cfg, 0, lay, pairs, logical, q1, q2)
    assert_parity(np.stack([o[b, h] for b, h in pairs]), ref, "decode full size")


@pytest.mark.parametrize("base", [W.C3_P4, W.C3_MX_P4], ids=["nvfp4_p4", "mxfp4_p4"])
def test_decode_p4_peaked_softmax(fa4, base):
    """A softmax scale 8x the usual makes many 16-key blocks of P' small against their tile maximum
    (under 6 * 2^-10, where a block scale taken from amax/6 alone would round to zero): the per-tile
    normalization must keep them, as the oracle does."""
    cfg = base.scaled(B=3, Hq=8, Hkv=2, ctx_lo=300, ctx_hi=1500)
    lay = W.decode_layout(cfg)
    scale = 8.0 / np.sqrt(cfg.d)
    o, _ = _gpu_decode(fa4, cfg, lay, scale=scale)
    _, _, _, _, logical = decode_cache(cfg, lay, 0)
    q, (q1, q2) = decode_query_quant(cfg, 0)
    pairs = [(b, h) for b in range(cfg.B) for h in range(cfg.Hq)]
    ref = decode_reference(cfg, 0, lay, pairs, logical, q1, q2, scale=scale)
    assert_parity(np.stack([o[b, h] for b, h in pairs]), ref, "decode p4 peaked")
    # the regime: in the first sequence's first head a third or more of the 16-key blocks lie under
    # 6 * 2^-10
    from oracle import decode as Dd
    qhat = Dd.dequant_query(q1, q2, cfg.kv_fmt).reshape(cfg.B, cfg.Hq, cfg.d)
    S = scale * (logical[(W.T_K, 0, 0)] @ qhat[0, 0])
    L = len(S) - len(S) % 128
    P = np.exp(S[:L].reshape(-1, 128) - S[:L].reshape(-1, 128).max(axis=1, keepdims=True))
    assert (P.reshape(-1, 16).max(axis=1) < 6 * 2.0 ** -10).mean() > 0.3


@pytest.mark.parametrize("base", [W.C3_MX, W.C3_MX_P4], ids=["mxfp4", "mxfp4_p4"])
def test_decode_mxfp4_smallest_v_scale(fa4, base):
    """V at 2^-127 of the usual size: every MXFP4 block of V gets the E8M0 code 0 (scale 2^-127), whose
    values code * 2^-127 (down to 2^-128) the kernel must take exactly, as the oracle does."""
    from oracle import quant as Q
    cfg = base.scaled(B=3, Hq=8, Hkv=2, ctx_lo=100, ctx_hi=900)
    lay = W.decode_layout(cfg)
    ctx, pt = lay.ctx_len.cuda(), lay.page_table.cuda()
    xk = W.decode_kv_padded(cfg, lay, W.T_K, 0)
    xv = W.decode_kv_padded(cfg, lay, W.T_V, 0) * 2.0 ** -127          # bf16 values, used by both sides
    kc = fa4.quantize_paged(xk.cuda(), fa4.FA4_MXFP4, ctx, pt, lay.num_pages)
    vc = fa4.quantize_paged(xv.cuda(), fa4.FA4_MXFP4, ctx, pt, lay.num_pages)
    q = W.decode_query(cfg, 0).cuda()
    pf = fa4.FA4_P_NVFP4 if cfg.p_fmt == "nvfp4" else fa4.FA4_P_FP8
    o, _ = fa4.decode(q, kc, vc, pt, ctx, cfg.Hkv, p_fmt=pf)
    o = o.cpu().numpy()
    _, _, _, _, logical = decode_cache(cfg, lay, 0)
    vs = vc["block_scales"].cpu().numpy()
    for b in range(cfg.B):
        L = int(lay.ctx_len[b])
        c = np.arange(L)
        phys = lay.page_table[b].numpy()[c // cfg.page_size]
        for h in range(cfg.Hkv):
            codes, scales = Q.mxfp4_quantize(xv[b, h, :L].double().numpy())
            assert not scales.any()                                         # the regime: code 0 throughout
            assert np.array_equal(vc["codes"].cpu().numpy()[phys, h, c % cfg.page_size], codes)
            assert np.array_equal(vs[phys, h, c % cfg.page_size], scales)
            logical[(W.T_V, b, h)] = Q.mxfp4_dequantize(codes, scales)
    q_, (q1, q2) = decode_query_quant(cfg, 0)
    pairs = [(b, h) for b in range(cfg.B) for h in range(cfg.Hq)]
    ref = decode_reference(cfg, 0, lay, pairs, logical, q1, q2)
    assert np.abs(ref).max() < 2.0 ** -120
    assert_parity(np.stack([o[b, h] for b, h in pairs]), ref, "decode with V at the smallest E8M0 scale")
