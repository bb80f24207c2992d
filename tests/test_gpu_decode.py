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


def _gpu_decode(fa4, cfg, lay, seed=0):
    ctx = lay.ctx_len.cuda()
    pt = lay.page_table.cuda()
    caches = []
    for tensor in (W.T_K, W.T_V):
        x = W.decode_kv_padded(cfg, lay, tensor, seed, device="cuda")
        fmt = fa4.FA4_NVFP4 if cfg.kv_fmt == "nvfp4" else fa4.FA4_MXFP4
        caches.append(fa4.quantize_paged(x, fmt, ctx, pt, lay.num_pages))
        del x
    q = W.decode_query(cfg, seed).cuda()
    o, _ = fa4.decode(q, caches[0], caches[1], pt, ctx, cfg.Hkv)
    torch.cuda.synchronize()
    return o.cpu().numpy(), caches


FMTS = pytest.mark.parametrize("base", [W.C3, W.C3_MX], ids=["nvfp4", "mxfp4"])


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
