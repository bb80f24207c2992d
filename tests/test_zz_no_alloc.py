"""fa4_decode_paged_noalloc (the decode with the library's own scratch, no workspace) through the C ABI
against fa4_decode_paged with a caller workspace: equal outputs, bit for bit, on two calls in a row, the
second with a smaller input, in both decode geometries."""
import ctypes

import numpy as np
import pytest
import torch

import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fa4():
    import fp8_quantized_attention_amd as m
    return m


def _gqa_case(fa4, base, B, ctx_lo, ctx_hi):
    cfg = base.scaled(B=B, ctx_lo=ctx_lo, ctx_hi=ctx_hi)
    lay = W.decode_layout(cfg)
    ctx, pt = lay.ctx_len.cuda(), lay.page_table.cuda()
    fmt = fa4.FA4_NVFP4 if cfg.kv_fmt == "nvfp4" else fa4.FA4_MXFP4
    caches = [fa4.quantize_paged(W.decode_kv_padded(cfg, lay, t, device="cuda"), fmt, ctx, pt, lay.num_pages)
              for t in (W.T_K, W.T_V)]
    q = W.decode_query(cfg).cuda()
    shape = (cfg.B, cfg.Hq, 1, cfg.d) if fmt == fa4.FA4_NVFP4 else (1, 1, cfg.B * cfg.Hq, cfg.d)
    qq = fa4.quantize(q.reshape(shape), fmt, dual=True)
    q1 = {"codes": qq["codes"], "block_scales": qq["block_scales"], "scales": qq["scales"]}
    q2 = {"codes": qq["codes2"], "block_scales": qq["block_scales2"], "scales": qq["scales2"]}
    a_ref, o_ref = fa4.decode_args(q1, q2, caches[0], caches[1], pt, ctx, cfg.Hq, cfg.Hkv, fmt=fmt)
    a_new, o_new = fa4.decode_args(q1, q2, caches[0], caches[1], pt, ctx, cfg.Hq, cfg.Hkv, fmt=fmt)
    keep = (caches, q, qq, ctx, pt)
    return a_ref, o_ref, a_new, o_new, keep


def _mla_case(fa4, B, ctx_lo, ctx_hi):
    cfg = W.C5_MLA.scaled(B=B, ctx_lo=ctx_lo, ctx_hi=ctx_hi)
    lay = W.decode_layout(cfg)
    ctx, pt = lay.ctx_len.cuda(), lay.page_table.cuda()
    x = W.decode_kv_padded(cfg, lay, W.T_K, device="cuda")[:, 0].contiguous()
    cache = fa4.quantize_paged_mla(x, ctx, pt, lay.num_pages)
    q = W.decode_query(cfg).cuda()
    qq = fa4.quantize(q.reshape(1, 1, cfg.B * cfg.Hq * 9, 64), fa4.FA4_MXFP4, dual=True)
    q1 = {"codes": qq["codes"], "block_scales": qq["block_scales"]}
    q2 = {"codes": qq["codes2"], "block_scales": qq["block_scales2"]}
    a_ref, o_ref = fa4.mla_decode_args(q1, q2, cache, pt, ctx, cfg.softmax_scale)
    a_new, o_new = fa4.mla_decode_args(q1, q2, cache, pt, ctx, cfg.softmax_scale)
    return a_ref, o_ref, a_new, o_new, (cache, q, qq, ctx, pt, x)


def _compare(fa4, case):
    a_ref, o_ref, a_new, o_new, _ = case
    ws = fa4.decode_workspace(a_ref, o_ref.device)
    assert fa4.lib.fa4_decode_paged(ctypes.byref(a_ref), ws.data_ptr(), ws.numel(), fa4._stream()) == fa4.FA4_OK
    o_new.fill_(float("nan"))
    st = fa4.lib.fa4_decode_paged_noalloc(ctypes.byref(a_new), fa4._stream())
    assert st == fa4.FA4_OK, fa4.lib.fa4_last_error()
    torch.cuda.synchronize()
    assert torch.isfinite(o_ref).all()
    assert torch.equal(o_new, o_ref)


@pytest.mark.parametrize("base", [W.C3, W.C3_MX], ids=["nvfp4", "mxfp4"])
def test_noalloc_gqa_two_calls(fa4, base):
    print(f"no-alloc decode, GQA {base.kv_fmt}: 16 sequences of 3000-9000 tokens, then 5 of 100-700", flush=True)
    _compare(fa4, _gqa_case(fa4, base, 16, 3000, 9000))
    _compare(fa4, _gqa_case(fa4, base, 5, 100, 700))


def test_noalloc_mla_two_calls(fa4):
    print("no-alloc decode, MLA: 8 sequences of 2000-5000 tokens, then 3 of 64-300", flush=True)
    _compare(fa4, _mla_case(fa4, 8, 2000, 5000))
    _compare(fa4, _mla_case(fa4, 3, 64, 300))


def test_noalloc_full_size_decode(fa4):
    """The decode workload itself (64 sequences, 32 -> 8 heads, 8K-32K tokens): 17 MB of partials, inside
    the scratch."""
    print("no-alloc decode, full-size NVFP4 GQA workload", flush=True)
    case = _gqa_case(fa4, W.C3, W.C3.B, W.C3.ctx_lo, W.C3.ctx_hi)
    assert fa4.lib.fa4_decode_workspace_bytes(ctypes.byref(case[0])) <= fa4.DECODE_SCRATCH_BYTES
    _compare(fa4, case)
