"""Full-size parity of every bit-exact object of the prefill and decode paths, in the launch
configuration the benchmark times.

For the 4K causal workload (seeds 0, 1 and 2), the 32K causal workload with tile selection, the 128K
chunked prefill (NVFP4 + Hadamard, selection) and the whole paged decode cache with its dual-residual
query (NVFP4 and MXFP4), the GPU's codes, block scales, tensor scales, per-token scales, P-fold data,
row norms, selection bitmaps and counts are compared bit for bit with the oracle's vectorised
quantizers and selector: every head and every row. The oracle runs per head in worker processes
(started fresh, so they hold no GPU state), each regenerating its head's inputs from the seeded
recipe.
"""
import multiprocessing as mp
import os
from concurrent.futures import ProcessPoolExecutor

import numpy as np
import pytest
import torch

import workloads as W
from oracle import quant as Q
from oracle import selection as S

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(900)]


@pytest.fixture(scope="module")
def fa4():
    import fp8_quantized_attention_amd as m
    return m


@pytest.fixture(scope="module")
def pool():
    n = max(1, min(16, len(os.sched_getaffinity(0)), os.cpu_count() or 1))
    with ProcessPoolExecutor(n, mp_context=mp.get_context("spawn")) as ex:
        yield ex


def _np(t):
    return t.detach().cpu().numpy()


def _fold_ref(sv):
    """Fold data of FP8 V from its per-token scales sv [L]: per 128-key tile the smallest power of two
    2^e with 448 * 2^e >= the tile's largest scale (found from that definition, by exponent search), and
    w = sv * 2^-e (exact)."""
    tiles = sv.reshape(-1, 128).astype(np.float64)
    sigma = tiles.max(axis=-1)
    e = np.full(sigma.shape, -127, np.int64)
    for _ in range(255):
        low = (448.0 * np.ldexp(1.0, e) < sigma) & (e < 127)
        if not low.any():
            break
        e = np.where(low, e + 1, e)
    return np.ldexp(1.0, e), (tiles * np.ldexp(1.0, -e)[:, None]).reshape(-1)


# ---------------------------------------------------------------------------------------- oracle workers

def _prefill_head_ref(cfg, seed, tensor, h):
    """Oracle outputs for one prefill head (worker process)."""
    x = W.prefill_head(cfg, tensor, 0, h, seed)
    if tensor == W.T_V:
        codes, sv = Q.fp8_per_token_quantize(x.float().numpy())
        fs, fw = _fold_ref(sv)
        return {"codes": codes, "scales": sv, "fold_scale": fs, "fold_w": fw}
    xf = x.float().numpy().astype(np.float64)
    xr = Q.hadamard_rotate(xf) if cfg.hadamard else xf
    out = {"norm2": Q.row_norm2(xf) if cfg.select else None}
    if cfg.qk_fmt == "mxfp4":
        out["codes"], out["block_scales"] = Q.mxfp4_quantize(xr)
    else:
        c, sb, st = Q.nvfp4_quantize(xr[None])
        out["codes"], out["block_scales"], out["tscale"] = c[0], sb[0], st[0]
    return out


def _cache_head_ref(cfg, tensor, b, h, L):
    """Oracle codes and scales of one (sequence, key head) of the paged decode cache (worker process)."""
    xf = W.decode_kv_head(cfg, tensor, b, h, L).float().numpy().astype(np.float64)
    if cfg.kv_fmt == "nvfp4":
        c, sb, st = Q.nvfp4_quantize(xf[None])
        return c[0], sb[0], st[0]
    c, sb = Q.mxfp4_quantize(xf)
    return c, sb, None


# ---------------------------------------------------------------------------------------- prefill

def _check_prefill(fa4, pool, cfg, seed):
    q, k, v = W.prefill_inputs(cfg, seed)
    fmt = {"mxfp4": fa4.FA4_MXFP4, "nvfp4": fa4.FA4_NVFP4}[cfg.qk_fmt]
    select = (5, 100) if cfg.select else None
    jobs = {(t, h): pool.submit(_prefill_head_ref, cfg, seed, t, h)
            for t, n in ((W.T_Q, cfg.Hq), (W.T_K, cfg.Hkv), (W.T_V, cfg.Hkv)) for h in range(n)}
    run = fa4.PrefillRunner(q.cuda(), k.cuda(), v.cuda(), cfg.causal, fmt=fmt, hadamard=cfg.hadamard, select=select)
    run.quantize()
    torch.cuda.synchronize()
    got = {W.T_Q: {key: (_np(t) if t is not None else None) for key, t in run.qq.items()},
           W.T_K: {key: (_np(t) if t is not None else None) for key, t in run.kq.items()},
           W.T_V: {key: _np(t) for key, t in run.vq.items()}}
    bitmap, counts = (_np(run.bitmap), _np(run.counts)) if select is not None else (None, None)
    del run
    torch.cuda.empty_cache()
    norms = {}
    for (t, h), job in jobs.items():
        ref, out = job.result(), got[t]
        what = (("q", "k", "v")[t], h)
        if t == W.T_V:
            assert np.array_equal(out["codes"][0, h], ref["codes"]), (what, "codes")
            assert np.array_equal(out["scales"][0, h], ref["scales"]), (what, "per-token scales")
            assert np.array_equal(out["fold_scale"][0, h].astype(np.float64), ref["fold_scale"]), (what, "fold scale")
            assert np.array_equal(out["fold_w"][0, h].astype(np.float64), ref["fold_w"]), (what, "fold w")
            continue
        assert np.array_equal(out["codes"][0, h], ref["codes"]), (what, "codes")
        assert np.array_equal(out["block_scales"][0, h], ref["block_scales"]), (what, "block scales")
        if cfg.qk_fmt == "nvfp4":
            assert out["scales"][h] == ref["tscale"], (what, "tensor scale")
        if select is not None:
            assert np.array_equal(out["norm2"][0, h], ref["norm2"]), (what, "row norms")
            norms[(t, h)] = ref["norm2"]
    if select is None:
        return
    group = cfg.Hq // cfg.Hkv
    for h in range(cfg.Hq):
        ref_bm, ref_cnt = S.select_tiles(norms[(W.T_Q, h)][None, None], norms[(W.T_K, h // group)][None, None],
                                         cfg.Lq, cfg.Lk, cfg.causal, 5, 100)
        assert counts[0, h] == ref_cnt[0, 0], (h, "count")
        assert np.array_equal(bitmap[0, h], ref_bm[0, 0]), (h, "bitmap")


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_prefill_4k_codes_full(fa4, pool, seed):
    _check_prefill(fa4, pool, W.C1, seed)


@pytest.mark.parametrize("cfg", [W.C2, W.C4], ids=["32k_select", "128k_chunk_nvfp4_hadamard_select"])
def test_prefill_select_codes_full(fa4, pool, cfg):
    _check_prefill(fa4, pool, cfg, 0)


# ---------------------------------------------------------------------------------------- decode

@pytest.mark.parametrize("base", [W.C3, W.C3_MX], ids=["nvfp4", "mxfp4"])
def test_decode_cache_and_query_full(fa4, pool, base):
    """The whole paged K/V cache of the decode workload (64 sequences, 8 key heads, contexts 8K-32K) and
    the dual-residual query, as the decode step quantizes them."""
    cfg = base
    lay = W.decode_layout(cfg)
    ctx, pt = lay.ctx_len.cuda(), lay.page_table.cuda()
    nv = cfg.kv_fmt == "nvfp4"
    fmt = fa4.FA4_NVFP4 if nv else fa4.FA4_MXFP4
    caches = []
    for tensor in (W.T_K, W.T_V):
        jobs = {(b, h): pool.submit(_cache_head_ref, cfg, tensor, b, h, int(lay.ctx_len[b]))
                for b in range(cfg.B) for h in range(cfg.Hkv)}
        x = W.decode_kv_padded(cfg, lay, tensor, device="cuda")
        out = fa4.quantize_paged(x, fmt, ctx, pt, lay.num_pages)
        torch.cuda.synchronize()
        caches.append(out)
        codes, scales = _np(out["codes"]), _np(out["block_scales"])
        tsc = _np(out["scales"]).reshape(cfg.B, cfg.Hkv) if nv else None
        del x
        torch.cuda.empty_cache()
        for (b, h), job in jobs.items():
            rc, rs, rt = job.result()
            L = int(lay.ctx_len[b])
            c = np.arange(L)
            phys = lay.page_table[b].numpy()[c // cfg.page_size]
            if nv:
                assert tsc[b, h] == rt, (tensor, b, h, "tensor scale")
            assert np.array_equal(codes[phys, h, c % cfg.page_size], rc), (tensor, b, h, "codes")
            assert np.array_equal(scales[phys, h, c % cfg.page_size], rs), (tensor, b, h, "block scales")
    q = W.decode_query(cfg)
    run = fa4.DecodeRunner(q.cuda(), caches[0], caches[1], pt, ctx, cfg.Hkv)
    run.quantize()
    torch.cuda.synchronize()
    rows = q.float().numpy().astype(np.float64).reshape(cfg.B * cfg.Hq, 1, cfg.d)
    if nv:
        (c1, s1, t1), (c2, s2, t2) = Q.dual_residual_quantize(rows)
        assert np.array_equal(_np(run.q1["scales"]), t1) and np.array_equal(_np(run.q2["scales"]), t2)
    else:
        (c1, s1), (c2, s2) = Q.dual_residual_quantize_mx(rows)
    n = cfg.B * cfg.Hq
    assert np.array_equal(_np(run.q1["codes"]).reshape(n, 1, -1), c1)
    assert np.array_equal(_np(run.q1["block_scales"]).reshape(n, 1, -1), s1)
    assert np.array_equal(_np(run.q2["codes"]).reshape(n, 1, -1), c2)
    assert np.array_equal(_np(run.q2["block_scales"]).reshape(n, 1, -1), s2)
