"""Oracle-side construction of reference results for the workloads (CPU only, float64).

Everything here starts from workloads.py's seeded inputs and calls only oracle/; nothing comes from
the GPU path. Per-head helpers keep the full-size workloads affordable: only the heads whose rows are
sampled are quantized and attended on the CPU.
"""
import numpy as np

import workloads as W
from oracle import attention as A
from oracle import decode as Dd
from oracle import formats as F
from oracle import outlier as OA
from oracle import quant as Q
from oracle import selection as S

# Parity bar for attention outputs: relative L2 and max-abs relative to max|O|.
REL_L2 = 1e-3
MAX_ABS = 2e-3


def rel_errors(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    rel = np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300)
    mx = np.abs(got - ref).max() / max(np.abs(ref).max(), 1e-300)
    return rel, mx


def assert_parity(got, ref, what="", slack=None):
    """rel-L2 <= REL_L2 and max-abs <= MAX_ABS max|ref|. slack: optional per-element allowance (the oracle's
    bound on probability roundings that are ties within FP32 evaluation error), added to the max-abs bar."""
    rel, mx = rel_errors(got, ref)
    if slack is not None:
        excess = np.maximum(np.abs(np.asarray(got, np.float64) - ref) - slack, 0.0)
        mx = excess.max() / max(np.abs(ref).max(), 1e-300)
    assert rel <= REL_L2 and mx <= MAX_ABS, f"{what}: rel-L2 {rel:.3e} max-abs/max {mx:.3e}"
    return rel, mx


def quant_head(cfg, x, rotate, scale=None, search=False):
    """Dequantized Q or K values of one head ([L, d] float64) under the workload's Q/K format.
    scale: optional per-channel smoothing factors [d] (float32 products); search: per-block scale search."""
    if scale is not None:
        x = F.fp32(x * np.asarray(scale, np.float64)).astype(np.float64)
    xr = Q.hadamard_rotate(x) if rotate else x
    if cfg.qk_fmt == "mxfp4":
        return Q.mxfp4_dequantize(*(OA.mxfp4_quantize_search(xr) if search else Q.mxfp4_quantize(xr)))
    if cfg.qk_fmt == "mxfp8":
        return Q.mxfp8_dequantize(*Q.mxfp8_quantize(xr))
    return Q.nvfp4_dequantize(*(OA.nvfp4_quantize_search(xr[None]) if search else Q.nvfp4_quantize(xr[None])))[0]


def prefill_reference(cfg, seed, heads, rows, select=None, q_all=None, k_all=None, v_all=None, smooth=None,
                      search=False, slack=False):
    """Oracle O and LSE for the listed (b, h) pairs and query rows.

    select = (num, den) enables tile selection (norms, tile maxima and top-k from the oracle).
    smooth = (q_scale [Hq, d], k_scale [Hkv, d]) static smoothing factors; search: K's scale search.
    q_all/k_all/v_all: optional host tensors already generated (else chunks are regenerated).
    Returns (O [len(heads), R, d], LSE [len(heads), R], bitmaps {(b, h): [nq, nk]}), and with slack=True
    also the oracle's rounding-tie allowance [len(heads), R, d] (attention.rounding_slack).
    """
    group = cfg.Hq // cfg.Hkv
    rows = np.asarray(rows)
    outs, lses, bitmaps, slacks = [], [], {}, []
    kv_cache = {}
    for (b, h) in heads:
        kvh = h // group
        q = (q_all[b, h] if q_all is not None else W.prefill_head(cfg, W.T_Q, b, h, seed)).double().numpy()
        if (b, kvh) not in kv_cache:
            k = (k_all[b, kvh] if k_all is not None else W.prefill_head(cfg, W.T_K, b, kvh, seed)).double().numpy()
            v = (v_all[b, kvh] if v_all is not None else W.prefill_head(cfg, W.T_V, b, kvh, seed)).double().numpy()
            kd = quant_head(cfg, k, cfg.hadamard, None if smooth is None else smooth[1][kvh], search)
            if cfg.v_fmt == "mxfp4k":
                vc, sv, vd = None, None, Q.mxfp4_keys_dequantize(*Q.mxfp4_keys_quantize(v))
            else:
                (vc, sv), vd = Q.fp8_per_token_quantize(v), None
            kn = Q.row_norm2(k)
            kv_cache = {(b, kvh): (k, v, kd, vc, sv, vd, kn)}
        k, v, kd, vc, sv, vd, kn = kv_cache[(b, kvh)]
        qd = quant_head(cfg, q, cfg.hadamard, None if smooth is None else smooth[0][h])
        bm = None
        if select is not None:
            qn = Q.row_norm2(q)
            bm, _ = S.select_tiles(qn[None, None], kn[None, None], cfg.Lq, cfg.Lk, cfg.causal, select[0], select[1])
            bm = bm[0, 0]
            bitmaps[(b, h)] = bm
        O, L = A.attention_prefill(qd[None, None], kd[None, None], None if vc is None else vc[None, None],
                                   None if sv is None else sv[None, None], cfg.causal,
                                   q_orig=q[None, None], k_orig=k[None, None], v_orig=v[None, None],
                                   bitmap=None if bm is None else bm[None, None], rows=rows,
                                   v_deq=None if vd is None else vd[None, None], p_fmt=cfg.p_fmt)
        outs.append(O[0, 0]); lses.append(L[0, 0])
        if slack:
            slacks.append(A.prefill_rounding_slack(
                qd[None, None], kd[None, None], None if vc is None else vc[None, None],
                None if sv is None else sv[None, None], cfg.causal, q_orig=q[None, None], k_orig=k[None, None],
                v_orig=v[None, None], bitmap=None if bm is None else bm[None, None], rows=rows,
                v_deq=None if vd is None else vd[None, None], p_fmt=cfg.p_fmt)[0, 0])
    if slack:
        return np.stack(outs), np.stack(lses), bitmaps, np.stack(slacks)
    return np.stack(outs), np.stack(lses), bitmaps


def decode_cache(cfg, layout, seed, pairs_only=None):
    """Oracle pages of K and V in cfg.kv_fmt (NVFP4 or MXFP4), quantized per (sequence, key head) and
    scattered by the page table.

    pairs_only: optional set of (b, kvh) to build (others stay zero). Returns
    ((kc, ks), (vc, vs), k_tscale, v_tscale, dequantized logical rows {(tensor, b, kvh): [L, d]}).
    """
    d, ps = cfg.d, cfg.page_size
    P = layout.num_pages
    nv = cfg.kv_fmt == "nvfp4"
    kc = np.zeros((P, cfg.Hkv, ps, d // 2), np.uint8)
    ks = np.zeros((P, cfg.Hkv, ps, d // (16 if nv else 32)), np.uint8)
    vc = np.zeros_like(kc); vs = np.zeros_like(ks)
    kt = np.zeros((cfg.B, cfg.Hkv), np.float32); vt = np.zeros_like(kt)
    logical = {}
    for b in range(cfg.B):
        L = int(layout.ctx_len[b])
        if L <= 0:
            continue
        c = np.arange(L)
        phys = layout.page_table[b].numpy()[c // ps]
        for h in range(cfg.Hkv):
            if pairs_only is not None and (b, h) not in pairs_only:
                continue
            for tensor, (codes, scales, ts) in [(W.T_K, (kc, ks, kt)), (W.T_V, (vc, vs, vt))]:
                x = W.decode_kv_head(cfg, tensor, b, h, L, seed).double().numpy()
                if nv:
                    qc, qs, qt = Q.nvfp4_quantize(x[None])
                    codes[phys, h, c % ps] = qc[0]
                    scales[phys, h, c % ps] = qs[0]
                    ts[b, h] = qt[0]
                    logical[(tensor, b, h)] = Q.nvfp4_dequantize(qc, qs, qt)[0]
                else:
                    qc, qs = Q.mxfp4_quantize(x)
                    codes[phys, h, c % ps] = qc
                    scales[phys, h, c % ps] = qs
                    logical[(tensor, b, h)] = Q.mxfp4_dequantize(qc, qs)
    return (kc, ks), (vc, vs), kt, vt, logical


def decode_query_quant(cfg, seed):
    q = W.decode_query(cfg, seed).double().numpy()
    rows = q.reshape(cfg.B * cfg.Hq, 1, cfg.d)
    return q, (Q.dual_residual_quantize(rows) if cfg.kv_fmt == "nvfp4" else Q.dual_residual_quantize_mx(rows))


def decode_reference(cfg, seed, layout, pairs, logical, q1, q2, scale=None):
    """Oracle O for the listed (b, h) pairs from contiguous dequantized rows (softmax scale 1/sqrt(d)
    unless given)."""
    scale = 1.0 / np.sqrt(cfg.d) if scale is None else scale
    qhat = Dd.dequant_query(q1, q2, cfg.kv_fmt).reshape(cfg.B, cfg.Hq, cfg.d)
    group = cfg.Hq // cfg.Hkv
    out = []
    for (b, h) in pairs:
        if int(layout.ctx_len[b]) <= 0:
            out.append(np.zeros(cfg.d, np.float32))      # empty context (decode_one)
            continue
        kh = logical[(W.T_K, b, h // group)]
        vh = logical[(W.T_V, b, h // group)]
        out.append(Dd.decode_one(qhat[b, h], kh, vh, scale, p_fmt=cfg.p_fmt).astype(np.float32))
    return np.stack(out)


def mla_cache(cfg, layout, seed, seqs=None):
    """Oracle MLA latent cache: each sequence's rows (576 wide) MXFP4-quantized per token and laid out
    in column-sliced pages [P][9][64][32] / [P][9][64][2]; seqs: optional subset of sequences to build
    (the rest stay zero). Returns (codes, scales, {b: (rows float64, codes [L, 288], scales [L, 18])})."""
    ns = cfg.d // 64
    codes = np.zeros((layout.num_pages, ns, cfg.page_size, 32), np.uint8)
    scales = np.zeros((layout.num_pages, ns, cfg.page_size, 2), np.uint8)
    rows = {}
    for b in (range(cfg.B) if seqs is None else seqs):
        L = int(layout.ctx_len[b])
        if L <= 0:
            continue
        x = W.decode_kv_head(cfg, W.T_K, b, 0, L, seed).double().numpy()
        qc, qs = Q.mxfp4_quantize(x)
        c = np.arange(L)
        phys = layout.page_table[b].numpy()[c // cfg.page_size]
        codes[phys, :, c % cfg.page_size] = qc.reshape(L, ns, 32)
        scales[phys, :, c % cfg.page_size] = qs.reshape(L, ns, 2)
        rows[b] = (x, qc, qs)
    return codes, scales, rows


def mla_query_quant(cfg, seed):
    q = W.decode_query(cfg, seed).double().numpy()
    return q, Q.dual_residual_quantize_mx(q.reshape(cfg.B * cfg.Hq, cfg.d))
