"""Prefill attention of the oracle: block-scaled QK^T, FP8 P and V, bf16 selected tiles.

TEST INFRASTRUCTURE: only the tests, the smoke check and the benchmark's
CPU-baseline leg may use this module. Shares no code with the GPU path.

Sources:
  * "MpFA QK4V8" (hotelren.com 6111405) sections 2.1-2.2 and 3.2-3.3: QK^T in
    4-bit with the per-group scales applied inside the product, V in 8-bit,
    softmax running max and sum kept in FP32 (here: float64 throughout).
  * "ThriftAttention" (ai-feeds.com summary), Method step 3: selected tiles are
    computed in high precision, the others in FP4, and both are merged through
    one online-softmax running max and sum.
  * "BitDecoding-FP4" (sns.style digest): the probabilities are quantized with
    a scale kept safe from underflow (here one scale per query row and
    128-key tile, taken from that tile's own row maximum).
  * "MXFP vs NVFP4" (tqpw.cn 81738) section 2.1: MX block scales are pure
    powers of two (E8M0). The per-tile scales of P and of the folded V scale
    below are read the same way, as powers of two.
  * "General notes on quantization" (zdszero), GEMM factoring: a low-precision
    product rescaled by the product of the operand scales; merging two scales
    into one (used to fold V's per-token scale into P).

Computation per (batch b, query head h, query row r), key head kv = h // (Hq/Hkv),
offset off = Lk - Lq (query r sits at key position off + r), scale = 1/sqrt(d),
tiles of 128 keys; column c of tile j is unmasked when not causal or c <= r + off:
  1. S_rc = scale * sum_d q~_rd k~_cd with the dequantized quantized Q/K, or
     with the original bf16 Q/K when tile j is selected; X_rc = S_rc log2(e).
  2. The tile's row scale is a power of two: r_rj = ceil(max of X_rc over the
     unmasked columns of tile j), and P'_rc = 2^(X_rc - r_rj) (0 for masked
     columns), so the row's largest P' lies in (1/2, 1].
  3. Unselected tile: sigma_j = max of s_v over the tile's keys; e_j = the smallest
     integer with 448 * 2^e_j >= sigma_j (clamped to [-127, 127]);
     w_c = s_v[c] * 2^-e_j (exact, <= 448); P^_rc = E4M3(P'_rc w_c) (one rounding
     from the float64 value); T_rj = 2^e_j sum_c P^_rc E4M3value(Vcode_c).
     Selected tile: T_rj = sum_c bf16(P'_rc) v_c with the original bf16 V.
  4. m_r = max_j r_rj, D_r = sum_j 2^(r_rj - m_r) sum_c P'_rc (unquantized P'),
     N_r = sum_j 2^(r_rj - m_r) T_rj; O_r = N_r / D_r (returned as float32),
     LSE_r = m_r ln 2 + ln D_r.
  MXFP4 probabilities with 4-bit V (p_fmt = "mxfp4", v_deq given): P^ = the MXFP4 quantization of P'
     over the same 32-key blocks (no per-token scale to fold, no 448), T_rj = sum_c P^_rc v_deq_c.
  MXFP4 probabilities (p_fmt = "mxfp4", FP8 V, unselected tiles): in step 3 P^ is the MXFP4
     quantization of the row of P'_rc w_c over 32 consecutive keys of the tile (keys 128 j + 32 b ..
     + 31): per block the MX scale 2^e_b (the smallest power of two with 6 * 2^e_b >= the block's
     largest P' w), codes E2M1(P' w 2^-e_b), P^ = code * 2^e_b; T_rj = 2^e_j sum_c P^_rc E4M3value(Vcode_c).
     ("BitDecoding-FP4": probabilities in FP4 under a scale that cannot underflow; "MXFP vs NVFP4"
     section 2.1: the MX block of 32 with an E8M0 scale. Blocks run along the keys, the contraction
     axis of PV, so a block-scaled product applies each block's scale.)
  4-bit V (v_deq given): V is MXFP4 with its 32-element blocks along the keys
     ("MpFA QK4V8" section 6 names 4-bit V as an extension without a format; blocks
     along the contraction axis of PV are the ones a block-scaled product can apply),
     v_deq its dequantized values. Unselected tile: P^_rc = E4M3(448 P'_rc),
     T_rj = (1/448) sum_c P^_rc v_deq_c.
Without rounding of P, every choice of the per-tile powers of two cancels and
O is exactly softmax(S) V. Because P' and P^ depend only on their own tile, the
result does not depend on the order in which tiles are visited;
`attend_rows_online` computes the same thing with a running maximum and sum.
"""
import numpy as np

from .formats import E4M3_MAX, bf16_round, e2m1_decode, e2m1_encode, e4m3_decode, e4m3_encode, fp32
from .quant import MX_BLOCK, mx_scale_exponent, mxfp4_dequantize, mxfp4_quantize

TILE = 128


def fold_exponent(sigma):
    """Smallest integer e with 448 * 2^e >= sigma (sigma > 0), clamped to [-127, 127] (exact
    comparisons: 448 * 2^e is exact in float64)."""
    e = int(np.ceil(np.log2(sigma / E4M3_MAX)))
    while E4M3_MAX * 2.0 ** (e - 1) >= sigma:
        e -= 1
    while E4M3_MAX * 2.0 ** e < sigma:
        e += 1
    return min(max(e, -127), 127)


def mxfp4_rows(x):
    """MXFP4 quantization of each row of x ([R, n], n a multiple of 32, values >= 0) over consecutive
    32-element blocks, returned dequantized (float64): the block-scaled quantizer of the inputs
    applied to the probabilities."""
    return mxfp4_dequantize(*mxfp4_quantize(x))


def mxfp4_tie_delta(arg, eps):
    """Per element of arg ([R, n] >= 0, 32-blocks along the last axis), the largest change of its MXFP4
    value when every element may be evaluated with a relative error up to its eps ([R, n]): each
    element may round to either neighbour of its perturbed argument, and the block scale may follow
    either end of the block maximum's range (a maximum within that error of 6 * 2^e). Returns [R, n]."""
    R, n = arg.shape
    a = arg.reshape(R, n // MX_BLOCK, MX_BLOCK)
    ep = eps.reshape(a.shape)
    amax = a.max(axis=-1)
    em = ep.max(axis=-1)
    e0 = mx_scale_exponent(amax)
    mid = e2m1_decode(e2m1_encode(a * np.ldexp(1.0, -e0)[..., None])) * np.ldexp(1.0, e0)[..., None]
    delta = np.zeros_like(a)
    for e in (mx_scale_exponent(amax * (1 - em)), e0, mx_scale_exponent(amax * (1 + em))):
        s = np.ldexp(1.0, e)[..., None]
        for f in (1 - ep, 1.0, 1 + ep):
            delta = np.maximum(delta, np.abs(e2m1_decode(e2m1_encode(a * f / s)) * s - mid))
    return delta.reshape(R, n)


def _tile_terms(S, unmasked, sel, vq_vals, s_v, v_orig, round_p=True, v_deq=None, p_fmt="fp8"):
    """Per-row (r, sum P', T) of one key tile, r the tile's power-of-two row reference in log2 units.
    S: [R, n] float64 scores (already scaled). v_deq: the tile's dequantized 4-bit V (else FP8 V).
    p_fmt: "fp8" (P^ in E4M3) or "mxfp4" (P^ in MXFP4 over 32-key blocks)."""
    X = np.where(unmasked, S * np.log2(np.e), -np.inf)
    has = unmasked.any(axis=1)
    r = np.where(has, np.ceil(X.max(axis=1, initial=-np.inf)), 0.0)
    P = np.where(unmasked, np.exp2(X - r[:, None]), 0.0)
    l = P.sum(axis=1)
    if sel:
        Pt = bf16_round(P) if round_p else P
        T = Pt @ v_orig
    elif v_deq is not None and p_fmt == "mxfp4":
        Ph = mxfp4_rows(P) if round_p else P
        T = Ph @ v_deq
    elif v_deq is not None:
        Ph = e4m3_decode(e4m3_encode(E4M3_MAX * P)) if round_p else E4M3_MAX * P
        T = (Ph @ v_deq) / E4M3_MAX
    else:
        e = fold_exponent(float(np.max(s_v)))
        w = s_v.astype(np.float64) * 2.0 ** -e
        Pw = P * w[None, :]
        if not round_p:
            Ph = Pw
        elif p_fmt == "mxfp4":
            Ph = mxfp4_rows(Pw)
        else:
            Ph = e4m3_decode(e4m3_encode(Pw))
        T = 2.0 ** e * (Ph @ vq_vals)
    return np.where(has, r, -np.inf), l, T


def _row_tiles(rows, Lq, Lk, causal, tile=TILE):
    """Key tiles visited by a group of rows from one q-tile (those holding an unmasked pair)."""
    off = Lk - Lq
    nk = Lk // tile
    i = rows[0] // tile
    if not causal:
        return list(range(nk))
    return [j for j in range(nk) if tile * j <= off + tile * i + tile - 1]


def attend_rows(rows, q_rows, k_deq, v_codes, s_v, scale, Lq, Lk, causal,
                q_orig_rows=None, k_orig=None, v_orig=None, sel_row=None, round_p=True,
                tile_order=None, v_deq=None, p_fmt="fp8"):
    """Two-pass O8 for a group of query rows that all lie in one 128-row q-tile.

    rows: [R] query indices; q_rows: [R, d] dequantized Q; k_deq: [Lk, d];
    v_codes: [Lk, d] E4M3 codes; s_v: [Lk] float32; sel_row: [nk] bool for
    this q-tile (None = nothing selected); v_deq: [Lk, d] dequantized 4-bit V (then
    v_codes and s_v are not used). Returns (O [R, d] float64, LSE [R]).
    """
    rows = np.asarray(rows)
    off = Lk - Lq
    vq_vals = e4m3_decode(v_codes) if v_deq is None else None
    tiles = _row_tiles(rows, Lq, Lk, causal)
    if tile_order is not None:
        tiles = [tiles[t] for t in tile_order]
    ms, ls, Ts = [], [], []
    for j in tiles:
        cs = np.arange(j * TILE, (j + 1) * TILE)
        unmasked = np.ones((len(rows), TILE), dtype=bool) if not causal else (cs[None, :] <= rows[:, None] + off)
        sel = bool(sel_row[j]) if sel_row is not None else False
        if sel:
            S = scale * (q_orig_rows @ k_orig[cs].T)
        else:
            S = scale * (q_rows @ k_deq[cs].T)
        m, l, T = _tile_terms(S, unmasked, sel, None if vq_vals is None else vq_vals[cs],
                              None if s_v is None else s_v[cs], v_orig[cs] if sel else None, round_p,
                              None if v_deq is None else v_deq[cs], p_fmt)
        ms.append(m); ls.append(l); Ts.append(T)
    M = np.stack(ms, axis=0)                       # [J, R] log2 units
    mrow = M.max(axis=0)
    f = np.exp2(M - mrow[None, :])                 # 2^(r_j - m), 0 for empty tiles
    D = (f * np.stack(ls, axis=0)).sum(axis=0)
    N = (f[:, :, None] * np.stack(Ts, axis=0)).sum(axis=0)
    return N / D[:, None], mrow * np.log(2.0) + np.log(D)


def attend_rows_online(rows, q_rows, k_deq, v_codes, s_v, scale, Lq, Lk, causal,
                       q_orig_rows=None, k_orig=None, v_orig=None, sel_row=None, round_p=True,
                       tile_order=None, v_deq=None, p_fmt="fp8"):
    """The same computation as attend_rows with a running max m, sum l and accumulator acc.

    For each tile (log2 units): m_new = max(m, r); acc = acc 2^(m - m_new) + T 2^(r - m_new);
    l = l 2^(m - m_new) + (sum P') 2^(r - m_new).
    """
    rows = np.asarray(rows)
    off = Lk - Lq
    vq_vals = e4m3_decode(v_codes) if v_deq is None else None
    tiles = _row_tiles(rows, Lq, Lk, causal)
    if tile_order is not None:
        tiles = [tiles[t] for t in tile_order]
    R, d = len(rows), (v_codes if v_deq is None else v_deq).shape[1]
    m = np.full(R, -np.inf)
    l = np.zeros(R)
    acc = np.zeros((R, d))
    for j in tiles:
        cs = np.arange(j * TILE, (j + 1) * TILE)
        unmasked = np.ones((R, TILE), dtype=bool) if not causal else (cs[None, :] <= rows[:, None] + off)
        sel = bool(sel_row[j]) if sel_row is not None else False
        S = scale * ((q_orig_rows @ k_orig[cs].T) if sel else (q_rows @ k_deq[cs].T))
        mt, lt, T = _tile_terms(S, unmasked, sel, None if vq_vals is None else vq_vals[cs],
                                None if s_v is None else s_v[cs], v_orig[cs] if sel else None, round_p,
                                None if v_deq is None else v_deq[cs], p_fmt)
        m_new = np.maximum(m, mt)
        a_old = np.where(np.isfinite(m), np.exp2(m - m_new), 0.0)
        a_new = np.where(np.isfinite(mt), np.exp2(mt - m_new), 0.0)
        acc = acc * a_old[:, None] + T * a_new[:, None]
        l = l * a_old + lt * a_new
        m = m_new
    return acc / l[:, None], m * np.log(2.0) + np.log(l)


def rounding_slack(rows, q_rows, k_deq, v_codes, s_v, scale, Lq, Lk, causal,
                   q_orig_rows=None, k_orig=None, v_orig=None, sel_row=None, v_deq=None, p_fmt="fp8"):
    """Per-row, per-column bound [R, d] on how far O moves when probability roundings that lie within the
    FP32 evaluation error of a rounding midpoint go to the other neighbour.

    The pages keep the softmax in FP32 ("MpFA QK4V8" section 3.3); `attend_rows` evaluates it in float64.
    A computation in FP32 reaches the rounded value (E4M3 of P' w_c, E4M3 of 448 P', bf16 of P') from an
    argument that differs from the float64 one by a relative amount of at most
        eps_rc = ln 2 * dX_rc + 2^-22 + 2^-24,   u = 2^-24,
        dX_rc = log2(e) * scale * (d / 8) u sum_i |q_ri| |k_ci| + 4 u |X_rc| + u |X_rc - r_rj|.
    The rounding model: the d products are exact in FP32 (4-, 8- and 16-bit operands) and are summed by
    matrix-core steps of 16 products that round at most twice each (d / 8 roundings along any path); the
    score-to-log2 factor carries up to 3 roundings (scale, log2(e), tensor scales) and the shifted argument
    one more; then two units in the last place for the exponential and one for the fold factor. Where the rounding of the argument times (1 - eps) or (1 + eps) differs from the
    float64 rounding, both neighbours are correct results. Each such element adds its larger rounding
    difference, times the absolute values of its V row as the tile's T uses them, weighted as in step 4:
        slack_r = (1 / D_r) sum_j 2^(r_rj - m_r) sum_c delta_rc |V_c|.
    The denominator D uses the unrounded P' and moves only by the evaluation error itself.
    MXFP4 probabilities (p_fmt = "mxfp4"): an element's FP4 rounding may go either way as above, and the
    block's scale either way when the block maximum lies within its error of a scale boundary
    (`mxfp4_tie_delta`).
    """
    rows = np.asarray(rows)
    off = Lk - Lq
    u = 2.0 ** -24
    d = (v_codes if v_deq is None else v_deq).shape[1]
    vq_vals = e4m3_decode(v_codes) if v_deq is None else None
    ms, ls, Ss = [], [], []
    for j in _row_tiles(rows, Lq, Lk, causal):
        cs = np.arange(j * TILE, (j + 1) * TILE)
        unmasked = np.ones((len(rows), TILE), dtype=bool) if not causal else (cs[None, :] <= rows[:, None] + off)
        sel = bool(sel_row[j]) if sel_row is not None else False
        qq, kk = (q_orig_rows, k_orig[cs]) if sel else (q_rows, k_deq[cs])
        S = scale * (qq @ kk.T)
        A = np.abs(qq) @ np.abs(kk).T
        X = np.where(unmasked, S * np.log2(np.e), -np.inf)
        has = unmasked.any(axis=1)
        r = np.where(has, np.ceil(X.max(axis=1, initial=-np.inf)), 0.0)
        P = np.where(unmasked, np.exp2(X - r[:, None]), 0.0)
        Xf = np.where(unmasked, X, 0.0)
        dX = np.log2(np.e) * scale * (d / 8) * u * A + 4 * u * np.abs(Xf) + u * np.abs(Xf - r[:, None])
        eps = np.log(2.0) * dX + 2.0 ** -22 + 2.0 ** -24
        if sel:
            rnd, arg, vabs, unit = bf16_round, P, np.abs(v_orig[cs]), 1.0
        elif v_deq is not None:
            rnd, arg, vabs, unit = (lambda x: e4m3_decode(e4m3_encode(x))), E4M3_MAX * P, np.abs(v_deq[cs]), 1.0 / E4M3_MAX
        else:
            e = fold_exponent(float(np.max(s_v[cs])))
            w = s_v[cs].astype(np.float64) * 2.0 ** -e
            rnd, arg, vabs, unit = (lambda x: e4m3_decode(e4m3_encode(x))), P * w[None, :], np.abs(vq_vals[cs]), 2.0 ** e
        if p_fmt == "mxfp4" and not sel and v_deq is not None:
            arg, vabs, unit = P, np.abs(v_deq[cs]), 1.0
            delta = mxfp4_tie_delta(arg, np.where(unmasked, eps, 0.0))
        elif p_fmt == "mxfp4" and not sel:
            delta = mxfp4_tie_delta(arg, np.where(unmasked, eps, 0.0))
        else:
            mid = rnd(arg)
            delta = np.maximum(np.abs(rnd(arg * (1 - eps)) - mid), np.abs(rnd(arg * (1 + eps)) - mid))
        delta = np.where(unmasked, delta, 0.0)
        ms.append(np.where(has, r, -np.inf))
        ls.append(P.sum(axis=1))
        Ss.append(unit * (delta @ vabs))
    M = np.stack(ms, axis=0)
    mrow = M.max(axis=0)
    f = np.exp2(M - mrow[None, :])
    D = (f * np.stack(ls, axis=0)).sum(axis=0)
    return (f[:, :, None] * np.stack(Ss, axis=0)).sum(axis=0) / D[:, None]


def prefill_rounding_slack(q_deq, k_deq, v_codes, s_v, causal, scale=None, q_orig=None, k_orig=None, v_orig=None,
                           bitmap=None, rows=None, heads=None, v_deq=None, p_fmt="fp8"):
    """`rounding_slack` over a batch, with the arguments and layout of `attention_prefill`; returns
    float64 [B, Hq, R, d]."""
    B, Hq, Lq, d = q_deq.shape
    Hkv, Lk = k_deq.shape[1], k_deq.shape[2]
    group = Hq // Hkv
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    rows = np.arange(Lq) if rows is None else np.asarray(rows)
    heads = [(b, h) for b in range(B) for h in range(Hq)] if heads is None else heads
    out = np.zeros((B, Hq, len(rows), d))
    qtile = rows // TILE
    for (b, h) in heads:
        kv = h // group
        for i in np.unique(qtile):
            sel_idx = np.nonzero(qtile == i)[0]
            rr = rows[sel_idx]
            out[b, h, sel_idx] = rounding_slack(
                rr, q_deq[b, h, rr], k_deq[b, kv], None if v_codes is None else v_codes[b, kv],
                None if s_v is None else s_v[b, kv], scale, Lq, Lk, causal,
                q_orig_rows=None if q_orig is None else q_orig[b, h, rr],
                k_orig=None if k_orig is None else k_orig[b, kv],
                v_orig=None if v_orig is None else v_orig[b, kv],
                sel_row=bitmap[b, h, i] if bitmap is not None else None,
                v_deq=None if v_deq is None else v_deq[b, kv], p_fmt=p_fmt)
    return out


def attention_prefill(q_deq, k_deq, v_codes, s_v, causal, scale=None,
                      q_orig=None, k_orig=None, v_orig=None, bitmap=None,
                      rows=None, heads=None, round_p=True, v_deq=None, p_fmt="fp8"):
    """O8 over a batch: q_deq [B, Hq, Lq, d]; k_deq [B, Hkv, Lk, d]; v_codes [B, Hkv, Lk, d]
    (E4M3 codes, token-major); s_v [B, Hkv, Lk]; optional originals (bf16 values as float64)
    and bitmap [B, Hq, nq, nk]; v_deq [B, Hkv, Lk, d]: dequantized 4-bit V instead of v_codes, s_v;
    p_fmt: "fp8" or "mxfp4" (the probabilities of the unselected tiles).

    rows: optional array of query rows to compute (default all); heads: optional
    list of (b, h) pairs (default all). Returns (O float32 [B, Hq, R, d],
    LSE float32 [B, Hq, R]) with R = len(rows); heads not listed stay zero.
    """
    B, Hq, Lq, d = q_deq.shape
    Hkv, Lk = k_deq.shape[1], k_deq.shape[2]
    group = Hq // Hkv
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    rows = np.arange(Lq) if rows is None else np.asarray(rows)
    heads = [(b, h) for b in range(B) for h in range(Hq)] if heads is None else heads
    O = np.zeros((B, Hq, len(rows), d), dtype=np.float32)
    LSE = np.zeros((B, Hq, len(rows)), dtype=np.float32)
    qtile = rows // TILE
    for (b, h) in heads:
        kv = h // group
        for i in np.unique(qtile):
            sel_idx = np.nonzero(qtile == i)[0]
            rr = rows[sel_idx]
            sel_row = bitmap[b, h, i] if bitmap is not None else None
            o, lse = attend_rows(
                rr, q_deq[b, h, rr], k_deq[b, kv], None if v_codes is None else v_codes[b, kv],
                None if s_v is None else s_v[b, kv], scale, Lq, Lk, causal,
                q_orig_rows=None if q_orig is None else q_orig[b, h, rr],
                k_orig=None if k_orig is None else k_orig[b, kv],
                v_orig=None if v_orig is None else v_orig[b, kv],
                sel_row=sel_row, round_p=round_p, v_deq=None if v_deq is None else v_deq[b, kv], p_fmt=p_fmt)
            O[b, h, sel_idx] = fp32(o)
            LSE[b, h, sel_idx] = fp32(lse)
    return O, LSE


def attention_reference(q, k, v, causal, scale=None):
    """Unquantized softmax(scale q k^T + mask) v in float64 (q: [..., Lq, d], k/v: [..., Lk, d]).

    Used to report the error that quantization adds; not a parity gate.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    Lq, d = q.shape[-2], q.shape[-1]
    Lk = k.shape[-2]
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    S = scale * (q @ np.swapaxes(k, -1, -2))
    if causal:
        r = np.arange(Lq)[:, None]
        c = np.arange(Lk)[None, :]
        S = np.where(c <= r + (Lk - Lq), S, -np.inf)
    S = S - S.max(axis=-1, keepdims=True)
    P = np.exp(S)
    return (P @ v) / P.sum(axis=-1, keepdims=True)
