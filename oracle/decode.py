"""Decode attention of the oracle over a paged FP4 KV cache (NVFP4 or MXFP4) with a dual-residual query.

TEST INFRASTRUCTURE: only the tests, the smoke check and the benchmark's
CPU-baseline leg may use this module. Shares no code with the GPU path.

Source: "BitDecoding-FP4: native FP4 KV-cache decoding" (sns.style digest):
the KV cache is stored in 4-bit microscaling form in pages; the query is split
into two FP4 tensors, the second carrying the residual of the first; the
probabilities are quantized with a scale that cannot underflow to zero; the
query heads sharing one key head (GQA) are processed together. "MpFA QK4V8"
(hotelren.com 6111405) section 3.3: FP32-or-better running max and sum.

Computation per (batch b, query head h), key head kv = h // (Hq/Hkv), keys
c in [0, L_b) (the query attends to every cached token), scale = 1/sqrt(d):
  q^ = dequant(Q1) + dequant(Q2) (float64); k^, v^ = dequantized cache rows;
  S_c = scale * q^ . k^_c; tiles of 128 keys from position 0 (the last may be partial);
  per tile: m~ = max S_c, P'_c = exp(S_c - m~), P^_c = E4M3(448 P'_c),
  T = (1/448) sum_c P^_c v^_c;
  m = max m~, D = sum e^(m~ - m) sum P', N = sum e^(m~ - m) T, O = N / D (float32).
The page table maps logical page p of sequence b (tokens 64p .. 64p+63) to a
physical page; a physical page holds [Hkv][64][...] rows.

Formats of the cache (the page reports both): NVFP4 (E4M3 scale per 16
elements along d and an FP32 tensor scale per (sequence, key head)) or MXFP4
(E8M0 scale per 32 elements along d, no tensor scale). The query residuals take
the cache's format. The probability steps are the same for both.

Probability format (p_fmt): "fp8" is the default above. "nvfp4" quantizes the
probabilities to FP4 with E4M3 block scales, the case in which the digest says
a block scale can round to zero for long contexts. The underflow-aware reading
used here: each tile row of P' is normalized to its own maximum (so that
maximum is exactly 1) and taken as one NVFP4 group, blocks of 16 consecutive
keys from the tile start. The group's tensor scale is then fl32(1/2688), which
puts a block whose maximum is amax_b at the E4M3 scale E4M3(~448 amax_b); a
block scale reaches zero only when amax_b < 2^-10 / 448, a block that carries
under 2.2e-6 of the tile's largest probability. P^ = the NVFP4 values
(code * s_b * s_t, approximately P') and T = sum_c P^_c v^_c.
"""
import numpy as np

from .formats import E4M3_MAX, e4m3_decode, e4m3_encode, fp32
from .quant import mxfp4_dequantize, nvfp4_dequantize, nvfp4_quantize

TILE = 128


def gather_pages(pages, page_table_b, L, page_size, kvh):
    """Logical rows [L, ...] of key head kvh for one sequence, read through its page table."""
    c = np.arange(L)
    phys = np.asarray(page_table_b)[c // page_size]
    return pages[phys, kvh, c % page_size]


def quantize_p_nvfp4(p):
    """P^ of one tile row p (float64, largest element exactly 1, at most 128 keys) in NVFP4: the
    row is one group (tensor scale from its amax 1), E4M3 scales per 16 keys from the row start; a
    ragged row is padded with zeros, which leaves every block maximum unchanged. Returns the
    dequantized values (float64, same length as p)."""
    n = len(p)
    x = np.concatenate([np.asarray(p, np.float64), np.zeros((-n) % 16)])[None, None, :]
    codes, sb, st = nvfp4_quantize(x)
    return nvfp4_dequantize(codes, sb, st)[0, 0, :n]


def decode_one(q_hat, k_hat, v_hat, scale, chunk=None, round_p=True, p_fmt="fp8", tile=TILE, pow2_ref=False):
    """O for one query row against L keys (v_hat may be narrower than k_hat). chunk: optional split
    length (multiple of the tile) whose partial results (m, l, O) are merged afterwards; the merged
    result equals the single pass. p_fmt: "fp8" (P^ = E4M3(448 P')) or "nvfp4" (quantize_p_nvfp4).
    tile: keys per probability tile (128; one 64-key page for the MLA geometry).
    An empty context (L = 0) has no softmax; its output is defined as zero (the pages do not cover it).
    pow2_ref: the tile reference is a power of two instead of the tile maximum (the prefill's rule,
    "MpFA QK4V8" section 3.3 per-tile P scaling): with x = S log2(e), r = ceil(max x), P' = 2^(x - r)
    (largest value in (1/2, 1]) and the tiles merge with exact weights 2^(r_j - max_j r_j)."""
    L = k_hat.shape[0]
    if L == 0:
        return np.zeros(v_hat.shape[1])   # no cached token: the softmax is empty and O is defined as 0
    if chunk is None:
        chunk = max(L, 1)
    assert chunk % tile == 0 or chunk >= L
    parts = []
    for s0 in range(0, L, chunk):
        ms, ls, Ts = [], [], []
        for t0 in range(s0, min(s0 + chunk, L), tile):
            cs = np.arange(t0, min(t0 + tile, L, s0 + chunk))
            S = scale * (k_hat[cs] @ q_hat)
            if pow2_ref:
                X = S * np.log2(np.e)
                r = np.ceil(X.max())
                P = np.exp2(X - r)
                m = r * np.log(2.0)              # merged below through exp(m_j - max m) = 2^(r_j - max r)
            else:
                m = S.max()
                P = np.exp(S - m)
            if not round_p:
                T = P @ v_hat[cs]
            elif p_fmt == "nvfp4":
                T = quantize_p_nvfp4(P) @ v_hat[cs]
            else:
                T = (e4m3_decode(e4m3_encode(E4M3_MAX * P)) @ v_hat[cs]) / E4M3_MAX
            ms.append(m); ls.append(P.sum()); Ts.append(T)
        M = np.array(ms)
        mm = M.max()
        f = np.exp(M - mm)
        parts.append((mm, (f * np.array(ls)).sum(), (f[:, None] * np.array(Ts)).sum(axis=0)))
    mm = max(p[0] for p in parts)
    D = sum(np.exp(p[0] - mm) * p[1] for p in parts)
    N = sum(np.exp(p[0] - mm) * p[2] for p in parts)
    return N / D


def dequant_query(q1, q2, fmt="nvfp4"):
    """q^ = dequant(Q1) + dequant(Q2): NVFP4 pairs (codes, sb, st) or MXFP4 pairs (codes, E8M0)."""
    deq = nvfp4_dequantize if fmt == "nvfp4" else mxfp4_dequantize
    return deq(*q1) + deq(*q2)


def decode_paged(q1, q2, k_pages, v_pages, k_tscale, v_tscale, page_table, ctx_len,
                 Hq, Hkv, page_size=64, scale=None, pairs=None, chunk=None, round_p=True, fmt="nvfp4",
                 p_fmt="fp8"):
    """O9 through the page table.

    fmt "nvfp4": q1, q2 = (codes [B*Hq, 1, d/2], block scales [B*Hq, 1, d/16], tensor scales
    [B*Hq]); k_pages / v_pages = (codes [P, Hkv, page_size, d/2], block scales [P, Hkv,
    page_size, d/16]); k_tscale / v_tscale [B, Hkv] float32.
    fmt "mxfp4": q1, q2 = (codes, E8M0 scales [B*Hq, 1, d/32]); pages hold E8M0 scales
    [P, Hkv, page_size, d/32]; the tensor-scale arguments are unused.
    p_fmt: probability format, "fp8" or "nvfp4" (decode_one).
    Returns O float32 [B, Hq, d]; pairs (optional) restricts the computed (b, h) pairs, the rest
    stay zero.
    """
    B = len(ctx_len)
    d = 2 * q1[0].shape[-1]
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    group = Hq // Hkv
    qhat = dequant_query(q1, q2, fmt).reshape(B, Hq, d)
    O = np.zeros((B, Hq, d), dtype=np.float32)
    pairs = [(b, h) for b in range(B) for h in range(Hq)] if pairs is None else pairs
    cache = {}
    for (b, h) in pairs:
        kv = h // group
        L = int(ctx_len[b])
        if L <= 0:
            continue                                  # empty context: O stays zero (decode_one)
        if (b, kv) not in cache:
            kc = gather_pages(k_pages[0], page_table[b], L, page_size, kv)
            ks = gather_pages(k_pages[1], page_table[b], L, page_size, kv)
            vc = gather_pages(v_pages[0], page_table[b], L, page_size, kv)
            vs = gather_pages(v_pages[1], page_table[b], L, page_size, kv)
            if fmt == "nvfp4":
                k_hat = nvfp4_dequantize(kc[None], ks[None], np.array([k_tscale[b, kv]]))[0]
                v_hat = nvfp4_dequantize(vc[None], vs[None], np.array([v_tscale[b, kv]]))[0]
            else:
                k_hat = mxfp4_dequantize(kc, ks)
                v_hat = mxfp4_dequantize(vc, vs)
            cache = {(b, kv): (k_hat, v_hat)}
        k_hat, v_hat = cache[(b, kv)]
        O[b, h] = fp32(decode_one(qhat[b, h], k_hat, v_hat, scale, chunk=chunk, round_p=round_p, p_fmt=p_fmt))
    return O


# ----------------------------------------------------------------------------------------------- MLA

MLA_SLICE = 64          # columns per slice of the latent cache's pages


def gather_mla_rows(codes, scales, page_table_b, L, page_size=64):
    """MXFP4 codes [L, d/2] and E8M0 scales [L, d/32] of one sequence's latent rows, read through its
    page table from column-sliced pages: codes [P][d/64][page_size][32], scales [P][d/64][page_size][2]
    (slice j holds columns 64 j .. 64 j + 63 of every row of the page)."""
    c = np.arange(L)
    phys = np.asarray(page_table_b)[c // page_size]
    rc = codes[phys, :, c % page_size]
    rs = scales[phys, :, c % page_size]
    return rc.reshape(L, -1), rs.reshape(L, -1)


def decode_mla(q1, q2, codes, scales, page_table, ctx_len, Hq, d_v, scale, page_size=64, pairs=None,
               chunk=None, round_p=True):
    """Decode in the MLA geometry ("BitDecoding-FP4" covers GQA and MLA attention; the geometry is
    not spelled out there): every query head of a sequence attends to one shared latent row per
    token, which is the key (all d values, the latent part and the rotary part) and whose first d_v
    values are the value. The cache is MXFP4 (E8M0 per 32 along the row); the query of each head is
    the dual residual pair (q1, q2 = (codes [B*Hq, d/2], E8M0 [B*Hq, d/32])) of its absorbed form.
    Probability tiles are one 64-key page, each with a power-of-two reference (decode_one's
    pow2_ref). Returns O float32 [B, Hq, d_v] (pairs: optional subset of (b, h) to compute; the rest
    stay zero)."""
    B = len(ctx_len)
    d = 2 * q1[0].shape[-1]
    qhat = (mxfp4_dequantize(*q1) + mxfp4_dequantize(*q2)).reshape(B, Hq, d)
    O = np.zeros((B, Hq, d_v), dtype=np.float32)
    pairs = [(b, h) for b in range(B) for h in range(Hq)] if pairs is None else pairs
    rows = {}
    for (b, h) in pairs:
        if int(ctx_len[b]) <= 0:
            continue                                  # empty context: O stays zero (decode_one)
        if b not in rows:
            k_hat = mxfp4_dequantize(*gather_mla_rows(codes, scales, page_table[b], int(ctx_len[b]), page_size))
            rows = {b: k_hat}
        k_hat = rows[b]
        O[b, h] = fp32(decode_one(qhat[b, h], k_hat, k_hat[:, :d_v], scale, chunk=chunk, round_p=round_p,
                                  tile=page_size, pow2_ref=True))
    return O
