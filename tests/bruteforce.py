"""Pure-Python brute force of the oracle's steps, for tiny shapes only.

Written independently of oracle/: formats round by scanning every code for the
nearest value (ties to the even code, i.e. the one whose last mantissa bit is
0), scales are found by searching their definition, attention is explicit
loops over rows, tiles and keys with Python floats (IEEE double). The tests
compare the vectorised oracle against these loops.
"""
import math
import struct


def f32(x):
    """Round a Python float to the nearest float32."""
    return struct.unpack("<f", struct.pack("<f", x))[0]


def _e2m1_value(code):
    s = -1.0 if code & 8 else 1.0
    e = (code >> 1) & 3
    m = code & 1
    return s * (0.5 * m if e == 0 else 2.0 ** (e - 1) * (1 + m / 2))


def _e4m3_value(code):
    s = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 15
    m = code & 7
    if e == 15 and m == 7:
        return float("nan")
    return s * (m * 2.0 ** -9 if e == 0 else 2.0 ** (e - 7) * (1 + m / 8))


E2M1 = [(c, _e2m1_value(c)) for c in range(8)]
E4M3 = [(c, _e4m3_value(c)) for c in range(127)]


def _nearest(a, table):
    best = None
    for c, v in table:
        dist = abs(a - v)
        if best is None or dist < best[1] or (dist == best[1] and c % 2 == 0):
            best = (c, dist)
    return best[0]


def e2m1_encode(x):
    sign = 8 if math.copysign(1.0, x) < 0 else 0
    return sign | _nearest(min(abs(x), 6.0), E2M1)


def e4m3_encode(x):
    sign = 0x80 if math.copysign(1.0, x) < 0 else 0
    return sign | _nearest(min(abs(x), 448.0), E4M3)


def e2m1_value(c):
    return _e2m1_value(c)


def e4m3_value(c):
    return _e4m3_value(c)


def mx_exponent(amax):
    """Smallest e in [-127, 127] with 6 * 2^e >= amax, by search."""
    if amax == 0:
        return -127
    e = -127
    while 6.0 * 2.0 ** e < amax and e < 127:
        e += 1
    return e


def mxfp4_row(x):
    """One row (list of floats) -> (codes list, E8M0 bytes list)."""
    codes, scales = [], []
    for b0 in range(0, len(x), 32):
        blk = x[b0:b0 + 32]
        e = mx_exponent(max(abs(v) for v in blk))
        scales.append(e + 127)
        codes += [e2m1_encode(v * 2.0 ** -e) for v in blk]
    return codes, scales


def mxfp4_row_values(codes, scales):
    return [e2m1_value(c) * 2.0 ** (scales[i // 32] - 127) for i, c in enumerate(codes)]


def nvfp4_group(rows):
    """rows: list of rows (floats, already float32 values) -> (codes, block scales, tensor scale)."""
    amax_t = max((abs(v) for r in rows for v in r), default=0.0)
    st = f32(amax_t / 2688.0)
    if st == 0:                      # amax_t == 0, or a quotient that underflows float32
        st = 1.0
    six_st = f32(6.0 * st)
    codes, sbs = [], []
    for r in rows:
        rc, rs = [], []
        for b0 in range(0, len(r), 16):
            blk = r[b0:b0 + 16]
            sb = e4m3_encode(f32(max(abs(v) for v in blk) / six_st))
            rs.append(sb)
            denom = f32(e4m3_value(sb) * st)
            for v in blk:
                if denom == 0:
                    rc.append(8 if math.copysign(1.0, v) < 0 else 0)
                else:
                    rc.append(e2m1_encode(f32(v / denom)))
        codes.append(rc)
        sbs.append(rs)
    return codes, sbs, st


def nvfp4_values(codes, sbs, st):
    return [[e2m1_value(c) * e4m3_value(sbs[i][j // 16]) * st for j, c in enumerate(row)]
            for i, row in enumerate(codes)]


def fp8_token(row):
    amax = max(abs(v) for v in row)
    sv = 1.0 if amax == 0 else f32(amax / 448.0)
    return [e4m3_encode(f32(v / sv)) for v in row], sv


def bf16(x):
    """Nearest bfloat16 to a double (8 significant bits), ties to even, by scanning neighbours."""
    if x == 0:
        return x
    m, e = math.frexp(abs(x))
    q = 2.0 ** (max(e, -125) - 8)
    lo = math.floor(abs(x) / q) * q
    hi = lo + q
    a = abs(x)
    if a - lo < hi - a:
        r = lo
    elif hi - a < a - lo:
        r = hi
    else:
        r = lo if (lo / q) % 2 == 0 else hi
    return math.copysign(r, x)


def attention_rows(rows, Q, K, Vc, sv, Qo, Ko, Vo, sel, Lq, Lk, causal, scale, round_p=True, Vd=None,
                   p_fmt="fp8"):
    """O8 by loops. Q/K: dequantized rows (lists); Vc: E4M3 codes; sv: per-key scales;
    Qo/Ko/Vo: original values for selected tiles; sel(i, j) -> bool. Vd: dequantized 4-bit V rows
    (then P^ = E4M3(448 P), T = sum P^ v / 448, and Vc, sv are not used). p_fmt "mxfp4": the tile's
    P' w (FP8 V) or P' (4-bit V) is MXFP4-quantized over blocks of 32 consecutive keys by mxfp4_row
    (masked keys 0), T = sum P^ v.
    Returns output rows."""
    off = Lk - Lq
    d = len((Vc if Vd is None else Vd)[0])
    out = []
    for r in rows:
        i = r // 128
        terms = []
        for j in range(Lk // 128):
            cols = [c for c in range(128 * j, 128 * j + 128) if (not causal) or c <= r + off]
            if not cols:
                continue
            s_sel = sel(i, j)
            S = {}
            for c in cols:
                a, b = (Qo[r], Ko[c]) if s_sel else (Q[r], K[c])
                S[c] = scale * sum(a[t] * b[t] for t in range(d))
            # row reference: the smallest integer >= the tile's largest score in log2 units
            x = {c: S[c] / math.log(2.0) for c in cols}
            m = math.ceil(max(x.values()))
            P = {c: 2.0 ** (x[c] - m) for c in cols}
            T = [0.0] * d
            if s_sel:
                for c in cols:
                    p = bf16(P[c]) if round_p else P[c]
                    for t in range(d):
                        T[t] += p * Vo[c][t]
            elif Vd is not None and p_fmt == "mxfp4" and round_p:
                row = [P.get(c, 0.0) for c in range(128 * j, 128 * j + 128)]
                vals = mxfp4_row_values(*mxfp4_row(row))
                for c in cols:
                    for t in range(d):
                        T[t] += vals[c - 128 * j] * Vd[c][t]
            elif Vd is not None:
                for c in cols:
                    p = e4m3_value(e4m3_encode(448.0 * P[c])) if round_p else 448.0 * P[c]
                    for t in range(d):
                        T[t] += p * Vd[c][t]
                T = [v / 448.0 for v in T]
            else:
                sigma = max(sv[128 * j:128 * j + 128])
                e = -127                              # smallest e with 448 * 2^e >= sigma
                while 448.0 * 2.0 ** e < sigma:
                    e += 1
                pw = {c: P[c] * sv[c] * 2.0 ** -e for c in cols}
                if round_p and p_fmt == "mxfp4":
                    row = [pw.get(c, 0.0) for c in range(128 * j, 128 * j + 128)]
                    vals = mxfp4_row_values(*mxfp4_row(row))
                    ph = {c: vals[c - 128 * j] for c in cols}
                elif round_p:
                    ph = {c: e4m3_value(e4m3_encode(pw[c])) for c in cols}
                else:
                    ph = pw
                for c in cols:
                    for t in range(d):
                        T[t] += ph[c] * e4m3_value(Vc[c][t])
                T = [2.0 ** e * v for v in T]
            terms.append((m, sum(P.values()), T))
        mm = max(t[0] for t in terms)
        D = sum(2.0 ** (t[0] - mm) * t[1] for t in terms)
        out.append([sum(2.0 ** (t[0] - mm) * t[2][k] for t in terms) / D for k in range(d)])
    return out


def decode_row(q, K, V, scale, round_p=True, p_fmt="fp8", tile=128, pow2_ref=False):
    """O9 by loops for one query row over len(K) keys, tiles of `tile` keys from 0 (V rows may be
    shorter than K rows). p_fmt "nvfp4": each tile's probabilities (largest exactly 1) form one NVFP4
    group, P^ its values, T = sum P^ v. pow2_ref: each tile's reference is 2^r, r the smallest
    integer >= the largest score in log2 units (P = 2^(S log2 e - r)), merged with weights 2^(r - max r)."""
    d = len(V[0])
    terms = []
    for t0 in range(0, len(K), tile):
        cols = range(t0, min(t0 + tile, len(K)))
        S = {c: scale * sum(q[t] * K[c][t] for t in range(len(q))) for c in cols}
        if pow2_ref:
            r = math.ceil(max(S[c] / math.log(2.0) for c in cols))
            P = {c: 2.0 ** (S[c] / math.log(2.0) - r) for c in cols}
            m = r * math.log(2.0)
        else:
            m = max(S.values())
            P = {c: math.exp(S[c] - m) for c in cols}
        T = [0.0] * d
        if round_p and p_fmt == "nvfp4":
            codes, sbs, st = nvfp4_group([[f32(P[c]) for c in cols]])
            ph = dict(zip(cols, nvfp4_values(codes, sbs, st)[0]))
            for c in cols:
                for t in range(d):
                    T[t] += 448.0 * ph[c] * V[c][t]
        else:
            for c in cols:
                p = e4m3_value(e4m3_encode(448.0 * P[c])) if round_p else 448.0 * P[c]
                for t in range(d):
                    T[t] += p * V[c][t]
        terms.append((m, sum(P.values()), [v / 448.0 for v in T]))
    mm = max(t[0] for t in terms)
    D = sum(math.exp(t[0] - mm) * t[1] for t in terms)
    return [sum(math.exp(t[0] - mm) * t[2][k] for t in terms) / D for k in range(d)]


def select_by_sort(a, b, valid, k):
    """Top-k tiles by (score desc, linear index asc) using Python's sort. a: [nq], b: [nk] floats."""
    nk = len(b)
    cand = []
    for i in range(len(a)):
        for j in range(nk):
            if valid(i, j):
                cand.append((-f32(a[i] * b[j]), i * nk + j))
    cand.sort()
    return sorted(idx for _, idx in cand[:k])
