"""The C ABI without a GPU: the library loads, exports what include/fa4.h declares, the ctypes mirror
matches the C struct layouts, and invalid arguments are rejected before anything is enqueued."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa4.h")

fa4 = pytest.importorskip("fp8_quantized_attention_amd")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fa4_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_function():
    names = _declared_functions()
    assert set(names) == set(fa4.EXPORTS)
    for n in names:
        assert hasattr(fa4.lib, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", fa4.LIB_PATH], capture_output=True, text=True).stdout
    for n in names:
        assert re.search(rf"\bT {n}\b", out), f"{n} not exported"


def test_struct_layouts_match_header(tmp_path):
    structs = {"fa4_qinput": fa4.QInput, "fa4_qoutput": fa4.QOutput, "fa4_attn_args": fa4.AttnArgs,
               "fa4_decode_args": fa4.DecodeArgs}
    lines = ['#include <stdio.h>', '#include <stddef.h>', f'#include "{HEADER}"', "int main(void) {"]
    for cname, py in structs.items():
        lines.append(f'printf("{cname} %zu\\n", sizeof({cname}));')
        for fname, _ in py._fields_:
            lines.append(f'printf("{cname}.{fname} %zu\\n", offsetof({cname}, {fname}));')
    lines.append("return 0; }")
    src = tmp_path / "layout.c"
    src.write_text("\n".join(lines))
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-std=c99", "-o", str(exe), str(src)], check=True)
    got = dict(l.split() for l in subprocess.run([str(exe)], capture_output=True, text=True).stdout.split("\n") if l)
    for cname, py in structs.items():
        assert int(got[cname]) == ctypes.sizeof(py), cname
        for fname, _ in py._fields_:
            assert int(got[f"{cname}.{fname}"]) == getattr(py, fname).offset, f"{cname}.{fname}"


def test_status_strings():
    assert fa4.lib.fa4_status_string(0) == b"ok"
    assert fa4.lib.fa4_status_string(fa4.FA4_ERR_WORKSPACE) == b"workspace too small"


def _q(**kw):
    base = dict(x=16, dtype=fa4.FA4_BF16, d=128, outer=1, heads=2, rows=256, stride_outer=2 * 256 * 128,
                stride_head=256 * 128, stride_row=128, row_counts=None, page_table=None, page_size=0,
                max_pages=0, num_pages=0, channel_scale=None)
    base.update(kw)
    return fa4.QInput(*[base[f] for f, _ in fa4.QInput._fields_])


def _call_q(qin, fmt=fa4.FA4_MXFP4, flags=0, codes=256, bs=256, sc=256, res=None, norm=None):
    qout = fa4.QOutput(fmt, codes, bs, sc)
    return fa4.lib.fa4_quantize_blockscaled(ctypes.byref(qin), flags, ctypes.byref(qout),
                                            ctypes.byref(res) if res is not None else None, norm, None)


def test_quantize_rejects_before_launch():
    assert fa4.lib.fa4_quantize_blockscaled(None, 0, None, None, None, None) == fa4.FA4_ERR_NULL
    assert _call_q(_q(d=96)) == fa4.FA4_ERR_UNSUPPORTED
    assert _call_q(_q(dtype=7)) == fa4.FA4_ERR_UNSUPPORTED
    assert _call_q(_q(), fmt=9) == fa4.FA4_ERR_UNSUPPORTED
    # MXFP4_KEYS (4-bit V): no flags, paging or row norms; rows in multiples of 32
    assert _call_q(_q(), fmt=fa4.FA4_MXFP4_KEYS, flags=fa4.FA4_HADAMARD128) == fa4.FA4_ERR_UNSUPPORTED
    assert _call_q(_q(rows=40, stride_head=40 * 128, stride_outer=2 * 40 * 128), fmt=fa4.FA4_MXFP4_KEYS) == \
        fa4.FA4_ERR_SHAPE
    assert _call_q(_q(), fmt=fa4.FA4_MXFP4_KEYS, norm=256) == fa4.FA4_ERR_UNSUPPORTED
    assert _call_q(_q(page_table=256, page_size=64, max_pages=4, num_pages=8), fmt=fa4.FA4_MXFP4_KEYS) == \
        fa4.FA4_ERR_UNSUPPORTED
    assert _call_q(_q(), fmt=fa4.FA4_MXFP4_KEYS, bs=None) == fa4.FA4_ERR_NULL
    assert _call_q(_q(x=None)) == fa4.FA4_ERR_NULL
    assert _call_q(_q(x=18)) == fa4.FA4_ERR_ALIGN
    assert _call_q(_q(x=24)) == fa4.FA4_ERR_ALIGN                     # 8-byte aligned is not enough
    assert _call_q(_q(stride_row=130)) == fa4.FA4_ERR_ALIGN
    assert _call_q(_q(stride_row=132)) == fa4.FA4_ERR_ALIGN          # bf16 rows: multiples of 8 elements
    assert _call_q(_q(), codes=None) == fa4.FA4_ERR_NULL
    assert _call_q(_q(), fmt=fa4.FA4_NVFP4, sc=None) == fa4.FA4_ERR_NULL
    assert _call_q(_q(d=64), flags=fa4.FA4_HADAMARD128) == fa4.FA4_ERR_UNSUPPORTED
    assert _call_q(_q(), fmt=fa4.FA4_FP8_TOKEN, flags=fa4.FA4_DUAL_RESIDUAL) == fa4.FA4_ERR_UNSUPPORTED
    assert _call_q(_q(), flags=fa4.FA4_DUAL_RESIDUAL) == fa4.FA4_ERR_NULL                # residual missing
    assert _call_q(_q(), fmt=fa4.FA4_NVFP4, flags=fa4.FA4_DUAL_RESIDUAL) == fa4.FA4_ERR_NULL
    res = fa4.QOutput(fa4.FA4_NVFP4, 256, 256, 256)                                      # format mismatch
    assert _call_q(_q(), flags=fa4.FA4_DUAL_RESIDUAL, res=res) == fa4.FA4_ERR_UNSUPPORTED
    res = fa4.QOutput(fa4.FA4_MXFP4, 264, 256, None)                                     # MXFP4: no scales
    assert _call_q(_q(), flags=fa4.FA4_DUAL_RESIDUAL, res=res) == fa4.FA4_ERR_ALIGN
    assert _call_q(_q(), flags=1 << 5) == fa4.FA4_ERR_UNSUPPORTED
    assert _call_q(_q(), fmt=fa4.FA4_FP8_TOKEN, flags=fa4.FA4_SCALE_SEARCH) == fa4.FA4_ERR_UNSUPPORTED
    assert _call_q(_q(), flags=fa4.FA4_SCALE_SEARCH | fa4.FA4_DUAL_RESIDUAL) == fa4.FA4_ERR_UNSUPPORTED
    assert _call_q(_q(channel_scale=258)) == fa4.FA4_ERR_ALIGN
    assert _call_q(_q(outer=70000)) == fa4.FA4_ERR_SHAPE
    assert _call_q(_q(page_table=64, page_size=64, max_pages=2, num_pages=4)) == fa4.FA4_ERR_SHAPE  # rows > 128
    assert b"rows=256" in fa4.lib.fa4_last_error()
    qout = fa4.QOutput(fa4.FA4_MXFP4, 256, 256, 256, 256, 256)                # fold data needs FP8
    assert fa4.lib.fa4_quantize_blockscaled(ctypes.byref(_q()), 0, ctypes.byref(qout), None, None, None) \
        == fa4.FA4_ERR_UNSUPPORTED
    qout = fa4.QOutput(fa4.FA4_FP8_TOKEN, 256, None, 256, 256, 256)
    assert fa4.lib.fa4_quantize_blockscaled(ctypes.byref(_q(rows=200)), 0, ctypes.byref(qout), None, None, None) \
        == fa4.FA4_ERR_UNSUPPORTED
    assert _call_q(_q(rows=0)) == fa4.FA4_OK                # nothing to do, no launch
    assert fa4.lib.fa4_last_error() == b""


def _call_qp(q=None, k=None, v=None, qf=fa4.FA4_MXFP4, kf=None, vout=None, qn=None, kn=None):
    q, k, v = q or _q(), k or _q(), v or _q()
    qo = fa4.QOutput(qf, 256, 256, None)
    ko = fa4.QOutput(qf if kf is None else kf, 256, 256, None)
    vo = vout or fa4.QOutput(fa4.FA4_FP8_TOKEN, 256, None, 256, 256, 256)
    return fa4.lib.fa4_quantize_prefill(*[ctypes.byref(t) for t in (q, k, v, qo, ko, vo)], qn, kn, None)


def test_quantize_prefill_rejects_before_launch():
    assert fa4.lib.fa4_quantize_prefill(None, None, None, None, None, None, None, None, None) == fa4.FA4_ERR_NULL
    assert _call_qp(qf=fa4.FA4_NVFP4) == fa4.FA4_ERR_UNSUPPORTED                 # Q/K: MXFP4 or MXFP8 only
    assert _call_qp(kf=fa4.FA4_MXFP8) == fa4.FA4_ERR_UNSUPPORTED                 # Q and K alike
    assert _call_qp(vout=fa4.QOutput(fa4.FA4_FP8_TOKEN, 256, None, 256)) == fa4.FA4_ERR_UNSUPPORTED   # no fold
    assert _call_qp(vout=fa4.QOutput(fa4.FA4_MXFP4, 256, 256, None, 256, 256)) == fa4.FA4_ERR_UNSUPPORTED
    v4 = fa4.QOutput(fa4.FA4_MXFP4_KEYS, 256, 256, None)                      # 4-bit V: MXFP4 Q/K, d = 128
    assert _call_qp(qf=fa4.FA4_MXFP8, vout=v4) == fa4.FA4_ERR_UNSUPPORTED
    assert _call_qp(q=_q(d=64, stride_row=64), k=_q(d=64, stride_row=64), v=_q(d=64, stride_row=64), vout=v4) == \
        fa4.FA4_ERR_UNSUPPORTED
    assert _call_qp(v=_q(rows=40, stride_head=40 * 128, stride_outer=2 * 40 * 128), vout=v4) == fa4.FA4_ERR_SHAPE
    assert _call_qp(k=_q(dtype=fa4.FA4_F32)) == fa4.FA4_ERR_UNSUPPORTED
    assert _call_qp(v=_q(d=64, stride_row=64)) == fa4.FA4_ERR_UNSUPPORTED
    assert _call_qp(k=_q(page_table=256, page_size=64, max_pages=4, num_pages=8)) == fa4.FA4_ERR_UNSUPPORTED
    assert _call_qp(v=_q(row_counts=256)) == fa4.FA4_ERR_UNSUPPORTED
    assert _call_qp(qn=256) == fa4.FA4_ERR_UNSUPPORTED                           # norms of both or neither
    assert _call_qp(v=_q(rows=200)) == fa4.FA4_ERR_UNSUPPORTED                   # V rows in whole 128-row tiles
    assert _call_qp(q=_q(x=None)) == fa4.FA4_ERR_NULL
    assert _call_qp(k=_q(x=24)) == fa4.FA4_ERR_ALIGN
    assert _call_qp(q=_q(rows=0), k=_q(rows=0), v=_q(rows=0)) == fa4.FA4_OK      # nothing to do, no launch
    assert fa4.lib.fa4_last_error() == b""


def test_smoothing_rejects_before_launch():
    f = lambda q, k, qs=256, ks=256: fa4.lib.fa4_smoothing_factors(ctypes.byref(q), ctypes.byref(k), qs, ks, None)
    q, k = _q(heads=8), _q(heads=2)
    assert fa4.lib.fa4_smoothing_factors(None, ctypes.byref(k), 256, 256, None) == fa4.FA4_ERR_NULL
    assert f(q, k, qs=None) == fa4.FA4_ERR_NULL
    assert f(_q(heads=7), k) == fa4.FA4_ERR_SHAPE                    # Hq not a multiple of Hkv
    assert f(q, _q(heads=2, d=64, stride_row=64)) == fa4.FA4_ERR_SHAPE   # d differs
    assert f(q, _q(heads=2, page_table=64, page_size=64, max_pages=4, num_pages=4)) == fa4.FA4_ERR_UNSUPPORTED
    assert f(q, _q(heads=2, x=24)) == fa4.FA4_ERR_ALIGN
    assert f(q, k, ks=258) == fa4.FA4_ERR_ALIGN
    assert f(_q(heads=8, dtype=5), k) == fa4.FA4_ERR_UNSUPPORTED


def _attn(**kw):
    base = dict(fmt=fa4.FA4_MXFP4, q_codes=256, q_scales=256, q_tscale=None, k_codes=256, k_scales=256,
                k_tscale=None, v_codes=256, v_scales=256, v_fold_w=256, v_fold_scale=256, q_bf16=None, k_bf16=None, v_bf16=None, bitmap=None,
                B=1, Hq=4, Hkv=2, Lq=256, Lk=512, d=128, causal=1, softmax_scale=0.088, o=256, lse=None,
                v_fmt=0, v_block_scales=None, p_fmt=fa4.FA4_P_FP8)
    base.update(kw)
    return fa4.AttnArgs(*[base[f] for f, _ in fa4.AttnArgs._fields_])


def test_attention_rejects_before_launch():
    call = lambda a: fa4.lib.fa4_attn_fwd(ctypes.byref(a), None)
    assert fa4.lib.fa4_attn_fwd(None, None) == fa4.FA4_ERR_NULL
    assert call(_attn(fmt=5)) == fa4.FA4_ERR_UNSUPPORTED
    assert call(_attn(Hq=3)) == fa4.FA4_ERR_SHAPE
    assert call(_attn(Lq=200)) == fa4.FA4_ERR_SHAPE
    assert call(_attn(Lq=1024, Lk=512)) == fa4.FA4_ERR_SHAPE          # causal with Lq > Lk
    assert call(_attn(d=96)) == fa4.FA4_ERR_UNSUPPORTED
    assert call(_attn(d=64, bitmap=256)) == fa4.FA4_ERR_UNSUPPORTED
    assert call(_attn(fmt=fa4.FA4_NVFP4, d=64)) == fa4.FA4_ERR_UNSUPPORTED
    assert call(_attn(fmt=fa4.FA4_NVFP4)) == fa4.FA4_ERR_NULL         # tensor scales missing
    assert call(_attn(bitmap=256)) == fa4.FA4_ERR_NULL                # bf16 originals missing
    assert call(_attn(o=None)) == fa4.FA4_ERR_NULL
    assert call(_attn(v_fold_w=None)) == fa4.FA4_ERR_NULL
    assert call(_attn(v_codes=264)) == fa4.FA4_ERR_ALIGN
    assert call(_attn(softmax_scale=0.0)) == fa4.FA4_ERR_SHAPE
    assert call(_attn(Lq=0)) == fa4.FA4_OK
    # 4-bit V: MXFP4 Q/K, d = 128; its E8M0 scales replace v_scales and the fold data
    v4 = dict(v_fmt=fa4.FA4_MXFP4_KEYS, v_scales=None, v_fold_w=None, v_fold_scale=None, v_block_scales=256)
    assert call(_attn(v_fmt=7)) == fa4.FA4_ERR_UNSUPPORTED
    assert call(_attn(**v4, bitmap=256)) == fa4.FA4_ERR_NULL            # selection needs the bf16 originals
    assert call(_attn(**v4, bitmap=256, q_bf16=256, k_bf16=256, v_bf16=256, Lq=0)) == fa4.FA4_OK
    assert call(_attn(**v4, fmt=fa4.FA4_NVFP4, q_tscale=256, k_tscale=256)) == fa4.FA4_ERR_UNSUPPORTED
    assert call(_attn(**{**v4, "v_block_scales": None})) == fa4.FA4_ERR_NULL
    assert call(_attn(**{**v4, "v_block_scales": 260})) == fa4.FA4_ERR_ALIGN
    assert call(_attn(**v4, Lq=0)) == fa4.FA4_OK
    # MXFP4 probabilities: MXFP4 Q/K, FP8 V, d = 128 (validated before the empty-shape early return)
    assert call(_attn(p_fmt=fa4.FA4_P_NVFP4)) == fa4.FA4_ERR_UNSUPPORTED
    assert call(_attn(p_fmt=9)) == fa4.FA4_ERR_UNSUPPORTED
    assert call(_attn(p_fmt=fa4.FA4_P_MXFP4, **v4, Lq=0)) == fa4.FA4_OK         # 4-bit V x FP4 P
    assert call(_attn(p_fmt=fa4.FA4_P_MXFP4, **v4, d=64)) == fa4.FA4_ERR_UNSUPPORTED
    assert call(_attn(p_fmt=fa4.FA4_P_MXFP4, fmt=fa4.FA4_NVFP4, q_tscale=256, k_tscale=256)) == fa4.FA4_ERR_UNSUPPORTED
    assert call(_attn(p_fmt=fa4.FA4_P_MXFP4, fmt=fa4.FA4_MXFP8)) == fa4.FA4_ERR_UNSUPPORTED
    assert call(_attn(p_fmt=fa4.FA4_P_MXFP4, d=64)) == fa4.FA4_ERR_UNSUPPORTED
    assert call(_attn(p_fmt=fa4.FA4_P_MXFP4, v_fold_w=None)) == fa4.FA4_ERR_NULL
    assert call(_attn(p_fmt=fa4.FA4_P_MXFP4, Lq=0)) == fa4.FA4_OK


def test_select_rejects_before_launch():
    f = fa4.lib.fa4_select_tiles
    assert f(256, 256, 1, 4, 3, 256, 256, 1, 5, 100, 256, None, None) == fa4.FA4_ERR_SHAPE
    assert f(256, 256, 1, 4, 2, 200, 256, 1, 5, 100, 256, None, None) == fa4.FA4_ERR_SHAPE
    assert f(256, 256, 1, 4, 2, 256, 256, 1, 101, 100, 256, None, None) == fa4.FA4_ERR_SHAPE
    assert f(256, 256, 1, 4, 2, 256, 128, 1, 5, 100, 256, None, None) == fa4.FA4_ERR_SHAPE
    assert f(256, 256, 1, 4, 2, 128 * 2048, 128 * 2048, 0, 5, 100, 256, None, None) == fa4.FA4_ERR_SHAPE
    assert f(None, 256, 1, 4, 2, 256, 256, 1, 5, 100, 256, None, None) == fa4.FA4_ERR_NULL


def _dec(**kw):
    base = dict(fmt=fa4.FA4_NVFP4, q1_codes=256, q1_scales=256, q1_tscale=256, q2_codes=256, q2_scales=256,
                q2_tscale=256,
                k_codes=256, k_scales=256, v_codes=256, v_scales=256, k_tscale=256, v_tscale=256,
                page_table=256, ctx_len=256, B=4, Hq=32, Hkv=8, d=128, page_size=64, max_pages=8, num_pages=32,
                softmax_scale=0.088, o=256, p_fmt=fa4.FA4_P_FP8, d_v=0)
    base.update(kw)
    return fa4.DecodeArgs(*[base[f] for f, _ in fa4.DecodeArgs._fields_])


def test_decode_rejects_before_launch():
    call = lambda a, ws=512, n=1 << 30: fa4.lib.fa4_decode_paged(ctypes.byref(a), ws, n, None)
    a = _dec()
    need = fa4.lib.fa4_decode_workspace_bytes(ctypes.byref(a))
    assert need == 4 * 8 * 1 * 4 * 130 * 4
    assert call(_dec(d=64)) == fa4.FA4_ERR_UNSUPPORTED
    assert call(_dec(page_size=32)) == fa4.FA4_ERR_UNSUPPORTED
    assert call(_dec(Hq=12)) == fa4.FA4_ERR_UNSUPPORTED               # not a multiple of Hkv = 8
    assert call(_dec(Hq=8 * 65)) == fa4.FA4_ERR_UNSUPPORTED           # more than 64 query heads per key head
    # groups of up to 4 query heads per workgroup: 8 per key head take two groups' partials
    assert fa4.lib.fa4_decode_workspace_bytes(ctypes.byref(_dec(Hq=64))) == 2 * need
    assert fa4.lib.fa4_decode_workspace_bytes(ctypes.byref(_dec(Hq=16))) == need
    assert fa4.lib.fa4_decode_workspace_bytes(ctypes.byref(_dec(Hq=8))) == need
    assert call(_dec(k_codes=None)) == fa4.FA4_ERR_NULL
    assert call(_dec(k_codes=264)) == fa4.FA4_ERR_ALIGN
    assert call(a, ws=512, n=need - 1) == fa4.FA4_ERR_WORKSPACE
    assert call(a, ws=None, n=need) == fa4.FA4_ERR_WORKSPACE
    assert call(a, ws=520, n=need) == fa4.FA4_ERR_ALIGN
    assert call(_dec(B=0)) == fa4.FA4_OK
    assert call(_dec(fmt=fa4.FA4_FP8_TOKEN)) == fa4.FA4_ERR_UNSUPPORTED
    assert call(_dec(p_fmt=2)) == fa4.FA4_ERR_UNSUPPORTED
    assert call(_dec(p_fmt=fa4.FA4_P_NVFP4), ws=512, n=need - 1) == fa4.FA4_ERR_WORKSPACE
    # NVFP4 needs its tensor scales; MXFP4 has none (the pointers are not read) and 4-byte scale rows
    assert call(_dec(v_tscale=None)) == fa4.FA4_ERR_NULL
    mx = dict(fmt=fa4.FA4_MXFP4, q1_tscale=None, q2_tscale=None, k_tscale=None, v_tscale=None)
    assert call(_dec(**mx), ws=512, n=need - 1) == fa4.FA4_ERR_WORKSPACE
    assert call(_dec(k_scales=260)) == fa4.FA4_ERR_ALIGN
    assert call(_dec(k_scales=260, **mx), ws=None, n=need) == fa4.FA4_ERR_WORKSPACE
    assert call(_dec(k_scales=258, **mx)) == fa4.FA4_ERR_ALIGN


def test_mla_decode_rejects_before_launch():
    call = lambda a, ws=512, n=1 << 30: fa4.lib.fa4_decode_paged(ctypes.byref(a), ws, n, None)
    mla = dict(fmt=fa4.FA4_MXFP4, d=576, d_v=512, Hq=16, Hkv=1, max_pages=60, q1_tscale=None, q2_tscale=None,
               k_tscale=None, v_tscale=None, v_codes=None, v_scales=None)
    a = _dec(**mla)
    need = fa4.lib.fa4_decode_workspace_bytes(ctypes.byref(a))
    assert need == 4 * 2 * 16 * 514 * 4                     # B x ceil(60 / 40) splits x heads x (m, l, O)
    assert call(a, ws=512, n=need - 1) == fa4.FA4_ERR_WORKSPACE
    assert call(a, ws=520, n=need) == fa4.FA4_ERR_ALIGN
    assert call(_dec(**{**mla, "fmt": fa4.FA4_NVFP4})) == fa4.FA4_ERR_UNSUPPORTED
    assert call(_dec(**{**mla, "p_fmt": fa4.FA4_P_NVFP4})) == fa4.FA4_ERR_UNSUPPORTED
    assert call(_dec(**{**mla, "Hq": 32})) == fa4.FA4_ERR_UNSUPPORTED
    assert call(_dec(**{**mla, "d": 128})) == fa4.FA4_ERR_UNSUPPORTED
    assert call(_dec(**{**mla, "d_v": 256})) == fa4.FA4_ERR_UNSUPPORTED
    assert call(_dec(**{**mla, "k_scales": 264})) == fa4.FA4_ERR_ALIGN
    assert call(_dec(**{**mla, "k_codes": None})) == fa4.FA4_ERR_NULL
    assert call(_dec(**{**mla, "B": 0})) == fa4.FA4_OK


def test_decode_noalloc_rejects_before_any_gpu_call():
    """fa4_decode_paged_noalloc checks its scratch need against the fixed size before it touches a device:
    NULL args, and shapes whose split partials exceed FA4_DECODE_SCRATCH_BYTES, are refused with nothing
    enqueued (no GPU here)."""
    assert fa4.lib.fa4_decode_paged_noalloc(None, None) == fa4.FA4_ERR_NULL
    text = open(HEADER).read()
    m = re.search(r"#define FA4_DECODE_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == fa4.DECODE_SCRATCH_BYTES
    # 64 sequences of up to 128K tokens, 8 key heads: 64 splits of 2048 keys each
    a = fa4.DecodeArgs(fa4.FA4_NVFP4, 16, 16, 16, 16, 16, 16, 16, 16, 16, 16, 16, 16, 16, 16,
                       64, 32, 8, 128, 64, 2048, 131072, 0.088, 16, fa4.FA4_P_FP8, 0)
    need = fa4.lib.fa4_decode_workspace_bytes(ctypes.byref(a))
    assert need > fa4.DECODE_SCRATCH_BYTES
    assert fa4.lib.fa4_decode_paged_noalloc(ctypes.byref(a), None) == fa4.FA4_ERR_WORKSPACE
    assert b"scratch" in fa4.lib.fa4_last_error()
