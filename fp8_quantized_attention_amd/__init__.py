"""Python binding of libfa4 (block-scaled low-bit fused attention on MI355X / gfx950).

Argument marshalling only: every step of the path runs in the HIP kernels behind the C ABI declared
in include/fa4.h. torch provides device memory and the current HIP stream. If the built library is
missing, importing this package raises: there is no fallback implementation.
"""
import ctypes
import math
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# FA4_LIBRARY may name another build of the same library (the sanitizer build of the host code)
LIB_PATH = os.environ.get("FA4_LIBRARY") or os.path.join(_HERE, "libfa4.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built; run `python fp8_quantized_attention_amd/build.py` "
                      "(or __graft_entry__.build()) first")
lib = ctypes.CDLL(LIB_PATH)

FA4_OK, FA4_ERR_NULL, FA4_ERR_SHAPE, FA4_ERR_UNSUPPORTED, FA4_ERR_ALIGN, FA4_ERR_WORKSPACE, FA4_ERR_HIP = range(7)
FA4_F32, FA4_BF16 = 0, 1
FA4_MXFP4, FA4_NVFP4, FA4_FP8_TOKEN, FA4_MXFP8, FA4_MXFP4_KEYS = 0, 1, 2, 3, 4
FA4_HADAMARD128, FA4_DUAL_RESIDUAL, FA4_SCALE_SEARCH = 1, 2, 4
FA4_P_FP8, FA4_P_NVFP4, FA4_P_MXFP4 = 0, 1, 2         # probability formats (decode: FP8, NVFP4; prefill: FP8, MXFP4)

EXPORTS = ["fa4_quantize_blockscaled", "fa4_quantize_prefill", "fa4_smoothing_factors", "fa4_select_tiles", "fa4_attn_fwd", "fa4_decode_workspace_bytes",
           "fa4_decode_paged", "fa4_decode_paged_noalloc", "fa4_status_string", "fa4_last_error"]
DECODE_SCRATCH_BYTES = 40 << 20                    # FA4_DECODE_SCRATCH_BYTES

_p = ctypes.c_void_p
_i32, _i64, _u32, _f32 = ctypes.c_int32, ctypes.c_int64, ctypes.c_uint32, ctypes.c_float


class QInput(ctypes.Structure):
    _fields_ = [("x", _p), ("dtype", _i32), ("d", _i32), ("outer", _i64), ("heads", _i32), ("rows", _i64),
                ("stride_outer", _i64), ("stride_head", _i64), ("stride_row", _i64),
                ("row_counts", _p), ("page_table", _p), ("page_size", _i32), ("max_pages", _i32),
                ("num_pages", _i64), ("channel_scale", _p)]


class QOutput(ctypes.Structure):
    _fields_ = [("fmt", _i32), ("codes", _p), ("block_scales", _p), ("scales", _p), ("fold_w", _p),
                ("fold_scale", _p)]


class AttnArgs(ctypes.Structure):
    _fields_ = [("fmt", _i32), ("q_codes", _p), ("q_scales", _p), ("q_tscale", _p),
                ("k_codes", _p), ("k_scales", _p), ("k_tscale", _p), ("v_codes", _p), ("v_scales", _p),
                ("v_fold_w", _p), ("v_fold_scale", _p), ("q_bf16", _p), ("k_bf16", _p), ("v_bf16", _p), ("bitmap", _p),
                ("B", _i32), ("Hq", _i32), ("Hkv", _i32), ("Lq", _i32), ("Lk", _i32), ("d", _i32),
                ("causal", _i32), ("softmax_scale", _f32), ("o", _p), ("lse", _p), ("v_fmt", _i32),
                ("v_block_scales", _p), ("p_fmt", _i32)]


class DecodeArgs(ctypes.Structure):
    _fields_ = [("fmt", _i32), ("q1_codes", _p), ("q1_scales", _p), ("q1_tscale", _p),
                ("q2_codes", _p), ("q2_scales", _p), ("q2_tscale", _p),
                ("k_codes", _p), ("k_scales", _p), ("v_codes", _p), ("v_scales", _p),
                ("k_tscale", _p), ("v_tscale", _p), ("page_table", _p), ("ctx_len", _p),
                ("B", _i32), ("Hq", _i32), ("Hkv", _i32), ("d", _i32), ("page_size", _i32), ("max_pages", _i32),
                ("num_pages", _i64), ("softmax_scale", _f32), ("o", _p), ("p_fmt", _i32), ("d_v", _i32)]


lib.fa4_quantize_blockscaled.argtypes = [ctypes.POINTER(QInput), _u32, ctypes.POINTER(QOutput),
                                         ctypes.POINTER(QOutput), _p, _p]
lib.fa4_quantize_blockscaled.restype = ctypes.c_int
lib.fa4_quantize_prefill.argtypes = [ctypes.POINTER(QInput)] * 3 + [ctypes.POINTER(QOutput)] * 3 + [_p, _p, _p]
lib.fa4_quantize_prefill.restype = ctypes.c_int
lib.fa4_smoothing_factors.argtypes = [ctypes.POINTER(QInput), ctypes.POINTER(QInput), _p, _p, _p]
lib.fa4_smoothing_factors.restype = ctypes.c_int
lib.fa4_select_tiles.argtypes = [_p, _p, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _p, _p, _p]
lib.fa4_select_tiles.restype = ctypes.c_int
lib.fa4_attn_fwd.argtypes = [ctypes.POINTER(AttnArgs), _p]
lib.fa4_attn_fwd.restype = ctypes.c_int
lib.fa4_decode_workspace_bytes.argtypes = [ctypes.POINTER(DecodeArgs)]
lib.fa4_decode_workspace_bytes.restype = ctypes.c_size_t
lib.fa4_decode_paged.argtypes = [ctypes.POINTER(DecodeArgs), _p, ctypes.c_size_t, _p]
lib.fa4_decode_paged.restype = ctypes.c_int
lib.fa4_decode_paged_noalloc.argtypes = [ctypes.POINTER(DecodeArgs), _p]
lib.fa4_decode_paged_noalloc.restype = ctypes.c_int
lib.fa4_status_string.argtypes = [ctypes.c_int]
lib.fa4_status_string.restype = ctypes.c_char_p
lib.fa4_last_error.argtypes = []
lib.fa4_last_error.restype = ctypes.c_char_p


class Fa4Error(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        detail = lib.fa4_last_error().decode()
        super().__init__(f"{where}: {lib.fa4_status_string(status).decode()} ({status}): {detail}")


def _check(status, where):
    if status != FA4_OK:
        raise Fa4Error(status, where)


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream():
    return torch.cuda.current_stream().cuda_stream


def _dtype_code(t):
    if t.dtype == torch.float32:
        return FA4_F32
    if t.dtype == torch.bfloat16:
        return FA4_BF16
    raise TypeError(f"unsupported input dtype {t.dtype}")


# ---------------------------------------------------------------------------------------------------- quantize

def _quant_buffers(x, fmt, dual=False, row_norms=False, fold=None, channel_scale=None):
    """Output tensors and the (input, output, residual) ABI descriptors of one quantization."""
    assert x.is_cuda and x.is_contiguous() and x.dim() == 4
    O, H, R, d = x.shape
    dev = x.device
    u8 = dict(dtype=torch.uint8, device=dev)
    out = {}
    if fmt == FA4_FP8_TOKEN:
        out["codes"] = torch.empty(O, H, R, d, **u8)
        out["scales"] = torch.empty(O, H, R, dtype=torch.float32, device=dev)
        bs = None
    elif fmt == FA4_MXFP4_KEYS:          # 4-bit V: blocks of 32 along the rows, codes per column
        out["codes"] = torch.empty(O, H, d, R // 2, **u8)
        out["block_scales"] = bs = torch.empty(O, H, d, R // 32, **u8)
        out["scales"] = None
    elif fmt == FA4_MXFP8:
        out["codes"] = torch.empty(O, H, R, d, **u8)
        out["block_scales"] = bs = torch.empty(O, H, R, d // 32, **u8)
        out["scales"] = None
    else:
        out["codes"] = torch.empty(O, H, R, d // 2, **u8)
        out["block_scales"] = bs = torch.empty(O, H, R, d // (32 if fmt == FA4_MXFP4 else 16), **u8)
        out["scales"] = torch.empty(O * H, dtype=torch.float32, device=dev) if fmt == FA4_NVFP4 else None
    qin = QInput(x.data_ptr(), _dtype_code(x), d, O, H, R, H * R * d, R * d, d, None, None, 0, 0, 0,
                 _ptr(channel_scale))
    if fold is None:
        fold = fmt == FA4_FP8_TOKEN and R % 128 == 0 and R > 0
    if fold:
        out["fold_w"] = torch.empty(O, H, R, dtype=torch.float32, device=dev)
        out["fold_scale"] = torch.empty(O, H, R // 128, dtype=torch.float32, device=dev)
    qout = QOutput(fmt, out["codes"].data_ptr(), _ptr(bs), _ptr(out["scales"]), _ptr(out.get("fold_w")),
                   _ptr(out.get("fold_scale")))
    res = None
    if dual:
        out["codes2"] = torch.empty_like(out["codes"])
        out["block_scales2"] = torch.empty_like(out["block_scales"])
        out["scales2"] = torch.empty_like(out["scales"]) if out["scales"] is not None else None
        res = QOutput(fmt, out["codes2"].data_ptr(), out["block_scales2"].data_ptr(), _ptr(out["scales2"]),
                      None, None)
    if row_norms:
        out["norm2"] = torch.empty(O, H, R, dtype=torch.float32, device=dev)
    return out, qin, qout, res


def quantize(x, fmt, hadamard=False, dual=False, row_norms=False, fold=None, channel_scale=None, search=False):
    """Quantize a [outer, heads, rows, d] tensor (float32 or bf16, contiguous on the GPU).

    Returns a dict: codes [outer, heads, rows, d/2 or d] uint8, block_scales (MXFP4: d/32, NVFP4: d/16
    per row), scales (NVFP4: [outer*heads] tensor scales; FP8: per-row), and with dual=True the
    residual's 'codes2', 'block_scales2', 'scales2'; with row_norms=True 'norm2' [outer, heads, rows];
    FP8 per-token output also carries the attention fold data 'fold_w' [outer, heads, rows] and
    'fold_scale' [outer, heads, rows/128] (default: when rows is a multiple of 128).
    channel_scale: optional [heads, d] float32 static smoothing factors (see smoothing_factors());
    search: the per-block scale search (MXFP4 / NVFP4).
    """
    out, qin, qout, res = _quant_buffers(x, fmt, dual, row_norms, fold, channel_scale)
    flags = (FA4_HADAMARD128 if hadamard else 0) | (FA4_DUAL_RESIDUAL if dual else 0) | \
        (FA4_SCALE_SEARCH if search else 0)
    _check(lib.fa4_quantize_blockscaled(ctypes.byref(qin), flags, ctypes.byref(qout),
                                        ctypes.byref(res) if res is not None else None,
                                        _ptr(out.get("norm2")), _stream()), "fa4_quantize_blockscaled")
    return out


def quantize_prefill(q, k, v, fmt=FA4_MXFP4, row_norms=False, v_fmt=FA4_FP8_TOKEN):
    """Q and K (MXFP4 or MXFP8, optional row norms) and V (FP8 per token with its fold data, or 4-bit V
    with v_fmt=FA4_MXFP4_KEYS and MXFP4 Q/K) of a prefill in one launch (fa4_quantize_prefill). Returns
    three dicts laid out as quantize() returns them; the values are the same bit for bit."""
    bufs = [_quant_buffers(q, fmt, row_norms=row_norms), _quant_buffers(k, fmt, row_norms=row_norms),
            _quant_buffers(v, v_fmt, fold=True if v_fmt == FA4_FP8_TOKEN else None)]
    (qo, qi, qd, _), (ko, ki, kd, _), (vo, vi, vd, _) = bufs
    _check(lib.fa4_quantize_prefill(ctypes.byref(qi), ctypes.byref(ki), ctypes.byref(vi), ctypes.byref(qd),
                                    ctypes.byref(kd), ctypes.byref(vd), _ptr(qo.get("norm2")), _ptr(ko.get("norm2")),
                                    _stream()), "fa4_quantize_prefill")
    return qo, ko, vo


def quantize_paged(x, fmt, ctx_len, page_table, num_pages, page_size=64, channel_scale=None, search=False):
    """Quantize a padded [B, Hkv, Lmax, d] cache tensor (rows r < ctx_len[b] exist) into pages.

    fmt FA4_NVFP4 or FA4_MXFP4. Returns a dict with 'fmt', codes [num_pages, Hkv, page_size, d/2],
    block_scales [num_pages, Hkv, page_size, d/16 (NVFP4) or d/32 (MXFP4)] and scales [B*Hkv] (NVFP4
    tensor scale per (sequence, key head); None for MXFP4).
    """
    assert fmt in (FA4_NVFP4, FA4_MXFP4) and x.is_cuda and x.is_contiguous()
    B, H, R, d = x.shape
    dev = x.device
    nv = fmt == FA4_NVFP4
    out = {
        "fmt": fmt,
        "codes": torch.zeros(num_pages, H, page_size, d // 2, dtype=torch.uint8, device=dev),
        "block_scales": torch.zeros(num_pages, H, page_size, d // (16 if nv else 32), dtype=torch.uint8,
                                    device=dev),
        "scales": torch.empty(B * H, dtype=torch.float32, device=dev) if nv else None,
    }
    qin = QInput(x.data_ptr(), _dtype_code(x), d, B, H, R, H * R * d, R * d, d, ctx_len.data_ptr(),
                 page_table.data_ptr(), page_size, page_table.shape[1], num_pages, _ptr(channel_scale))
    qout = QOutput(fmt, out["codes"].data_ptr(), out["block_scales"].data_ptr(), _ptr(out["scales"]), None, None)
    _check(lib.fa4_quantize_blockscaled(ctypes.byref(qin), FA4_SCALE_SEARCH if search else 0, ctypes.byref(qout),
                                        None, None, _stream()), "fa4_quantize_blockscaled(paged)")
    return out


def smoothing_factors(q_calib, k_calib):
    """Static smoothing factors from calibration tensors q [B, Hq, L, d] and k [B, Hkv, L', d] (contiguous,
    float32 or bf16): returns (q_scale [Hq, d], k_scale [Hkv, d]) float32 powers of two, to be passed as
    channel_scale when quantizing Q and K (QK^T unchanged)."""
    assert q_calib.is_contiguous() and k_calib.is_contiguous()
    dev = q_calib.device
    qs = torch.empty(q_calib.shape[1], q_calib.shape[3], dtype=torch.float32, device=dev)
    ks = torch.empty(k_calib.shape[1], k_calib.shape[3], dtype=torch.float32, device=dev)

    def qin(x):
        O, H, R, d = x.shape
        return QInput(x.data_ptr(), _dtype_code(x), d, O, H, R, H * R * d, R * d, d, None, None, 0, 0, 0, None)

    qi, ki = qin(q_calib), qin(k_calib)
    _check(lib.fa4_smoothing_factors(ctypes.byref(qi), ctypes.byref(ki), qs.data_ptr(), ks.data_ptr(), _stream()),
           "fa4_smoothing_factors")
    return qs, ks


# ---------------------------------------------------------------------------------------------------- select

def select_tiles(q_norm2, k_norm2, causal, num=5, den=100):
    """q_norm2 [B, Hq, Lq], k_norm2 [B, Hkv, Lk] -> (bitmap [B, Hq, Lq/128, Lk/128] uint8, counts [B, Hq])."""
    B, Hq, Lq = q_norm2.shape
    Hkv, Lk = k_norm2.shape[1], k_norm2.shape[2]
    bitmap = torch.empty(B, Hq, Lq // 128, Lk // 128, dtype=torch.uint8, device=q_norm2.device)
    counts = torch.empty(B, Hq, dtype=torch.int32, device=q_norm2.device)
    _check(lib.fa4_select_tiles(q_norm2.data_ptr(), k_norm2.data_ptr(), B, Hq, Hkv, Lq, Lk, int(causal),
                                num, den, bitmap.data_ptr(), counts.data_ptr(), _stream()), "fa4_select_tiles")
    return bitmap, counts


# ---------------------------------------------------------------------------------------------------- attention

def attn_fwd(q, k, v, causal, fmt, Hq, Hkv, Lq, Lk, d, B=1, bitmap=None, q_bf16=None, k_bf16=None,
             v_bf16=None, softmax_scale=None, want_lse=True, out=None, lse=None, v_fmt=FA4_FP8_TOKEN,
             p_fmt=FA4_P_FP8):
    """Prefill attention from quantized operands (dicts as returned by quantize()).

    q/k hold MXFP4, NVFP4 or MXFP8 codes and scales; v holds FP8 per-token codes and scales
    (v_fmt FA4_FP8_TOKEN) or 4-bit V (v_fmt FA4_MXFP4_KEYS, MXFP4 Q/K only; selected tiles read v_bf16).
    p_fmt: probabilities of the quantized tiles, FA4_P_FP8 or FA4_P_MXFP4 (MXFP4 Q/K, d = 128; FP8 or 4-bit V).
    Returns (o [B, Hq, Lq, d] float32, lse [B, Hq, Lq] float32 or None).
    """
    v4 = v_fmt == FA4_MXFP4_KEYS
    dev = q["codes"].device
    if out is None:
        out = torch.empty(B, Hq, Lq, d, dtype=torch.float32, device=dev)
    if want_lse and lse is None:
        lse = torch.empty(B, Hq, Lq, dtype=torch.float32, device=dev)
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(d)
    a = AttnArgs(fmt, q["codes"].data_ptr(), q["block_scales"].data_ptr(), _ptr(q.get("scales")),
                 k["codes"].data_ptr(), k["block_scales"].data_ptr(), _ptr(k.get("scales")),
                 v["codes"].data_ptr(), _ptr(v.get("scales")), _ptr(v.get("fold_w")), _ptr(v.get("fold_scale")),
                 _ptr(q_bf16), _ptr(k_bf16), _ptr(v_bf16), _ptr(bitmap),
                 B, Hq, Hkv, Lq, Lk, d, int(causal), softmax_scale, out.data_ptr(), _ptr(lse if want_lse else None),
                 v_fmt if v4 else 0, _ptr(v.get("block_scales")) if v4 else None, p_fmt)
    _check(lib.fa4_attn_fwd(ctypes.byref(a), _stream()), "fa4_attn_fwd")
    return out, (lse if want_lse else None)


# ---------------------------------------------------------------------------------------------------- decode

def decode_args(q1, q2, kcache, vcache, page_table, ctx_len, Hq, Hkv, d=128, page_size=64, softmax_scale=None,
                out=None, fmt=FA4_NVFP4, p_fmt=FA4_P_FP8):
    B = ctx_len.shape[0]
    if out is None:
        out = torch.empty(B, Hq, d, dtype=torch.float32, device=ctx_len.device)
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(d)
    a = DecodeArgs(fmt, q1["codes"].data_ptr(), q1["block_scales"].data_ptr(), _ptr(q1.get("scales")),
                   q2["codes"].data_ptr(), q2["block_scales"].data_ptr(), _ptr(q2.get("scales")),
                   kcache["codes"].data_ptr(), kcache["block_scales"].data_ptr(),
                   vcache["codes"].data_ptr(), vcache["block_scales"].data_ptr(),
                   _ptr(kcache.get("scales")), _ptr(vcache.get("scales")),
                   page_table.data_ptr(), ctx_len.data_ptr(), B, Hq, Hkv, d, page_size, page_table.shape[1],
                   kcache["codes"].shape[0], softmax_scale, out.data_ptr(), p_fmt, 0)
    return a, out


def decode_workspace(a, device):
    n = lib.fa4_decode_workspace_bytes(ctypes.byref(a))
    return torch.empty(max(n, 256), dtype=torch.uint8, device=device)


def decode_paged(q1, q2, kcache, vcache, page_table, ctx_len, Hq, Hkv, d=128, page_size=64, softmax_scale=None,
                 workspace=None, out=None, fmt=FA4_NVFP4, p_fmt=FA4_P_FP8):
    """Decode attention for one query token per sequence. q1/q2: dicts of the dual-residual query
    ([B, Hq, 1, d] rows); kcache / vcache: paged dicts from quantize_paged(); all in format fmt.
    p_fmt: probability format, FA4_P_FP8 (0) or FA4_P_NVFP4."""
    a, out = decode_args(q1, q2, kcache, vcache, page_table, ctx_len, Hq, Hkv, d, page_size, softmax_scale, out,
                         fmt, p_fmt)
    if workspace is None:
        workspace = decode_workspace(a, ctx_len.device)
    _check(lib.fa4_decode_paged(ctypes.byref(a), workspace.data_ptr(), workspace.numel(), _stream()),
           "fa4_decode_paged")
    return out


def decode_paged_noalloc(args, stream=None):
    """fa4_decode_paged_noalloc on a DecodeArgs struct (from decode_args or mla_decode_args): the decode
    attention with the library's own scratch, no workspace allocated."""
    _check(lib.fa4_decode_paged_noalloc(ctypes.byref(args), _stream() if stream is None else stream),
           "fa4_decode_paged_noalloc")


# ---------------------------------------------------------------------------------------------------- MLA decode

MLA_D, MLA_DV, MLA_H = 576, 512, 16


def quantize_paged_mla(x, ctx_len, page_table, num_pages, page_size=64):
    """MXFP4 latent cache from a padded [B, Lmax, 576] tensor (rows r < ctx_len[b] exist): column-sliced
    pages, codes [num_pages, 9, page_size, 32] and E8M0 scales [num_pages, 9, page_size, 2] (the rows
    quantized as nine 64-wide heads)."""
    assert x.is_cuda and x.is_contiguous() and x.shape[-1] == MLA_D
    B, R, d = x.shape
    ns = d // 64
    dev = x.device
    out = {"fmt": FA4_MXFP4,
           "codes": torch.zeros(num_pages, ns, page_size, 32, dtype=torch.uint8, device=dev),
           "block_scales": torch.zeros(num_pages, ns, page_size, 2, dtype=torch.uint8, device=dev)}
    qin = QInput(x.data_ptr(), _dtype_code(x), 64, B, ns, R, R * d, 64, d, ctx_len.data_ptr(), page_table.data_ptr(),
                 page_size, page_table.shape[1], num_pages, None)
    qout = QOutput(FA4_MXFP4, out["codes"].data_ptr(), out["block_scales"].data_ptr(), None, None, None)
    _check(lib.fa4_quantize_blockscaled(ctypes.byref(qin), 0, ctypes.byref(qout), None, None, _stream()),
           "fa4_quantize_blockscaled(paged MLA)")
    return out


def mla_decode_args(q1, q2, cache, page_table, ctx_len, softmax_scale, out=None):
    B = ctx_len.shape[0]
    if out is None:
        out = torch.empty(B, MLA_H, MLA_DV, dtype=torch.float32, device=ctx_len.device)
    a = DecodeArgs(FA4_MXFP4, q1["codes"].data_ptr(), q1["block_scales"].data_ptr(), None,
                   q2["codes"].data_ptr(), q2["block_scales"].data_ptr(), None,
                   cache["codes"].data_ptr(), cache["block_scales"].data_ptr(), None, None, None, None,
                   page_table.data_ptr(), ctx_len.data_ptr(), B, MLA_H, 1, MLA_D, cache["codes"].shape[2],
                   page_table.shape[1], cache["codes"].shape[0], softmax_scale, out.data_ptr(), FA4_P_FP8, MLA_DV)
    return a, out


def decode_mla(q, cache, page_table, ctx_len, softmax_scale, workspace=None, out=None):
    """One decode step in the MLA geometry: q [B, 16, 576] absorbed queries (bf16 or float32) -> MXFP4
    dual residual -> attention over the shared latent rows (key: all 576 values, value: the first 512).
    Returns (o [B, 16, 512] float32, the quantized query)."""
    B, H, d = q.shape
    assert H == MLA_H and d == MLA_D
    qq = quantize(q.reshape(1, 1, B * H * (d // 64), 64), FA4_MXFP4, dual=True)
    q1 = {"codes": qq["codes"], "block_scales": qq["block_scales"]}
    q2 = {"codes": qq["codes2"], "block_scales": qq["block_scales2"]}
    a, out = mla_decode_args(q1, q2, cache, page_table, ctx_len, softmax_scale, out)
    if workspace is None:
        workspace = decode_workspace(a, ctx_len.device)
    _check(lib.fa4_decode_paged(ctypes.byref(a), workspace.data_ptr(), workspace.numel(), _stream()),
           "fa4_decode_paged(MLA)")
    return out, qq


class DecodeMlaRunner:
    """Preallocated MLA decode step: MXFP4 dual-residual query quantization plus paged attention."""

    def __init__(self, q, cache, page_table, ctx_len, softmax_scale):
        B, H, d = q.shape
        assert H == MLA_H and d == MLA_D and q.is_contiguous()
        dev = q.device
        rows = B * H * (d // 64)
        u8 = dict(dtype=torch.uint8, device=dev)
        self.q = q
        self.q1 = {"codes": torch.empty(B, H, d // 2, **u8), "block_scales": torch.empty(B, H, d // 32, **u8)}
        self.q2 = {k: torch.empty_like(t) for k, t in self.q1.items()}
        self._qi = QInput(q.data_ptr(), _dtype_code(q), 64, 1, 1, rows, rows * 64, rows * 64, 64, None, None, 0, 0, 0,
                          None)
        self._qo = QOutput(FA4_MXFP4, self.q1["codes"].data_ptr(), self.q1["block_scales"].data_ptr(), None, None, None)
        self._qr = QOutput(FA4_MXFP4, self.q2["codes"].data_ptr(), self.q2["block_scales"].data_ptr(), None, None, None)
        self.args, self.o = mla_decode_args(self.q1, self.q2, cache, page_table, ctx_len, softmax_scale)
        self.ws = decode_workspace(self.args, dev)
        self._keep = (cache, page_table, ctx_len)

    def quantize(self, stream=None):
        _check(lib.fa4_quantize_blockscaled(ctypes.byref(self._qi), FA4_DUAL_RESIDUAL, ctypes.byref(self._qo),
                                            ctypes.byref(self._qr), None, _stream() if stream is None else stream),
               "fa4_quantize_blockscaled")

    def attention(self, stream=None):
        _check(lib.fa4_decode_paged(ctypes.byref(self.args), self.ws.data_ptr(), self.ws.numel(),
                                    _stream() if stream is None else stream), "fa4_decode_paged(MLA)")

    def run(self):
        self.quantize()
        self.attention()
        return self.o


# ---------------------------------------------------------------------------------------------------- pipelines

def prefill(q, k, v, causal, fmt=FA4_MXFP4, hadamard=False, select=None, softmax_scale=None, want_lse=True,
            smooth=None, search=False, v_fmt=FA4_FP8_TOKEN, p_fmt=FA4_P_FP8):
    """Whole prefill path: quantize Q/K (MXFP4 or NVFP4, optional Hadamard), V to FP8 per token,
    optionally select the top num/den tiles for bf16 (select=(num, den)), then fused attention with the
    probabilities in p_fmt (FA4_P_FP8 or FA4_P_MXFP4).

    q [B, Hq, Lq, d], k / v [B, Hkv, Lk, d]: contiguous float32 or bf16 CUDA tensors (bf16 needed for
    selection, whose tiles read the originals). Returns a dict with 'o', 'lse', 'bitmap', 'counts',
    and the quantized operands 'q', 'k', 'v'.
    """
    B, Hq, Lq, d = q.shape
    Hkv, Lk = k.shape[1], k.shape[2]
    sel = select is not None
    qs, ks = smooth if smooth is not None else (None, None)
    if fmt in (FA4_MXFP4, FA4_MXFP8) and not hadamard and smooth is None and not search and \
            (v_fmt == FA4_FP8_TOKEN or (fmt == FA4_MXFP4 and d == 128)):
        qq, kq, vq = quantize_prefill(q, k, v, fmt, row_norms=sel, v_fmt=v_fmt)     # one launch for all three
    else:
        qq = quantize(q, fmt, hadamard=hadamard, row_norms=sel, channel_scale=qs)
        kq = quantize(k, fmt, hadamard=hadamard, row_norms=sel, channel_scale=ks, search=search)
        vq = quantize(v, v_fmt)
    bitmap = counts = None
    if sel:
        bitmap, counts = select_tiles(qq["norm2"], kq["norm2"], causal, select[0], select[1])
    o, lse = attn_fwd(qq, kq, vq, causal, fmt, Hq, Hkv, Lq, Lk, d, B=B, bitmap=bitmap,
                      q_bf16=q if sel else None, k_bf16=k if sel else None, v_bf16=v if sel else None,
                      softmax_scale=softmax_scale, want_lse=want_lse, v_fmt=v_fmt, p_fmt=p_fmt)
    return {"o": o, "lse": lse, "bitmap": bitmap, "counts": counts, "q": qq, "k": kq, "v": vq}


def decode(q, kcache, vcache, page_table, ctx_len, Hkv, softmax_scale=None, workspace=None, out=None, p_fmt=FA4_P_FP8):
    """One decode step: q [B, Hq, d] (bf16 or float32) -> dual-residual query in the cache's format (NVFP4
    or MXFP4, from kcache['fmt']) -> paged attention with probabilities in p_fmt (FA4_P_FP8 or
    FA4_P_NVFP4). Returns (o [B, Hq, d] float32, the quantized query)."""
    B, Hq, d = q.shape
    fmt = kcache.get("fmt", FA4_NVFP4)
    # NVFP4 needs a tensor scale per (sequence, head): one group per row; MXFP4 rows are independent,
    # so they go as one group of B*Hq rows (same output layout, far fewer workgroups)
    shape = (B, Hq, 1, d) if fmt == FA4_NVFP4 else (1, 1, B * Hq, d)
    qq = quantize(q.reshape(shape), fmt, dual=True)
    q1 = {"codes": qq["codes"], "block_scales": qq["block_scales"], "scales": qq["scales"]}
    q2 = {"codes": qq["codes2"], "block_scales": qq["block_scales2"], "scales": qq["scales2"]}
    o = decode_paged(q1, q2, kcache, vcache, page_table, ctx_len, Hq, Hkv, d, softmax_scale=softmax_scale,
                     workspace=workspace, out=out, fmt=fmt, p_fmt=p_fmt)
    return o, qq


# ---------------------------------------------------------------------------------------------------- runners

class QuantizeRunner:
    """Preallocated quantization of one [outer, heads, rows, d] tensor (MXFP4 or NVFP4), optionally with a
    Hadamard rotation, static smoothing factors (channel_scale [heads, d]) and the scale search."""

    def __init__(self, x, fmt, hadamard=False, channel_scale=None, search=False):
        O, H, R, d = x.shape
        dev = x.device
        u8, f32 = dict(dtype=torch.uint8, device=dev), dict(dtype=torch.float32, device=dev)
        self.x, self.channel_scale = x, channel_scale
        self.out = {"codes": torch.empty(O, H, R, d // 2, **u8),
                    "block_scales": torch.empty(O, H, R, d // (32 if fmt == FA4_MXFP4 else 16), **u8),
                    "scales": torch.empty(O * H, **f32) if fmt == FA4_NVFP4 else None}
        self._qi = QInput(x.data_ptr(), _dtype_code(x), d, O, H, R, H * R * d, R * d, d, None, None, 0, 0, 0,
                          _ptr(channel_scale))
        self._qo = QOutput(fmt, self.out["codes"].data_ptr(), self.out["block_scales"].data_ptr(),
                           _ptr(self.out["scales"]), None, None)
        self._fl = (FA4_HADAMARD128 if hadamard else 0) | (FA4_SCALE_SEARCH if search else 0)

    def run(self, stream=None):
        _check(lib.fa4_quantize_blockscaled(ctypes.byref(self._qi), self._fl, ctypes.byref(self._qo), None, None,
                                            _stream() if stream is None else stream), "fa4_quantize_blockscaled")
        return self.out


class PrefillRunner:
    """Preallocated prefill path for repeated calls on fixed shapes (benchmarks, serving loops).

    Builds every ABI argument struct once; run() enqueues the quantizer, selector and attention calls
    on the current stream with no allocation. Inputs are read from the tensors given here, so refill
    them in place to change the data.
    """

    def __init__(self, q, k, v, causal, fmt=FA4_MXFP4, hadamard=False, select=None, softmax_scale=None,
                 smooth=None, search=False, v_fmt=FA4_FP8_TOKEN, p_fmt=FA4_P_FP8):
        self.q, self.k, self.v = q, k, v
        B, Hq, Lq, d = q.shape
        Hkv, Lk = k.shape[1], k.shape[2]
        dev = q.device
        self.sel = select is not None
        self.causal, self.fmt, self.select = causal, fmt, select
        self.flags = FA4_HADAMARD128 if hadamard else 0
        u8, f32 = dict(dtype=torch.uint8, device=dev), dict(dtype=torch.float32, device=dev)
        nb = d // (16 if fmt == FA4_NVFP4 else 32)
        cw = d if fmt == FA4_MXFP8 else d // 2                   # code bytes per row
        self.qq = {"codes": torch.empty(B, Hq, Lq, cw, **u8), "block_scales": torch.empty(B, Hq, Lq, nb, **u8),
                   "scales": torch.empty(B * Hq, **f32) if fmt == FA4_NVFP4 else None,
                   "norm2": torch.empty(B, Hq, Lq, **f32) if self.sel else None}
        self.kq = {"codes": torch.empty(B, Hkv, Lk, cw, **u8), "block_scales": torch.empty(B, Hkv, Lk, nb, **u8),
                   "scales": torch.empty(B * Hkv, **f32) if fmt == FA4_NVFP4 else None,
                   "norm2": torch.empty(B, Hkv, Lk, **f32) if self.sel else None}
        v4 = v_fmt == FA4_MXFP4_KEYS
        if v4:
            self.vq = {"codes": torch.empty(B, Hkv, d, Lk // 2, **u8), "block_scales": torch.empty(B, Hkv, d, Lk // 32, **u8)}
        else:
            self.vq = {"codes": torch.empty(B, Hkv, Lk, d, **u8), "scales": torch.empty(B, Hkv, Lk, **f32),
                       "fold_w": torch.empty(B, Hkv, Lk, **f32), "fold_scale": torch.empty(B, Hkv, Lk // 128, **f32)}
        self.o = torch.empty(B, Hq, Lq, d, **f32)
        self.lse = torch.empty(B, Hq, Lq, **f32)
        self.bitmap = torch.empty(B, Hq, Lq // 128, Lk // 128, **u8) if self.sel else None
        self.counts = torch.empty(B, Hq, dtype=torch.int32, device=dev) if self.sel else None

        def qin(x, cs=None):
            O, H, R, dd = x.shape
            return QInput(x.data_ptr(), _dtype_code(x), dd, O, H, R, H * R * dd, R * dd, dd, None, None, 0, 0, 0,
                          _ptr(cs))

        def qout(fm, t):
            return QOutput(fm, t["codes"].data_ptr(), _ptr(t.get("block_scales")), _ptr(t.get("scales")),
                           _ptr(t.get("fold_w")), _ptr(t.get("fold_scale")))

        self.smooth = smooth
        qs, ks = smooth if smooth is not None else (None, None)
        self._qi = [qin(q, qs), qin(k, ks), qin(v)]
        self._qo = [qout(fmt, self.qq), qout(fmt, self.kq), qout(FA4_MXFP4_KEYS if v4 else FA4_FP8_TOKEN, self.vq)]
        self._norms = [_ptr(self.qq["norm2"]), _ptr(self.kq["norm2"]), None]
        self._fl = [self.flags, self.flags | (FA4_SCALE_SEARCH if search else 0), 0]
        # MXFP4 / MXFP8 Q and K with FP8 V and no rotation or search: one launch for all three
        self.fused = fmt in (FA4_MXFP4, FA4_MXFP8) and self.flags == 0 and not search and \
            (not v4 or (fmt == FA4_MXFP4 and d == 128))
        if softmax_scale is None:
            softmax_scale = 1.0 / math.sqrt(d)
        self._attn = AttnArgs(fmt, self.qq["codes"].data_ptr(), self.qq["block_scales"].data_ptr(),
                              _ptr(self.qq["scales"]), self.kq["codes"].data_ptr(),
                              self.kq["block_scales"].data_ptr(), _ptr(self.kq["scales"]),
                              self.vq["codes"].data_ptr(), _ptr(self.vq.get("scales")),
                              _ptr(self.vq.get("fold_w")), _ptr(self.vq.get("fold_scale")),
                              q.data_ptr() if self.sel else None, k.data_ptr() if self.sel else None,
                              v.data_ptr() if self.sel else None, _ptr(self.bitmap),
                              B, Hq, Hkv, Lq, Lk, d, int(causal), softmax_scale, self.o.data_ptr(),
                              self.lse.data_ptr(), FA4_MXFP4_KEYS if v4 else 0,
                              _ptr(self.vq.get("block_scales")) if v4 else None, p_fmt)
        self.shape = (B, Hq, Hkv, Lq, Lk, d)

    def quantize(self, stream=None):
        s = _stream() if stream is None else stream
        if self.fused:
            qi, qo = self._qi, self._qo
            _check(lib.fa4_quantize_prefill(ctypes.byref(qi[0]), ctypes.byref(qi[1]), ctypes.byref(qi[2]),
                                            ctypes.byref(qo[0]), ctypes.byref(qo[1]), ctypes.byref(qo[2]),
                                            self._norms[0], self._norms[1], s), "fa4_quantize_prefill")
        else:
            for i in range(3):
                _check(lib.fa4_quantize_blockscaled(ctypes.byref(self._qi[i]), self._fl[i],
                                                    ctypes.byref(self._qo[i]), None, self._norms[i], s),
                       "fa4_quantize_blockscaled")
        if self.sel:
            B, Hq, Hkv, Lq, Lk, d = self.shape
            _check(lib.fa4_select_tiles(self.qq["norm2"].data_ptr(), self.kq["norm2"].data_ptr(), B, Hq, Hkv, Lq, Lk,
                                        int(self.causal), self.select[0], self.select[1], self.bitmap.data_ptr(),
                                        self.counts.data_ptr(), s), "fa4_select_tiles")

    def attention(self, stream=None):
        _check(lib.fa4_attn_fwd(ctypes.byref(self._attn), _stream() if stream is None else stream), "fa4_attn_fwd")

    def run(self):
        self.quantize()
        self.attention()
        return self.o


class DecodeRunner:
    """Preallocated decode step: dual-residual query quantization (in the cache's format, NVFP4 or MXFP4)
    plus paged attention."""

    def __init__(self, q, kcache, vcache, page_table, ctx_len, Hkv, softmax_scale=None, p_fmt=FA4_P_FP8):
        B, Hq, d = q.shape
        dev = q.device
        self.q = q
        fmt = kcache.get("fmt", FA4_NVFP4)
        nv = fmt == FA4_NVFP4
        u8, f32 = dict(dtype=torch.uint8, device=dev), dict(dtype=torch.float32, device=dev)
        self.q1 = {"codes": torch.empty(B, Hq, 1, d // 2, **u8),
                   "block_scales": torch.empty(B, Hq, 1, d // (16 if nv else 32), **u8),
                   "scales": torch.empty(B * Hq, **f32) if nv else None}
        self.q2 = {k: (torch.empty_like(t) if t is not None else None) for k, t in self.q1.items()}
        if nv:      # one group per (sequence, head): its own tensor scale
            self._qi = QInput(q.data_ptr(), _dtype_code(q), d, B, Hq, 1, Hq * d, d, d, None, None, 0, 0, 0)
        else:       # independent rows: one group of B*Hq rows
            self._qi = QInput(q.data_ptr(), _dtype_code(q), d, 1, 1, B * Hq, B * Hq * d, B * Hq * d, d, None, None,
                              0, 0, 0)
        self._qo = QOutput(fmt, self.q1["codes"].data_ptr(), self.q1["block_scales"].data_ptr(),
                           _ptr(self.q1["scales"]), None, None)
        self._qr = QOutput(fmt, self.q2["codes"].data_ptr(), self.q2["block_scales"].data_ptr(),
                           _ptr(self.q2["scales"]), None, None)
        self.args, self.o = decode_args(self.q1, self.q2, kcache, vcache, page_table, ctx_len, Hq, Hkv, d,
                                        softmax_scale=softmax_scale, fmt=fmt, p_fmt=p_fmt)
        self.ws = decode_workspace(self.args, dev)
        self._keep = (kcache, vcache, page_table, ctx_len)

    def quantize(self, stream=None):
        _check(lib.fa4_quantize_blockscaled(ctypes.byref(self._qi), FA4_DUAL_RESIDUAL, ctypes.byref(self._qo),
                                            ctypes.byref(self._qr), None, _stream() if stream is None else stream),
               "fa4_quantize_blockscaled")

    def attention(self, stream=None):
        _check(lib.fa4_decode_paged(ctypes.byref(self.args), self.ws.data_ptr(), self.ws.numel(),
                                    _stream() if stream is None else stream), "fa4_decode_paged")

    def run(self):
        self.quantize()
        self.attention()
        return self.o
