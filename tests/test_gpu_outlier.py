"""GPU outlier-aware key quantization (static smoothing factors, channel scaling, per-block scale
search) vs the oracle: factors, codes and scales bit for bit; attention within the parity bar."""
import numpy as np
import pytest
import torch

import workloads as W
from oracle import formats as F
from oracle import outlier as OA
from oracle import quant as Q
from oracle_cases import assert_parity, prefill_reference

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fa4():
    import fp8_quantized_attention_amd as m
    return m


def _np(t):
    return t.detach().cpu().numpy()


def _special(rows, seed):
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal((rows, 128)) * np.exp2(rng.integers(-20, 20, (rows, 1)))).astype(np.float32)
    x[:, rng.permutation(128)[:4]] *= 20.0
    x[0] = 0.0
    x[1, :32] = np.float32([0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0, -6.0] * 4)
    x[2, :16] = np.float32([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, -0.25] * 2)
    return x


def test_smoothing_factors_match_oracle(fa4):
    cfg = W.C4.scaled(Hq=8, Hkv=2, Lq=256, Lk=384)
    q, k, _ = W.prefill_inputs(cfg)
    q[0, 3, :, 7] = 0                                       # a channel with a zero maximum in one head only
    k[0, 1, :, 9] = 0                                       # and one with a zero key maximum
    qs, ks = fa4.smoothing_factors(q.cuda().contiguous(), k.cuda().contiguous())
    rq, rk = OA.smoothing_factors(q.float().numpy(), k.float().numpy())
    assert np.array_equal(_np(qs), rq) and np.array_equal(_np(ks), rk)
    assert _np(ks)[1, 9] == 1.0


@pytest.mark.parametrize("fmt", ["mxfp4", "nvfp4"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("rows", [40, 200])
def test_scale_search_bit_exact(fa4, fmt, dtype, rows):
    x = np.stack([_special(rows, 5), _special(rows, 6)])[None]            # [1, 2, rows, 128]
    t = torch.from_numpy(np.ascontiguousarray(x))
    if dtype == "bf16":
        t = t.to(torch.bfloat16)
    xf = t.float().numpy()[0].astype(np.float64)
    out = fa4.quantize(t.cuda(), fa4.FA4_MXFP4 if fmt == "mxfp4" else fa4.FA4_NVFP4, search=True)
    if fmt == "mxfp4":
        c, s = OA.mxfp4_quantize_search(xf)
    else:
        c, s, st = OA.nvfp4_quantize_search(xf)
        assert np.array_equal(_np(out["scales"]), st)
    assert np.array_equal(_np(out["block_scales"])[0], s)
    assert np.array_equal(_np(out["codes"])[0], c)


@pytest.mark.parametrize("fmt", ["mxfp4", "nvfp4"])
def test_smoothing_rotation_search_bit_exact(fa4, fmt):
    cfg = W.C4.scaled(Hq=4, Hkv=2, Lq=128, Lk=256)
    q, k, _ = W.prefill_inputs(cfg)
    qs, ks = fa4.smoothing_factors(q.cuda(), k.cuda())
    code = fa4.FA4_MXFP4 if fmt == "mxfp4" else fa4.FA4_NVFP4
    out = fa4.quantize(k.cuda(), code, hadamard=True, channel_scale=ks, search=True, row_norms=True)
    kf = k.float().numpy().astype(np.float64)[0]                          # [2, 256, 128]
    ksn = _np(ks).astype(np.float64)
    xs = Q.hadamard_rotate(F.fp32(kf * ksn[:, None, :]).astype(np.float64))
    if fmt == "mxfp4":
        c, s = OA.mxfp4_quantize_search(xs)
    else:
        c, s, st = OA.nvfp4_quantize_search(xs)
        assert np.array_equal(_np(out["scales"]), st)
    assert np.array_equal(_np(out["block_scales"])[0], s) and np.array_equal(_np(out["codes"])[0], c)
    assert np.array_equal(_np(out["norm2"])[0], Q.row_norm2(kf))            # norms of the unscaled rows


def test_paged_cache_search_bit_exact(fa4):
    cfg = W.C3.scaled(B=3, Hq=8, Hkv=2, ctx_lo=200, ctx_hi=700)
    lay = W.decode_layout(cfg)
    x = W.decode_kv_padded(cfg, lay, W.T_K, device="cuda")
    out = fa4.quantize_paged(x, fa4.FA4_NVFP4, lay.ctx_len.cuda(), lay.page_table.cuda(), lay.num_pages, search=True)
    for b in range(cfg.B):
        L = int(lay.ctx_len[b])
        c = np.arange(L)
        phys = lay.page_table[b].numpy()[c // 64]
        for h in range(cfg.Hkv):
            xr = W.decode_kv_head(cfg, W.T_K, b, h, L).float().numpy().astype(np.float64)
            rc, rs, rt = OA.nvfp4_quantize_search(xr[None])
            assert _np(out["scales"])[b * cfg.Hkv + h] == rt[0]
            assert np.array_equal(_np(out["codes"])[phys, h, c % 64], rc[0])
            assert np.array_equal(_np(out["block_scales"])[phys, h, c % 64], rs[0])


@pytest.mark.parametrize("base", ["c1", "c4"])
def test_prefill_with_smoothing_and_search(fa4, base):
    """End to end: static smoothing of Q and K plus K's scale search, through the fused attention."""
    cfg = (W.C1.scaled(Hq=2, Hkv=2, Lq=512, Lk=512) if base == "c1"
           else W.C4.scaled(Hq=4, Hkv=1, Lq=256, Lk=768))
    q, k, v = W.prefill_inputs(cfg)
    qc, kc, vc = q.cuda(), k.cuda(), v.cuda()
    qs, ks = fa4.smoothing_factors(qc, kc)
    fmt = fa4.FA4_MXFP4 if cfg.qk_fmt == "mxfp4" else fa4.FA4_NVFP4
    sel = (5, 100) if cfg.select else None
    res = fa4.prefill(qc, kc, vc, cfg.causal, fmt=fmt, hadamard=cfg.hadamard, select=sel, smooth=(qs, ks),
                      search=True)
    torch.cuda.synchronize()
    heads = [(0, h) for h in range(cfg.Hq)]
    rows = np.arange(cfg.Lq)
    ref, lse, _, slack = prefill_reference(cfg, 0, heads, rows, select=sel, q_all=q, k_all=k, v_all=v,
                                           smooth=(_np(qs), _np(ks)), search=True, slack=True)
    assert_parity(_np(res["o"])[0], ref, f"prefill {base} smoothing + search", slack)


@pytest.mark.parametrize("rows", [6, 100])
@pytest.mark.parametrize("search", [False, True])
def test_nvfp4_subnormal_tensor_maximum(fa4, rows, search):
    """Groups whose maximum is subnormal (1e-42: fl32(amax / 2688) underflows, so s_t = 1 and the group
    quantizes as all zeros; 1e-39 and 3e-40: a subnormal tensor scale) and one normal group, plain and
    with the scale search, on the one-launch (<= 64 rows) and multi-pass paths: bit for bit."""
    rng = np.random.default_rng(11)
    g = []
    for amax in (1e-42, 1e-39, 3e-40, 1e-30):
        x = rng.standard_normal((rows, 128))
        g.append((x / np.abs(x).max() * amax).astype(np.float32))
    x = np.stack(g)[None]                                             # [1, 4, rows, 128]
    out = fa4.quantize(torch.from_numpy(np.ascontiguousarray(x)).cuda(), fa4.FA4_NVFP4, search=search)
    xf = x[0].astype(np.float64)
    c, s, st = OA.nvfp4_quantize_search(xf) if search else Q.nvfp4_quantize(xf)
    assert st[0] == 1.0
    assert np.array_equal(_np(out["scales"]), st)
    assert np.array_equal(_np(out["block_scales"])[0], s)
    assert np.array_equal(_np(out["codes"])[0], c)
