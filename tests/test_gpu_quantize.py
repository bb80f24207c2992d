"""GPU quantizers vs the oracle: codes, block scales, tensor scales, per-token scales and row norms
must match bit for bit."""
import numpy as np
import pytest
import torch

import workloads as W
from oracle import quant as Q

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fa4():
    import fp8_quantized_attention_amd as m
    return m


def _np(t):
    return t.detach().cpu().numpy()


def _special_rows(d=128, rows=64, seed=0):
    """float32 rows mixing zeros, signed zeros, tiny and huge magnitudes and exact E2M1 ties."""
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal((rows, d)) * np.exp2(rng.integers(-30, 30, (rows, 1)))).astype(np.float32)
    x[0] = 0.0
    x[1] = -0.0
    x[2] = 1e-40                                   # subnormal
    x[3, :32] = [6.0, 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, -0.25, -0.75, -1.25, -1.75, -2.5, -3.5, -5.0, 5.5,
                 0.0, -0.0, 3.0, 4.0, 1.5, 0.5, 1.0, 2.0, -6.0, 6.0, 0.1, -0.1, 2.75, 4.5, 5.25, 0.3]
    x[4] = 3.0e38
    x[5, ::2] = 0.0
    x[6] = np.float32(6.0) * np.float32(2.0 ** -126)
    return x


def test_mxfp4_tiny_fp32_d64(fa4):
    q, k, v = W.prefill_inputs(W.C0)
    out = fa4.quantize(q.cuda(), fa4.FA4_MXFP4, row_norms=True)
    codes, scales = Q.mxfp4_quantize(q.numpy())
    assert np.array_equal(_np(out["codes"]), codes)
    assert np.array_equal(_np(out["block_scales"]), scales)
    assert np.array_equal(_np(out["norm2"]), Q.row_norm2(q.numpy()))


def test_mxfp4_bf16_outliers_and_special_values(fa4):
    cfg = W.C1.scaled(Hq=2, Hkv=2, Lq=512, Lk=512)
    _, k, _ = W.prefill_inputs(cfg)
    out = fa4.quantize(k.cuda(), fa4.FA4_MXFP4, row_norms=True)
    kf = k.float().numpy()
    codes, scales = Q.mxfp4_quantize(kf)
    assert np.array_equal(_np(out["codes"]), codes)
    assert np.array_equal(_np(out["block_scales"]), scales)
    assert np.array_equal(_np(out["norm2"]), Q.row_norm2(kf))
    x = _special_rows()[None, None]
    out = fa4.quantize(torch.from_numpy(x).cuda(), fa4.FA4_MXFP4)
    codes, scales = Q.mxfp4_quantize(x)
    assert np.array_equal(_np(out["codes"]), codes)
    assert np.array_equal(_np(out["block_scales"]), scales)


def _fold_exponent(sigma):
    """Smallest e with 448 * 2^e >= sigma, clamped to [-127, 127] (search from the definition)."""
    e = -127
    while 448.0 * 2.0 ** e < sigma and e < 127:
        e += 1
    return e


def test_fp8_per_token(fa4):
    cfg = W.C1.scaled(Hq=2, Hkv=2, Lq=512, Lk=512)
    _, _, v = W.prefill_inputs(cfg)
    out = fa4.quantize(v.cuda(), fa4.FA4_FP8_TOKEN)
    codes, sv = Q.fp8_per_token_quantize(v.float().numpy())
    assert np.array_equal(_np(out["codes"]), codes)
    assert np.array_equal(_np(out["scales"]), sv)
    # fold data: 2^e per tile (the smallest power of two with 448 * 2^e >= the tile max of s_v) and
    # w = s_v * 2^-e, both exact
    tiles = sv.reshape(1, 2, -1, 128).astype(np.float64)
    e = np.vectorize(_fold_exponent)(tiles.max(axis=-1))
    assert np.array_equal(_np(out["fold_scale"]).astype(np.float64), 2.0 ** e)
    assert np.array_equal(_np(out["fold_w"]).astype(np.float64), (tiles * 2.0 ** -e[..., None]).reshape(1, 2, -1))
    x = _special_rows(seed=1)[None, None]
    x[0, 0, 4] = 1e30                                # stays finite through the per-token scale
    out = fa4.quantize(torch.from_numpy(x).cuda(), fa4.FA4_FP8_TOKEN)
    codes, sv = Q.fp8_per_token_quantize(x)
    assert np.array_equal(_np(out["codes"]), codes)
    assert np.array_equal(_np(out["scales"]), sv)


@pytest.mark.parametrize("hadamard", [False, True])
def test_nvfp4_tensor_block_scales_and_hadamard(fa4, hadamard):
    cfg = W.C4.scaled(Hq=8, Hkv=2, Lq=256, Lk=1024)
    q, k, _ = W.prefill_inputs(cfg)
    for x in (q, k):
        out = fa4.quantize(x.cuda(), fa4.FA4_NVFP4, hadamard=hadamard, row_norms=True)
        xf = x.float().numpy().astype(np.float64)
        xr = Q.hadamard_rotate(xf) if hadamard else xf
        B, H, L, d = x.shape
        codes, sb, st = Q.nvfp4_quantize(xr.reshape(B * H, L, d))
        assert np.array_equal(_np(out["scales"]), st)
        assert np.array_equal(_np(out["block_scales"]).reshape(B * H, L, -1), sb)
        assert np.array_equal(_np(out["codes"]).reshape(B * H, L, -1), codes)
        assert np.array_equal(_np(out["norm2"]), Q.row_norm2(xf))


def test_nvfp4_special_values_and_empty(fa4):
    x = _special_rows(seed=2).reshape(2, 32, 128)[None]
    out = fa4.quantize(torch.from_numpy(np.ascontiguousarray(x)).cuda(), fa4.FA4_NVFP4)
    codes, sb, st = Q.nvfp4_quantize(x[0])
    assert np.array_equal(_np(out["scales"]), st)
    assert np.array_equal(_np(out["block_scales"])[0], sb)
    assert np.array_equal(_np(out["codes"])[0], codes)
    empty = torch.zeros(1, 3, 0, 128, device="cuda")
    out = fa4.quantize(empty, fa4.FA4_NVFP4)
    assert np.array_equal(_np(out["scales"]), np.ones(3, np.float32))


@pytest.mark.parametrize("rows", [40, 100])
def test_nvfp4_dual_group_sizes(fa4, rows):
    """Groups of at most 64 rows take the one-launch path, larger ones the multi-pass one: both must
    give the oracle's codes and tensor scales, for Q1 and the residual Q2, on special values."""
    x = np.concatenate([_special_rows(rows=rows, seed=3), _special_rows(rows=rows, seed=4)])
    x = np.ascontiguousarray(x.reshape(1, 2, rows, 128))
    out = fa4.quantize(torch.from_numpy(x).cuda(), fa4.FA4_NVFP4, dual=True)
    (c1, s1, t1), (c2, s2, t2) = Q.dual_residual_quantize(x[0].astype(np.float64))
    assert np.array_equal(_np(out["scales"]), t1) and np.array_equal(_np(out["scales2"]), t2)
    assert np.array_equal(_np(out["block_scales"])[0], s1) and np.array_equal(_np(out["codes"])[0], c1)
    assert np.array_equal(_np(out["block_scales2"])[0], s2) and np.array_equal(_np(out["codes2"])[0], c2)


def test_dual_residual_query(fa4):
    q = W.decode_query(W.C3)                          # [64, 32, 128] bf16
    out = fa4.quantize(q.reshape(64, 32, 1, 128).cuda(), fa4.FA4_NVFP4, dual=True)
    (c1, s1, t1), (c2, s2, t2) = Q.dual_residual_quantize(q.float().numpy().reshape(64 * 32, 1, 128))
    assert np.array_equal(_np(out["scales"]), t1) and np.array_equal(_np(out["scales2"]), t2)
    assert np.array_equal(_np(out["block_scales"]).reshape(2048, 1, -1), s1)
    assert np.array_equal(_np(out["block_scales2"]).reshape(2048, 1, -1), s2)
    assert np.array_equal(_np(out["codes"]).reshape(2048, 1, -1), c1)
    assert np.array_equal(_np(out["codes2"]).reshape(2048, 1, -1), c2)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_mxfp8_codes_and_scales(fa4, d, dtype):
    x = np.ascontiguousarray(_special_rows(d=d, rows=96, seed=7).reshape(1, 2, 48, d))
    t = torch.from_numpy(x)
    if dtype == "bf16":
        t = t.to(torch.bfloat16)
    out = fa4.quantize(t.cuda(), fa4.FA4_MXFP8)
    codes, scales = Q.mxfp8_quantize(t.float().numpy().astype(np.float64))
    assert out["scales"] is None
    assert np.array_equal(_np(out["codes"]), codes) and np.array_equal(_np(out["block_scales"]), scales)


@pytest.mark.parametrize("special", [False, True])
@pytest.mark.parametrize("layout", ["row_groups", "one_group"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_dual_residual_query_mxfp4(fa4, special, layout, dtype):
    """MXFP4 dual residual: Q1 = MXFP4(q), Q2 = MXFP4(fl32(q - dequant(Q1))), bit for bit. Layouts: n
    groups of one row, and one group of n rows (the decode query's layout, chunked by rows per workgroup);
    n = 2048 for the decode query and 67 (not a multiple of the chunk) for the special rows."""
    if special:
        q = torch.from_numpy(np.concatenate([_special_rows(rows=64), _special_rows(rows=8, seed=9)[5:]]))
    else:
        q = W.decode_query(W.C3).float().reshape(64 * 32, 128)
    if dtype == "bf16":
        q = q.to(torch.bfloat16)
    n = q.shape[0]
    shape = (1, n, 1, 128) if layout == "row_groups" else (1, 1, n, 128)
    out = fa4.quantize(q.reshape(shape).contiguous().cuda(), fa4.FA4_MXFP4, dual=True)
    q = q.float().reshape(n, 1, 128)
    (c1, s1), (c2, s2) = Q.dual_residual_quantize_mx(q.numpy().reshape(n, 1, 128))
    assert out["scales"] is None and out["scales2"] is None
    assert np.array_equal(_np(out["block_scales"]).reshape(n, 1, -1), s1)
    assert np.array_equal(_np(out["block_scales2"]).reshape(n, 1, -1), s2)
    assert np.array_equal(_np(out["codes"]).reshape(n, 1, -1), c1)
    assert np.array_equal(_np(out["codes2"]).reshape(n, 1, -1), c2)


@pytest.mark.parametrize("base", [W.C3, W.C3_MX], ids=["nvfp4", "mxfp4"])
def test_paged_kv_cache(fa4, base):
    from oracle_cases import decode_cache
    cfg = base.scaled(B=3, Hq=8, Hkv=2, ctx_lo=200, ctx_hi=700)
    lay = W.decode_layout(cfg)
    (kc, ks), (vc, vs), kt, vt, _ = decode_cache(cfg, lay, 0)
    ctx = lay.ctx_len.cuda()
    pt = lay.page_table.cuda()
    fmt = fa4.FA4_NVFP4 if cfg.kv_fmt == "nvfp4" else fa4.FA4_MXFP4
    for tensor, (rc, rs, rt) in [(W.T_K, (kc, ks, kt)), (W.T_V, (vc, vs, vt))]:
        x = W.decode_kv_padded(cfg, lay, tensor, device="cuda")
        out = fa4.quantize_paged(x, fmt, ctx, pt, lay.num_pages)
        if fmt == fa4.FA4_NVFP4:
            assert np.array_equal(_np(out["scales"]).reshape(cfg.B, cfg.Hkv), rt)
        # compare every row that exists
        for b in range(cfg.B):
            L = int(lay.ctx_len[b])
            c = np.arange(L)
            phys = lay.page_table[b].numpy()[c // 64]
            assert np.array_equal(_np(out["codes"])[phys, :, c % 64], rc[phys, :, c % 64])
            assert np.array_equal(_np(out["block_scales"])[phys, :, c % 64], rs[phys, :, c % 64])



def _keys_layout(codes):
    """The attention's storage order of MXFP4_KEYS codes: within each 32-value block, position j holds
    value 8 ((j >> 2) & 3) + 4 (j >> 4) + (j & 3) (nibbles repacked two per byte, low first)."""
    c = np.stack([codes & 15, codes >> 4], axis=-1).reshape(codes.shape[:-1] + (-1, 32))
    j = np.arange(32)
    perm = 8 * ((j >> 2) & 3) + 4 * (j >> 4) + (j & 3)
    c = c[..., perm].reshape(codes.shape[:-1] + (-1, 2))
    return (c[..., 0] | (c[..., 1] << 4)).astype(np.uint8)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_mxfp4_keys_codes_and_scales(fa4, d, dtype):
    """4-bit V: MXFP4 blocks along the rows of each column, bit for bit, in the attention's key order."""
    x = np.concatenate([_special_rows(d=d, rows=64, seed=8), _special_rows(d=d, rows=64, seed=9),
                        np.random.default_rng(3).standard_normal((128, d)).astype(np.float32)])
    x = np.ascontiguousarray(x.reshape(1, 2, 128, d))
    t = torch.from_numpy(x)
    if dtype == "bf16":
        t = t.to(torch.bfloat16)
    out = fa4.quantize(t.cuda(), fa4.FA4_MXFP4_KEYS)
    codes, scales = Q.mxfp4_keys_quantize(t.float().numpy().astype(np.float64))
    assert out["codes"].shape == (1, 2, d, 64) and out["block_scales"].shape == (1, 2, d, 4)
    assert np.array_equal(_np(out["block_scales"]), scales)
    assert np.array_equal(_np(out["codes"]), _keys_layout(codes))


@pytest.mark.parametrize("fmt", ["mxfp4", "mxfp8"])
@pytest.mark.parametrize("dtype,d", [("f32", 64), ("f32", 128), ("bf16", 128)])
@pytest.mark.parametrize("norms", [False, True])
def test_prefill_quantize_one_launch(fa4, fmt, dtype, d, norms):
    """fa4_quantize_prefill: Q and K (a ragged last 64-row chunk in Q) and V with its fold data, all
    against the oracle bit for bit, and equal to the three separate calls."""
    g = torch.Generator().manual_seed(21)
    dt = torch.float32 if dtype == "f32" else torch.bfloat16
    B, Hq, Hkv, Lq, Lk = 2, 4, 2, 200, 384
    q = (torch.randn(B, Hq, Lq, d, generator=g) * 2).to(dt)
    k = torch.randn(B, Hkv, Lk, d, generator=g)
    k[..., 3] *= 20.0                                   # an outlier channel
    k = k.to(dt)
    v = (torch.randn(B, Hkv, Lk, d, generator=g) * torch.rand(B, Hkv, Lk, 1, generator=g) * 8).to(dt)
    v[0, 1, 130] = 0.0                                  # an all-zero token (scale 1)
    F = fa4.FA4_MXFP4 if fmt == "mxfp4" else fa4.FA4_MXFP8
    qq, kq, vq = fa4.quantize_prefill(q.cuda(), k.cuda(), v.cuda(), F, row_norms=norms)
    torch.cuda.synchronize()
    quant = Q.mxfp4_quantize if fmt == "mxfp4" else Q.mxfp8_quantize
    for x, out in ((q, qq), (k, kq)):
        xf = x.float().numpy().astype(np.float64)
        codes, sc = quant(xf)
        assert np.array_equal(_np(out["codes"]), codes)
        assert np.array_equal(_np(out["block_scales"]), sc)
        if norms:
            assert np.array_equal(_np(out["norm2"]), Q.row_norm2(xf))
    codes, sv = Q.fp8_per_token_quantize(v.float().numpy())
    assert np.array_equal(_np(vq["codes"]), codes)
    assert np.array_equal(_np(vq["scales"]), sv)
    tiles = sv.reshape(B, Hkv, -1, 128).astype(np.float64)
    e = np.vectorize(_fold_exponent)(tiles.max(axis=-1))
    assert np.array_equal(_np(vq["fold_scale"]).astype(np.float64), 2.0 ** e)
    assert np.array_equal(_np(vq["fold_w"]).astype(np.float64), (tiles * 2.0 ** -e[..., None]).reshape(B, Hkv, -1))
    sep = [fa4.quantize(x.cuda(), F, row_norms=norms) for x in (q, k)] + [fa4.quantize(v.cuda(), fa4.FA4_FP8_TOKEN)]
    for a, b in zip((qq, kq, vq), sep):
        for key, t in b.items():
            if t is not None:
                assert torch.equal(a[key], t), key


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("dual", [False, True])
def test_nvfp4_one_row_groups(fa4, d, dtype, dual):
    """NVFP4 of one-row groups (one row per (outer, head), the decode query's shape), with zero, signed-zero,
    subnormal, huge and tie-laden rows, and a group count that leaves part of the last workgroup idle:
    tensor scales, block scales and codes of Q1 (and Q2) bit for bit."""
    rows = _special_rows(d=d, rows=70, seed=5)
    t = torch.from_numpy(np.ascontiguousarray(rows.reshape(7, 10, 1, d)))
    if dtype == "bf16":
        t = t.to(torch.bfloat16)
    out = fa4.quantize(t.cuda(), fa4.FA4_NVFP4, dual=dual)
    x = t.float().numpy().astype(np.float64).reshape(70, 1, d)
    if dual:
        (c1, s1, t1), (c2, s2, t2) = Q.dual_residual_quantize(x)
        assert np.array_equal(_np(out["scales2"]), t2)
        assert np.array_equal(_np(out["block_scales2"]).reshape(70, 1, -1), s2)
        assert np.array_equal(_np(out["codes2"]).reshape(70, 1, -1), c2)
    else:
        c1, s1, t1 = Q.nvfp4_quantize(x)
    assert np.array_equal(_np(out["scales"]), t1)
    assert np.array_equal(_np(out["block_scales"]).reshape(70, 1, -1), s1)
    assert np.array_equal(_np(out["codes"]).reshape(70, 1, -1), c1)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_prefill_quantize_one_launch_v4(fa4, dtype):
    """fa4_quantize_prefill with 4-bit V: MXFP4 Q and K and V's MXFP4 blocks along the keys (in the
    attention's key order), against the oracle and the separate calls, bit for bit; an odd number of
    32-key units leaves the last workgroup half idle."""
    g = torch.Generator().manual_seed(23)
    dt = torch.float32 if dtype == "f32" else torch.bfloat16
    B, Hq, Hkv, Lq, Lk = 1, 4, 3, 192, 96
    q = torch.randn(B, Hq, Lq, 128, generator=g).to(dt)
    k = torch.randn(B, Hkv, Lk, 128, generator=g).to(dt)
    v = (torch.randn(B, Hkv, Lk, 128, generator=g) * torch.rand(B, Hkv, Lk, 1, generator=g) * 8).to(dt)
    v[0, 2, 40:72] = 0.0                                # an all-zero block of keys
    qq, kq, vq = fa4.quantize_prefill(q.cuda(), k.cuda(), v.cuda(), fa4.FA4_MXFP4, v_fmt=fa4.FA4_MXFP4_KEYS)
    torch.cuda.synchronize()
    for x, out in ((q, qq), (k, kq)):
        codes, sc = Q.mxfp4_quantize(x.float().numpy().astype(np.float64))
        assert np.array_equal(_np(out["codes"]), codes) and np.array_equal(_np(out["block_scales"]), sc)
    codes, scales = Q.mxfp4_keys_quantize(v.float().numpy().astype(np.float64))
    assert np.array_equal(_np(vq["block_scales"]), scales)
    assert np.array_equal(_np(vq["codes"]), _keys_layout(codes))
    sep = [fa4.quantize(x.cuda(), fa4.FA4_MXFP4) for x in (q, k)] + [fa4.quantize(v.cuda(), fa4.FA4_MXFP4_KEYS)]
    for a, b in zip((qq, kq, vq), sep):
        for key, t in b.items():
            if t is not None:
                assert torch.equal(a[key], t), key
