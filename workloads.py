"""Seeded synthetic inputs for block-scaled low-bit attention (no method arithmetic here).

Both the CPU oracle's tests and the GPU path draw their inputs from this
module and from nothing else they share. It only draws random numbers and
lays them out; it never quantizes, rotates or attends.

Recipe (the same for every workload):
  * every (tensor, batch, head) chunk has its own torch CPU generator seeded by
    chunk_seed(seed, workload, tensor, b, h), so any chunk can be regenerated
    alone;
  * values are float32 N(0, 1); the key tensors of the long-context workloads
    carry 4 fixed outlier channels per key head (torch.randperm(d)[:4] of that
    chunk's own generator) multiplied by 20 in float32;
  * bf16 workloads then round to bfloat16 (torch's cast, nearest-even);
  * decode context lengths are uniform integers in [lo, hi]; the physical page
    ids are one random permutation of all pages, handed out in logical order.

The shapes follow the long-context workloads of the pages (32K-token prefill,
128K-token caches, 8K-32K decode contexts with grouped-query heads); the
synthetic tensors stand in for the models and datasets those pages measure on.
"""
from dataclasses import dataclass, replace

import torch

T_Q, T_K, T_V, T_OUTLIER, T_CTX, T_PERM = 0, 1, 2, 3, 4, 5


def chunk_seed(seed, workload, tensor, b, h):
    return ((((int(seed) * 16 + int(workload)) * 8 + int(tensor)) * 1024 + int(b)) * 64 + int(h))


def _gen(seed, workload, tensor, b, h):
    return torch.Generator().manual_seed(chunk_seed(seed, workload, tensor, b, h))


@dataclass(frozen=True)
class Prefill:
    name: str
    workload: int
    B: int
    Hq: int
    Hkv: int
    Lq: int
    Lk: int
    d: int
    causal: bool
    dtype: str              # "f32" or "bf16"
    qk_fmt: str             # "mxfp4" or "nvfp4"
    outliers: bool = False
    hadamard: bool = False
    select: bool = False
    v_fmt: str = "fp8"      # "fp8" (E4M3 per token) or "mxfp4k" (MXFP4, 32-blocks along the keys)
    p_fmt: str = "fp8"      # probabilities of the quantized tiles: "fp8" (E4M3) or "mxfp4" (32-key MX blocks)

    def scaled(self, **kw):
        return replace(self, **kw)


@dataclass(frozen=True)
class Decode:
    name: str
    workload: int
    B: int
    Hq: int
    Hkv: int
    d: int
    page_size: int
    ctx_lo: int
    ctx_hi: int
    kv_fmt: str = "nvfp4"        # format of the paged K/V cache and of the query residuals
    p_fmt: str = "fp8"           # format of the probabilities before PV: "fp8" or "nvfp4"
    d_v: int = 0                 # MLA geometry: value width (the first d_v of each latent row); 0 = GQA
    softmax_scale: float = 0.0   # 0: 1/sqrt(d)

    def scaled(self, **kw):
        return replace(self, **kw)


# The five workloads. C0 is the small case the oracle finishes in seconds.
C0 = Prefill("tiny_prefill_mxfp4", 0, B=1, Hq=2, Hkv=2, Lq=256, Lk=256, d=64, causal=False,
             dtype="f32", qk_fmt="mxfp4")
C1 = Prefill("prefill_4k_causal_mxfp4", 1, B=1, Hq=32, Hkv=32, Lq=4096, Lk=4096, d=128, causal=True,
             dtype="bf16", qk_fmt="mxfp4", outliers=True)
C2 = Prefill("prefill_32k_causal_select5", 2, B=1, Hq=32, Hkv=32, Lq=32768, Lk=32768, d=128, causal=True,
             dtype="bf16", qk_fmt="mxfp4", outliers=True, select=True)
C3 = Decode("decode_paged_nvfp4_gqa", 3, B=64, Hq=32, Hkv=8, d=128, page_size=64, ctx_lo=8192, ctx_hi=32768)
C4 = Prefill("chunked_prefill_128k_nvfp4_hadamard_select5", 4, B=1, Hq=32, Hkv=8, Lq=2048, Lk=131072, d=128,
             causal=True, dtype="bf16", qk_fmt="nvfp4", outliers=True, hadamard=True, select=True)
WORKLOADS = [C0, C1, C2, C3, C4]
# The 4K causal prefill with Q and K in MXFP8 (E4M3 elements, E8M0 scale per 32; "MXFP vs NVFP4"
# section 4.2's policy for the attention inputs): the same values as C1.
C1_MX8 = replace(C1, name="prefill_4k_causal_mxfp8", qk_fmt="mxfp8")
# The 4K causal prefill with 4-bit V (MXFP4 with 32-element blocks along the keys): same values as C1.
C1_V4 = replace(C1, name="prefill_4k_causal_mxfp4_v4", v_fmt="mxfp4k")
# The 4K causal prefill with the probabilities in MXFP4 (E8M0 scale per 32 keys) against FP8 V: same values.
C1_P4 = replace(C1, name="prefill_4k_causal_mxfp4_p4", p_fmt="mxfp4")
# 4-bit V and MXFP4 probabilities together (both PV operands FP4, block-scaled along the keys): same values.
C1_V4P4 = replace(C1_V4, name="prefill_4k_causal_mxfp4_v4p4", p_fmt="mxfp4")
# The decode workload over an MXFP4 cache (E8M0 scale per 32 elements, no tensor scale): the same
# sequences, lengths, pages and values as C3 (same workload id, hence the same seeds).
C3_MX = replace(C3, name="decode_paged_mxfp4_gqa", kv_fmt="mxfp4")
C3_P4 = replace(C3, name="decode_paged_nvfp4_gqa_p4", p_fmt="nvfp4")
C3_MX_P4 = replace(C3_MX, name="decode_paged_mxfp4_gqa_p4", p_fmt="nvfp4")
# MLA-shaped decode: 16 query heads (one tensor-parallel shard of a 128-head model) over one shared
# latent row per token, 512 latent + 64 rotary values (the key); the value is the latent part. The
# softmax scale is that of the un-absorbed 128 + 64 query-key width. Contexts and pages as C3.
C5_MLA = Decode("decode_paged_mla_mxfp4", 5, B=64, Hq=16, Hkv=1, d=576, page_size=64, ctx_lo=8192,
                ctx_hi=32768, kv_fmt="mxfp4", d_v=512, softmax_scale=192 ** -0.5)


def _chunk(seed, wl, tensor, b, h, rows, d, outliers, dtype):
    g = _gen(seed, wl, tensor, b, h)
    x = torch.randn(rows, d, generator=g, dtype=torch.float32)
    if outliers:
        go = _gen(seed, wl, T_OUTLIER, b, h)
        ch = torch.randperm(d, generator=go)[:4]
        x[:, ch] *= 20.0
    return x.to(torch.bfloat16) if dtype == "bf16" else x


def prefill_head(cfg, tensor, b, h, seed=0):
    """One [L, d] chunk: tensor T_Q (query head h) or T_K / T_V (key head h)."""
    rows = cfg.Lq if tensor == T_Q else cfg.Lk
    outl = cfg.outliers and tensor == T_K
    return _chunk(seed, cfg.workload, tensor, b, h, rows, cfg.d, outl, cfg.dtype)


def prefill_inputs(cfg, seed=0):
    """q [B, Hq, Lq, d], k and v [B, Hkv, Lk, d] on the CPU (float32 or bfloat16)."""
    dt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    q = torch.empty(cfg.B, cfg.Hq, cfg.Lq, cfg.d, dtype=dt)
    k = torch.empty(cfg.B, cfg.Hkv, cfg.Lk, cfg.d, dtype=dt)
    v = torch.empty(cfg.B, cfg.Hkv, cfg.Lk, cfg.d, dtype=dt)
    for b in range(cfg.B):
        for h in range(cfg.Hq):
            q[b, h] = prefill_head(cfg, T_Q, b, h, seed)
        for h in range(cfg.Hkv):
            k[b, h] = prefill_head(cfg, T_K, b, h, seed)
            v[b, h] = prefill_head(cfg, T_V, b, h, seed)
    return q, k, v


@dataclass
class DecodeLayout:
    ctx_len: torch.Tensor        # [B] int32
    page_table: torch.Tensor     # [B, max_pages] int32, -1 past each sequence's pages
    num_pages: int
    max_pages: int


def decode_layout(cfg, seed=0):
    g = _gen(seed, cfg.workload, T_CTX, 0, 0)
    ctx = torch.randint(cfg.ctx_lo, cfg.ctx_hi + 1, (cfg.B,), generator=g, dtype=torch.int64)
    npg = (ctx + cfg.page_size - 1) // cfg.page_size
    total = int(npg.sum())
    max_pages = (cfg.ctx_hi + cfg.page_size - 1) // cfg.page_size
    perm = torch.randperm(total, generator=_gen(seed, cfg.workload, T_PERM, 0, 0))
    pt = torch.full((cfg.B, max_pages), -1, dtype=torch.int32)
    off = 0
    for b in range(cfg.B):
        n = int(npg[b])
        pt[b, :n] = perm[off:off + n].to(torch.int32)
        off += n
    return DecodeLayout(ctx.to(torch.int32), pt, total, max_pages)


def decode_query(cfg, seed=0):
    """q [B, Hq, d] bfloat16 (one query token per sequence)."""
    q = torch.empty(cfg.B, cfg.Hq, cfg.d, dtype=torch.bfloat16)
    for b in range(cfg.B):
        q[b] = _chunk(seed, cfg.workload, T_Q, b, 0, cfg.Hq, cfg.d, False, "bf16")
    return q


def decode_kv_head(cfg, tensor, b, kvh, L, seed=0):
    """[L, d] bfloat16 keys (tensor T_K) or values (T_V) of sequence b, key head kvh."""
    return _chunk(seed, cfg.workload, tensor, b, kvh, L, cfg.d, False, "bf16")


def decode_kv_padded(cfg, layout, tensor, seed=0, device="cpu"):
    """[B, Hkv, Lmax, d] bfloat16 with the rows past each context length zero."""
    Lmax = int(layout.ctx_len.max())
    out = torch.zeros(cfg.B, cfg.Hkv, Lmax, cfg.d, dtype=torch.bfloat16, device=device)
    for b in range(cfg.B):
        L = int(layout.ctx_len[b])
        for h in range(cfg.Hkv):
            out[b, h, :L] = decode_kv_head(cfg, tensor, b, h, L, seed).to(device)
    return out
