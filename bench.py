#!/usr/bin/env python3
"""Benchmark of block-scaled low-bit fused attention on one MI355X.

One step = the whole prefill path on the 32K causal workload with tile selection (B=1, H=32,
L=32768, d=128; the largest single-GPU prefill workload): MXFP4 quantization of Q and K with their
row norms and FP8 per-token quantization of V (with its P-fold data) in one launch, the top-5% tile
selection, then the fused attention kernel (MXFP4/FP8 tiles and bf16 selected tiles merged through
one online softmax), inputs resident in HBM. Each timed loop follows W untimed steps and at least
0.1 s of untimed back-to-back steps. `value` is prefill TFLOP/s over the step (algorithmic flops:
4 d per unmasked query-key pair). The line also carries:
  roofline      the attention kernel alone: its algorithmic flops / its average launch time (HIP
                events on the launch stream) against the dense MXFP4 MFMA peak, plus the kernel's
                HBM traffic per launch from the recorded FETCH_SIZE / WRITE_SIZE counters;
  error         the GPU output on sampled heads and rows against unquantized attention (float64
                softmax(q k^T / sqrt(d)) v of the bf16 originals): relative L2 and max-abs / max|O|;
                with tile selection also the error of the same kernel without selected tiles and the
                share of that error the selected tiles remove;
  legs          the other prefill workloads (4K causal MXFP4; 128K chunked prefill with NVFP4 +
                Hadamard and tile selection) and the 4K variants (4-bit V, MXFP8 Q/K, MXFP4
                probabilities, and both), each with its own roofline and error;
  decode        the paged NVFP4 decode step (64 sequences, 32 -> 8 GQA heads, contexts 8K-32K):
                KV-cache GB/s, the decode kernels' HBM roofline and the error;
  decode_mxfp4, decode_p4, decode_mxfp4_p4
                the same decode over an MXFP4 cache and / or with NVFP4 probabilities;
  decode_mla    decode in the MLA geometry (64 sequences, 16 heads over one shared 576-wide MXFP4
                latent row per token, value = its first 512 values, contexts 8K-32K);
  k_quant       (--outlier) quantization of the 128K-token chunked-prefill keys (NVFP4 + Hadamard)
                plain, with static smoothing, and with smoothing + the per-block scale search;
  cpu_baseline  the CPU oracle (float64 numpy) on a bounded sample of the headline workload.
Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-legs] [--no-decode]
                       [--no-error] [--no-cpu-baseline] [--quick] [--copy-probe] [--summarize-counters DIR]

HBM traffic: `--copy-probe` adds one untimed plain device copy of COPY_BYTES, so that a
`rocprofv3 --pmc FETCH_SIZE` (then `WRITE_SIZE`) run of this script records the counters of the
measured kernels and of a copy of known size together. `--summarize-counters DIR` turns the
counter CSVs under DIR into profiles/traffic.json: per kernel instantiation, the counter reads per
dispatch, each scaled by (known copy bytes / what the counter read for the copy), with a hash of the
kernel's sources. The benchmark reports that traffic only while the sources still hash the same
(the counters describe the kernel they were taken on), and null otherwise.
"""
import argparse
import csv
import glob
import hashlib
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import workloads as W  # noqa: E402

METRIC = "prefill attn TFLOP/s + decode KV GB/s, as % of MXFP4-MFMA / HBM peak"
MXFP4_PEAK_TFLOPS = 10100.0          # dense MFMA, FP4/FP6
FP8_PEAK_TFLOPS = 5000.0             # dense MFMA, FP8 (the peak of an MXFP8 QK^T workload)
BF16_PEAK_TFLOPS = 2500.0            # dense MFMA, bf16 / fp16
HBM_PEAK_GBS = 8000.0
COPY_BYTES = 1 << 30                 # calibration copy: reads and writes this many bytes
TRAFFIC_JSON = os.path.join(ROOT, "profiles", "traffic.json")
CSRC = os.path.join(ROOT, "fp8_quantized_attention_amd", "csrc")
# Kernel instantiations whose counters are recorded, with the sources whose change invalidates them.
# Attention kernel: <d, Q/K format (0 MXFP4, 1 NVFP4, 3 MXFP8), causal, selection, 4-bit V, MXFP4 P>
# (MXFP4 without selection: 4K causal; MXFP4 with selection: 32K; NVFP4 with selection: the 128K
# chunked prefill; MXFP4 probabilities, 4-bit V, both, and MXFP8: 4K causal). Decode: <cache format (1 NVFP4, 0 MXFP4), probability format (0 FP8, 1 NVFP4)>.
ATTN_SRC = ["attn_fwd.hip", "fa4_device.h"]
DEC_SRC = ["decode.hip", "fa4_device.h"]
KERNEL_SOURCES = {
    "attn_fwd_kernel<128, 0, true, false, false, false>": ATTN_SRC,
    "attn_fwd_kernel<128, 0, true, true, false, false>": ATTN_SRC,
    "attn_fwd_kernel<128, 1, true, true, false, false>": ATTN_SRC,
    "attn_fwd_kernel<128, 0, true, false, false, true>": ATTN_SRC,
    "attn_fwd_kernel<128, 0, true, false, true, true>": ATTN_SRC,
    "attn_fwd_kernel<128, 0, true, false, true, false>": ATTN_SRC,
    "attn_fwd_kernel<128, 3, true, false, false, false>": ATTN_SRC,
    "decode_split_kernel<1, 0>": DEC_SRC,
    "decode_split_kernel<0, 0>": DEC_SRC,
    "decode_split_kernel<1, 1>": DEC_SRC,
    "decode_split_kernel<0, 1>": DEC_SRC,
    "decode_mla_kernel": ["decode_mla.hip", "fa4_device.h"],
}
PREFILL = [W.C1, W.C2, W.C4, W.C1_MX8, W.C1_V4, W.C1_P4, W.C1_V4P4]


def attn_kernel_name(cfg, select):
    """The attention kernel instantiation fa4_attn_fwd launches for this workload."""
    fmt = {"mxfp4": 0, "nvfp4": 1, "mxfp8": 3}[cfg.qk_fmt]
    b = lambda x: "true" if x else "false"   # noqa: E731
    return (f"attn_fwd_kernel<{cfg.d}, {fmt}, {b(cfg.causal)}, {b(select)}, {b(cfg.v_fmt == 'mxfp4k')}, "
            f"{b(cfg.p_fmt == 'mxfp4')}>")


def sources_sha(kernel):
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def copy_probe():
    """One plain device-to-device copy of COPY_BYTES (the counters' calibration kernel)."""
    src = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst
    torch.cuda.empty_cache()


def summarize_counters(root):
    """Counter CSVs (rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE runs of `bench.py --copy-probe`) ->
    profiles/traffic.json with per-dispatch bytes for the measured kernels. The calibration copy is
    the runtime's copy kernel dispatch that moved at least a quarter of COPY_BYTES (the input
    uploads are far smaller)."""
    rows = {}                                            # (key, counter) -> {dispatch: KiB}
    for f in glob.glob(os.path.join(root, "**", "*counter_collection.csv"), recursive=True):
        for r in csv.DictReader(open(f)):
            name, ctr, kib = r["Kernel_Name"], r["Counter_Name"], float(r["Counter_Value"])
            key = next((k for k in KERNEL_SOURCES if k in name), None)
            if key is None and "copyBuffer" in name and kib * 1024.0 >= COPY_BYTES / 4:
                key = "copy"
            if key is not None:
                d = rows.setdefault((key, ctr), {})
                d[(f, r["Dispatch_Id"])] = d.get((f, r["Dispatch_Id"]), 0.0) + kib
    per = {k: sum(d.values()) / len(d) for k, d in rows.items()}
    fac = {c: COPY_BYTES / (per[("copy", c)] * 1024.0) for c in ("FETCH_SIZE", "WRITE_SIZE") if ("copy", c) in per}
    out = {"copy_bytes": COPY_BYTES, "copy_kib_raw": {c: per[("copy", c)] for c in fac}, "scale": fac,
           "kernels": {}}
    try:                                                 # keep kernels this run did not cover
        with open(TRAFFIC_JSON) as fh:
            out["kernels"] = {k: v for k, v in json.load(fh).get("kernels", {}).items() if k in KERNEL_SOURCES}
    except (OSError, ValueError):
        pass
    for k in KERNEL_SOURCES:
        if (k, "FETCH_SIZE") in per and (k, "WRITE_SIZE") in per and len(fac) == 2:
            fb = per[(k, "FETCH_SIZE")] * 1024.0 * fac["FETCH_SIZE"]
            wb = per[(k, "WRITE_SIZE")] * 1024.0 * fac["WRITE_SIZE"]
            out["kernels"][k] = {"fetch_kib_raw": per[(k, "FETCH_SIZE")], "write_kib_raw": per[(k, "WRITE_SIZE")],
                                 "fetch_bytes": fb, "write_bytes": wb, "traffic_bytes": fb + wb,
                                 "dispatches": len(rows[(k, "FETCH_SIZE")]), "sources_sha": sources_sha(k)}
    os.makedirs(os.path.dirname(TRAFFIC_JSON), exist_ok=True)
    with open(TRAFFIC_JSON, "w") as fh:
        json.dump(out, fh, indent=1)
    print(json.dumps(out, indent=1))


def recorded_traffic(kernel):
    """HBM bytes per dispatch recorded for `kernel`, or None when absent or taken on other sources."""
    try:
        with open(TRAFFIC_JSON) as fh:
            rec = json.load(fh)["kernels"][kernel]
    except (OSError, KeyError, ValueError):
        return None
    return rec["traffic_bytes"] if rec.get("sources_sha") == sources_sha(kernel) else None


def causal_pairs(Lq, Lk, causal):
    if not causal:
        return Lq * Lk
    off = Lk - Lq
    return sum(min(Lk, off + r + 1) for r in range(Lq))


def prefill_flops(cfg):
    return 4.0 * cfg.d * causal_pairs(cfg.Lq, cfg.Lk, cfg.causal) * cfg.B * cfg.Hq


WARM_S = 0.1


def _warm(fn, n, quick=False):
    """n untimed calls, continued until at least WARM_S seconds of back-to-back work have run, so that
    the timed loop does not start on clocks still ramping up after the host-side input generation."""
    for _ in range(n):
        fn()
    torch.cuda.synchronize()
    if quick:
        return
    t = time.perf_counter()
    while time.perf_counter() - t < WARM_S:
        for _ in range(8):
            fn()
        torch.cuda.synchronize()


def _time_loop(fn, n):
    """Average ms of n back-to-back calls of fn, HIP events on the current (launch) stream."""
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record()
    for _ in range(n):
        fn()
    t1.record()
    torch.cuda.synchronize()
    return t0.elapsed_time(t1) / n


# ---------------------------------------------------------------------------------------------- errors

def _rel(got, ref):
    got, ref = np.asarray(got, np.float64), np.asarray(ref, np.float64)
    return (float(np.linalg.norm(got - ref) / np.linalg.norm(ref)),
            float(np.abs(got - ref).max() / np.abs(ref).max()))


def exact_attention_rows(q, k, v, rows, off, causal, scale):
    """float64 softmax(q k^T * scale) v for query rows `rows` of one head (q [Lq, d], k/v [Lk, d],
    float64), query i at key position off + i when causal. Unquantized: the reference for the error."""
    s = (q[rows] @ k.T) * scale
    if causal:
        s = np.where(np.arange(k.shape[0])[None, :] > (off + rows)[:, None], -np.inf, s)
    s -= s.max(axis=1, keepdims=True)
    p = np.exp(s)
    return (p @ v) / p.sum(axis=1, keepdims=True)


def sample_heads_rows(cfg):
    heads = [(0, 0), (0, cfg.Hq // 2 + 1)]
    rows = np.unique(np.concatenate([np.linspace(0, cfg.Lq - 1, 96).astype(np.int64),
                                     np.arange(cfg.Lq - 32, cfg.Lq)]))
    return heads, rows


def prefill_error(cfg, q, k, v, outs):
    """Error of each GPU output in `outs` ({name: o [B, Hq, Lq, d] tensor}) against unquantized
    attention on the sampled heads and rows."""
    heads, rows = sample_heads_rows(cfg)
    group = cfg.Hq // cfg.Hkv
    ref, got = [], {n: [] for n in outs}
    for (b, h) in heads:
        qh = q[b, h].double().cpu().numpy()
        kh = k[b, h // group].double().cpu().numpy()
        vh = v[b, h // group].double().cpu().numpy()
        ref.append(exact_attention_rows(qh, kh, vh, rows, cfg.Lk - cfg.Lq, cfg.causal, cfg.d ** -0.5))
        for n, o in outs.items():
            got[n].append(o[b, h][torch.from_numpy(rows).to(o.device)].cpu().numpy())
    res = {"sample": f"heads {heads}, {len(rows)} query rows (96 spread + the last 32)", "reference":
           "unquantized float64 attention of the bf16 inputs"}
    for n in outs:
        rel, mx = _rel(np.stack(got[n]), np.stack(ref))
        res[n] = {"rel_l2": rel, "max_abs_over_max": mx}
    return res


# ---------------------------------------------------------------------------------------------- prefill

def visited_tiles(cfg):
    """128 x 128 (query, key) tiles the attention visits (those holding an unmasked pair)."""
    nq, nk, off = cfg.Lq // 128, cfg.Lk // 128, cfg.Lk - cfg.Lq
    per_head = sum(min(nk, (off + 128 * i + 127) // 128 + 1) if cfg.causal else nk for i in range(nq))
    return per_head * cfg.B * cfg.Hq


def mixed_ceiling_tflops(cfg, bf16_frac):
    """The dense-MFMA ceiling of the workload's mix of products: half of the flops are QK^T at the Q/K
    format's rate (MXFP4 10.1 PF and MXFP8 5.0 PF, both with native block scales; NVFP4, whose E4M3
    scales on 16 elements the matrix cores do not take, at the fp16 rate 2.5 PF), half PV at the V/P
    rate (FP8 5.0 PF; 4-bit V times FP8 P and FP8 V times FP4 P also run at the FP8 rate, 4-bit V times
    FP4 P at the FP4 rate), and the selected tiles' share of both at the bf16 rate (2.5 PF)."""
    qk = {"mxfp4": MXFP4_PEAK_TFLOPS, "nvfp4": BF16_PEAK_TFLOPS, "mxfp8": FP8_PEAK_TFLOPS}[cfg.qk_fmt]
    pv = MXFP4_PEAK_TFLOPS if (cfg.v_fmt == "mxfp4k" and cfg.p_fmt == "mxfp4") else FP8_PEAK_TFLOPS
    f = bf16_frac
    per_tflop = 0.5 * ((1 - f) / qk + f / BF16_PEAK_TFLOPS) + 0.5 * ((1 - f) / pv + f / BF16_PEAK_TFLOPS)
    return 1.0 / per_tflop


def time_prefill(fa4, cfg, steps, warmup, quick=False, error=True):
    """Times one prefill workload: (ms per whole step, ms per attention launch, error dict or None,
    fraction of visited tiles computed in bf16).
    The step loop has no events inside it; the attention kernel is timed on its own loop of
    back-to-back launches over the same inputs."""
    q, k, v = (t.cuda() for t in W.prefill_inputs(cfg))
    fmt = {"mxfp4": fa4.FA4_MXFP4, "nvfp4": fa4.FA4_NVFP4, "mxfp8": fa4.FA4_MXFP8}[cfg.qk_fmt]
    vf = fa4.FA4_MXFP4_KEYS if cfg.v_fmt == "mxfp4k" else fa4.FA4_FP8_TOKEN
    pf = fa4.FA4_P_MXFP4 if cfg.p_fmt == "mxfp4" else fa4.FA4_P_FP8
    select = (5, 100) if cfg.select else None
    run = fa4.PrefillRunner(q, k, v, cfg.causal, fmt=fmt, hadamard=cfg.hadamard, select=select, v_fmt=vf,
                            p_fmt=pf)
    _warm(run.run, warmup, quick)
    step_ms = _time_loop(run.run, steps)
    attn_ms = _time_loop(run.attention, steps)
    bf16_frac = float(run.counts.sum().item()) / visited_tiles(cfg) if select is not None else 0.0
    err = None
    if error:
        run.run()
        outs = {"gpu": run.o}
        if select is not None:          # the same quantized operands without selected tiles
            o_ns, _ = fa4.attn_fwd(run.qq, run.kq, run.vq, cfg.causal, fmt, cfg.Hq, cfg.Hkv, cfg.Lq, cfg.Lk, cfg.d,
                                   B=cfg.B, want_lse=False, v_fmt=vf, p_fmt=pf)
            outs["gpu_no_selection"] = o_ns
        torch.cuda.synchronize()
        err = prefill_error(cfg, q, k, v, outs)
        if select is not None:
            e1, e0 = err["gpu"]["rel_l2"], err["gpu_no_selection"]["rel_l2"]
            err["selection_gap_recovered"] = 1.0 - e1 / e0
    del run, q, k, v
    torch.cuda.empty_cache()
    return step_ms, attn_ms, err, bf16_frac


def prefill_record(fa4, cfg, args, headline=False):
    step_ms, attn_ms, err, bf16_frac = time_prefill(fa4, cfg, args.steps, args.warmup, args.quick, not args.no_error)
    mixed = mixed_ceiling_tflops(cfg, bf16_frac)
    flops = prefill_flops(cfg)
    achieved = flops / (attn_ms * 1e-3) / 1e12
    peak = FP8_PEAK_TFLOPS if cfg.qk_fmt == "mxfp8" else MXFP4_PEAK_TFLOPS
    kname = attn_kernel_name(cfg, cfg.select)
    rec = {
        "workload": cfg.name, "value": flops / (step_ms * 1e-3) / 1e12, "unit": "TFLOP/s", "ms_per_step": step_ms,
        "dtype": cfg.qk_fmt + ("+fp4v" if cfg.v_fmt == "mxfp4k" else "+fp8") + ("+fp4p" if cfg.p_fmt == "mxfp4" else "")
        + ("+bf16tiles" if cfg.select else ""),
        "config": {"workload": cfg.name, "B": cfg.B, "Hq": cfg.Hq, "Hkv": cfg.Hkv, "Lq": cfg.Lq, "Lk": cfg.Lk,
                   "d": cfg.d, "causal": cfg.causal, "qk_format": cfg.qk_fmt, "hadamard": cfg.hadamard,
                   "bf16_tiles": "5%" if cfg.select else "none", "algorithmic_flops": flops},
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": peak, "unit": "TFLOP/s",
                     "frac": achieved / peak, "traffic": recorded_traffic(kname) if kname in KERNEL_SOURCES else None,
                     "kernel": kname, "kernel_ms": attn_ms,
                     "mixed_ceiling": {"peak": mixed, "frac": achieved / mixed, "bf16_tile_fraction": bf16_frac,
                                       "note": "QK^T and PV each at their operand formats' dense MFMA rate"}},
        "other_kernels_ms": step_ms - attn_ms,
        "error_vs_unquantized": err,
    }
    print(f"[bench] prefill {cfg.name}: step {step_ms:.4f} ms, attention {attn_ms:.4f} ms "
          f"({achieved:.0f} TFLOP/s, {100 * achieved / peak:.1f}% of peak)", file=sys.stderr, flush=True)
    return rec


# ---------------------------------------------------------------------------------------------- decode

_KV_CACHE = {}


def decode_kv_inputs(cfg):
    """Padded K and V of a decode workload on the GPU, generated once per (workload id, shape): the
    cache- and probability-format variants of one workload share their sequences and values."""
    key = (cfg.workload, cfg.B, cfg.Hkv, cfg.d, cfg.ctx_lo, cfg.ctx_hi)
    if key not in _KV_CACHE:
        _KV_CACHE.clear()
        lay = W.decode_layout(cfg)
        _KV_CACHE[key] = (lay, [W.decode_kv_padded(cfg, lay, t, device="cuda") for t in (W.T_K, W.T_V)])
    return _KV_CACHE[key]


DEC_PAIRS = [(0, 0), (7, 5), (21, 13), (33, 30), (50, 18), (63, 31)]


def decode_error(q, k, v, ctx, o, pairs, group, scale, d_v=None):
    """GPU decode output vs unquantized float64 attention of the bf16 query and cache rows."""
    ref, got = [], []
    for (b, h) in pairs:
        L = int(ctx[b])
        kh = k[b, h // group, :L].double().cpu().numpy()
        vh = (v[b, h // group, :L] if v is not None else k[b, h // group, :L, :d_v]).double().cpu().numpy()
        qh = q[b, h].double().cpu().numpy()
        s = (kh @ qh) * scale
        p = np.exp(s - s.max())
        ref.append((p @ vh) / p.sum())
        got.append(o[b, h].cpu().numpy())
    rel, mx = _rel(np.stack(got), np.stack(ref))
    return {"sample": f"(sequence, head) pairs {pairs}", "reference": "unquantized float64 attention of the bf16 "
            "query and cache rows", "gpu": {"rel_l2": rel, "max_abs_over_max": mx}}


def time_decode(fa4, cfg, steps, warmup, quick=False, error=True):
    lay, xs = decode_kv_inputs(cfg)
    ctx, pt = lay.ctx_len.cuda(), lay.page_table.cuda()
    nv = cfg.kv_fmt == "nvfp4"
    caches = [fa4.quantize_paged(x, fa4.FA4_NVFP4 if nv else fa4.FA4_MXFP4, ctx, pt, lay.num_pages) for x in xs]
    q = W.decode_query(cfg).cuda()
    run = fa4.DecodeRunner(q, caches[0], caches[1], pt, ctx, cfg.Hkv,
                           p_fmt=fa4.FA4_P_NVFP4 if cfg.p_fmt == "nvfp4" else fa4.FA4_P_FP8)
    _warm(run.run, warmup, quick)
    step_ms = _time_loop(run.run, steps)
    kern_ms = _time_loop(run.attention, steps)
    err = None
    if error:
        run.run()
        torch.cuda.synchronize()
        err = decode_error(q, xs[0], xs[1], lay.ctx_len, run.o, DEC_PAIRS, cfg.Hq // cfg.Hkv, cfg.d ** -0.5)
    # K and V codes plus block scales (d/16 E4M3 or d/32 E8M0 bytes) per (token, key head)
    kv_bytes = float(lay.ctx_len.double().sum()) * cfg.Hkv * 2 * (cfg.d // 2 + cfg.d // (16 if nv else 32))
    return step_ms, kern_ms, kv_bytes, int(lay.ctx_len.sum()), err


def time_decode_mla(fa4, cfg, steps, warmup, quick=False, error=True):
    _KV_CACHE.clear()
    torch.cuda.empty_cache()
    lay = W.decode_layout(cfg)
    ctx, pt = lay.ctx_len.cuda(), lay.page_table.cuda()
    x = W.decode_kv_padded(cfg, lay, W.T_K, device="cuda")
    cache = fa4.quantize_paged_mla(x[:, 0].contiguous(), ctx, pt, lay.num_pages)
    q = W.decode_query(cfg).cuda()
    run = fa4.DecodeMlaRunner(q, cache, pt, ctx, cfg.softmax_scale)
    _warm(run.run, warmup, quick)
    step_ms = _time_loop(run.run, steps)
    kern_ms = _time_loop(run.attention, steps)
    err = None
    if error:
        run.run()
        torch.cuda.synchronize()
        err = decode_error(q, x, None, lay.ctx_len, run.o, [(b, h % 16) for b, h in DEC_PAIRS], cfg.Hq,
                           cfg.softmax_scale, d_v=cfg.d_v)
    del x
    torch.cuda.empty_cache()
    # one latent row per token: d/2 code bytes + d/32 E8M0 bytes
    kv_bytes = float(lay.ctx_len.double().sum()) * (cfg.d // 2 + cfg.d // 32)
    return step_ms, kern_ms, kv_bytes, int(lay.ctx_len.sum()), err


def decode_record(key, dcfg, step_ms, kern_ms, kv_bytes, tokens, err, kname, kernel):
    gbs = kv_bytes / (kern_ms * 1e-3) / 1e9
    print(f"[bench] {key} ({dcfg.kv_fmt}, P {dcfg.p_fmt}): step {step_ms:.4f} ms, kernels {kern_ms:.4f} ms, "
          f"{gbs:.0f} GB/s", file=sys.stderr, flush=True)
    return {"metric": "decode KV GB/s", "workload": dcfg.name, "value": kv_bytes / (step_ms * 1e-3) / 1e9,
            "unit": "GB/s", "ms_per_step": step_ms, "kv_bytes": kv_bytes, "context_tokens": tokens,
            "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": gbs / HBM_PEAK_GBS, "traffic": recorded_traffic(kname),
                         "traffic_kernel": kname, "kernel": kernel, "kernel_ms": kern_ms},
            "error_vs_unquantized": err}


def time_k_quant(fa4, steps, warmup):
    """Outlier-aware key quantization on the chunked-prefill workload's keys (B1, 8 key heads, 131072
    tokens, d128, bf16 with x20 outlier channels): NVFP4 + Hadamard, plain / smoothing / smoothing + search.
    The smoothing factors come from a 2048-token calibration prefix of Q and K."""
    cfg = W.C4
    q, k, _ = W.prefill_inputs(cfg)
    qc, kc = q.cuda(), k.cuda()
    del q, k
    qs, ks = fa4.smoothing_factors(qc, kc[:, :, :2048].contiguous())
    in_bytes = kc.numel() * 2
    out_bytes = kc.numel() // 2 + kc.numel() // 16 + 4 * cfg.Hkv
    res = {"workload": cfg.name + " keys", "rows": cfg.Lk, "heads": cfg.Hkv, "format": "nvfp4+hadamard",
           "algorithmic_bytes": 2 * in_bytes + out_bytes, "note": "two passes over the input (tensor maximum, codes)"}
    for name, cs, search in (("plain", None, False), ("smoothing", ks, False), ("smoothing+search", ks, True)):
        run = fa4.QuantizeRunner(kc, fa4.FA4_NVFP4, hadamard=True, channel_scale=cs, search=search)
        _warm(run.run, warmup)
        ms = _time_loop(run.run, steps)
        res[name] = {"ms": ms, "GB/s": (2 * in_bytes + out_bytes) / (ms * 1e-3) / 1e9}
        print(f"[bench] k_quant {name}: {ms:.4f} ms", file=sys.stderr, flush=True)
    del qc, kc
    torch.cuda.empty_cache()
    return res


# ---------------------------------------------------------------------------------------------- CPU oracle

def cpu_baseline(cfg, rows_n):
    """The oracle as it stands on one query head of the workload: quantize that head's Q, K and V
    (whole sequence), select its tiles, attend `rows_n` query rows spread over the sequence."""
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    from oracle_cases import prefill_reference
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        threads = 1
    rows = np.unique(np.linspace(0, cfg.Lq - 1, rows_n).astype(np.int64))
    t = time.time()
    prefill_reference(cfg, 0, [(0, 0)], rows, (5, 100) if cfg.select else None)
    secs = time.time() - t
    off = cfg.Lk - cfg.Lq
    pairs = float(np.minimum(cfg.Lk, off + rows + 1).sum()) if cfg.causal else float(len(rows) * cfg.Lk)
    flops = 4.0 * cfg.d * pairs
    return {"value": flops / secs / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "host_cpu_count": os.cpu_count(), "affinity_cpus": len(os.sched_getaffinity(0)),
            "sample": f"head (0, 0) of {cfg.name}: quantize its Q, K, V ({cfg.Lk} rows each)"
                      f"{', select its tiles' if cfg.select else ''}, attend {len(rows)} query rows spread over "
                      f"the sequence ({pairs:.3g} query-key pairs); {secs:.1f} s; cores = the numpy BLAS threads "
                      f"(element-wise numpy runs on one)"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=W.C2.name, choices=[c.name for c in PREFILL])
    ap.add_argument("--no-legs", action="store_true", help="skip the other prefill workloads")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-p4", action="store_true", help="skip the decode steps with NVFP4 probabilities")
    ap.add_argument("--no-error", action="store_true", help="skip the errors against unquantized attention")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=160, help="query rows of the CPU oracle's sample")
    ap.add_argument("--quick", action="store_true", help="no 0.1 s warm loop (profiler runs)")
    ap.add_argument("--copy-probe", action="store_true")
    ap.add_argument("--outlier", action="store_true", help="also time the outlier-aware key quantization")
    ap.add_argument("--summarize-counters", metavar="DIR")
    args = ap.parse_args()
    if args.summarize_counters:
        summarize_counters(args.summarize_counters)
        return
    if args.gpus != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    import fp8_quantized_attention_amd as fa4

    cfg = next(c for c in PREFILL if c.name == args.workload)
    if args.copy_probe:
        copy_probe()
    head = prefill_record(fa4, cfg, args, headline=True)
    line = {
        "metric": METRIC,
        "value": head["value"],
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": head["dtype"],
        "data": "synthetic",
        "config": head["config"],
        "roofline": head["roofline"],
        "other_kernels_ms": head["other_kernels_ms"],
        "error_vs_unquantized": head["error_vs_unquantized"],
    }
    if not args.no_legs:
        line["legs"] = {}
        for lcfg in (W.C1, W.C2, W.C4, W.C1_V4, W.C1_MX8, W.C1_P4, W.C1_V4P4):
            if lcfg.name != cfg.name:
                line["legs"][lcfg.name] = prefill_record(fa4, lcfg, args)
    if not args.no_decode:
        dec = [("decode", W.C3), ("decode_mxfp4", W.C3_MX)]
        if not args.no_p4:
            dec += [("decode_p4", W.C3_P4), ("decode_mxfp4_p4", W.C3_MX_P4)]
        for key, dcfg in dec:
            res = time_decode(fa4, dcfg, args.steps, args.warmup, args.quick, not args.no_error)
            kname = "decode_split_kernel<%d, %d>" % (dcfg.kv_fmt == "nvfp4", dcfg.p_fmt == "nvfp4")
            line[key] = decode_record(key, dcfg, *res, kname, "decode_split+combine")
            torch.cuda.empty_cache()
        _KV_CACHE.clear()
        res = time_decode_mla(fa4, W.C5_MLA, args.steps, args.warmup, args.quick, not args.no_error)
        line["decode_mla"] = decode_record("decode_mla", W.C5_MLA, *res, "decode_mla_kernel", "decode_mla+combine")
        torch.cuda.empty_cache()
    if args.outlier:
        line["k_quant"] = time_k_quant(fa4, args.steps, args.warmup)
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(cfg, args.cpu_rows)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
