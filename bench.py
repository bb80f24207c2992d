#!/usr/bin/env python3
"""Benchmark of block-scaled low-bit fused attention on one MI355X.

One step = the whole prefill path on the 4K causal workload (B=1, H=32, L=4096, d=128): MXFP4
quantization of Q and K and FP8 per-token quantization of V (with its P-fold data), in one launch,
then the fused attention kernel, inputs resident in HBM. Each timed loop follows W untimed steps and
at least 0.1 s of untimed back-to-back steps. `value` is prefill attention TFLOP/s over the step
(algorithmic flops: 4 d per unmasked query-key pair). The same line carries:
  roofline      the attention kernel alone: its algorithmic flops / its average launch time (HIP
                events on the launch stream) against the dense MXFP4 MFMA peak;
  decode        the paged NVFP4 decode step (64 sequences, 32 -> 8 GQA heads, contexts 8K-32K):
                KV-cache GB/s, and the decode kernels' HBM roofline;
  decode_mxfp4  the same decode step over an MXFP4 cache (same sequences and values);
  decode_p4, decode_mxfp4_p4
                the two decode steps with the probabilities in NVFP4 (E4M3 scales per 16 keys)
                instead of FP8;
  decode_mla    decode in the MLA geometry (64 sequences, 16 heads over one shared 576-wide MXFP4
                latent row per token, value = its first 512 values, contexts 8K-32K): KV GB/s;
  k_quant       (--outlier) quantization of the 128K-token chunked-prefill keys (NVFP4 + Hadamard)
                plain, with static smoothing, and with smoothing + the per-block scale search;
  cpu_baseline  the CPU oracle (float64 numpy) on a bounded sample of the same workload.
Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-decode] [--no-cpu-baseline]
                       [--copy-probe] [--summarize-counters DIR]

HBM traffic: `--copy-probe` adds one untimed plain device copy of COPY_BYTES, so that a
`rocprofv3 --pmc FETCH_SIZE` (then `WRITE_SIZE`) run of this script records the counters of the
measured kernels and of a copy of known size together. `--summarize-counters DIR` turns the
counter CSVs under DIR into profiles/traffic.json: per kernel, the counter reads per dispatch, each
scaled by (known copy bytes / what the counter read for the copy), with a hash of the kernel's
sources. The benchmark reports that traffic only while the sources still hash the same (the
counters describe the kernel they were taken on), and null otherwise.
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
HBM_PEAK_GBS = 8000.0
COPY_BYTES = 1 << 30                 # calibration copy: reads and writes this many bytes
TRAFFIC_JSON = os.path.join(ROOT, "profiles", "traffic.json")
CSRC = os.path.join(ROOT, "fp8_quantized_attention_amd", "csrc")
# sources whose change invalidates a kernel's recorded counters
# (template arguments of the decode kernel: cache format 1 = NVFP4, 0 = MXFP4; probability format
# 0 = FP8, 1 = NVFP4)
KERNEL_SOURCES = {
    "attn_fwd_kernel": ["attn_fwd.hip", "fa4_device.h"],
    "decode_split_kernel<1, 0>": ["decode.hip", "fa4_device.h"],
    "decode_split_kernel<0, 0>": ["decode.hip", "fa4_device.h"],
    "decode_split_kernel<1, 1>": ["decode.hip", "fa4_device.h"],
    "decode_split_kernel<0, 1>": ["decode.hip", "fa4_device.h"],
    "decode_mla_kernel": ["decode_mla.hip", "fa4_device.h"],
}


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


def _warm(fn, n):
    """n untimed calls, continued until at least WARM_S seconds of back-to-back work have run, so that
    the timed loop does not start on clocks still ramping up after the host-side input generation."""
    for _ in range(n):
        fn()
    torch.cuda.synchronize()
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


def time_prefill(fa4, cfg, steps, warmup, select):
    """(ms per whole step, ms per attention launch). The step loop has no events inside it; the
    attention kernel is timed on its own loop of back-to-back launches over the same inputs."""
    q, k, v = (t.cuda() for t in W.prefill_inputs(cfg))
    fmt = {"mxfp4": fa4.FA4_MXFP4, "nvfp4": fa4.FA4_NVFP4, "mxfp8": fa4.FA4_MXFP8}[cfg.qk_fmt]
    vf = fa4.FA4_MXFP4_KEYS if cfg.v_fmt == "mxfp4k" else fa4.FA4_FP8_TOKEN
    run = fa4.PrefillRunner(q, k, v, cfg.causal, fmt=fmt, hadamard=cfg.hadamard, select=select, v_fmt=vf)
    _warm(run.run, warmup)
    step_ms = _time_loop(run.run, steps)
    attn_ms = _time_loop(run.attention, steps)
    return step_ms, attn_ms


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


def time_decode(fa4, cfg, steps, warmup):
    lay, xs = decode_kv_inputs(cfg)
    ctx, pt = lay.ctx_len.cuda(), lay.page_table.cuda()
    nv = cfg.kv_fmt == "nvfp4"
    caches = [fa4.quantize_paged(x, fa4.FA4_NVFP4 if nv else fa4.FA4_MXFP4, ctx, pt, lay.num_pages) for x in xs]
    q = W.decode_query(cfg).cuda()
    run = fa4.DecodeRunner(q, caches[0], caches[1], pt, ctx, cfg.Hkv,
                           p_fmt=fa4.FA4_P_NVFP4 if cfg.p_fmt == "nvfp4" else fa4.FA4_P_FP8)
    _warm(run.run, warmup)
    step_ms = _time_loop(run.run, steps)
    kern_ms = _time_loop(run.attention, steps)
    # K and V codes plus block scales (d/16 E4M3 or d/32 E8M0 bytes) per (token, key head)
    kv_bytes = float(lay.ctx_len.double().sum()) * cfg.Hkv * 2 * (cfg.d // 2 + cfg.d // (16 if nv else 32))
    return step_ms, kern_ms, kv_bytes, int(lay.ctx_len.sum())


def time_decode_mla(fa4, cfg, steps, warmup):
    _KV_CACHE.clear()
    torch.cuda.empty_cache()
    lay = W.decode_layout(cfg)
    ctx, pt = lay.ctx_len.cuda(), lay.page_table.cuda()
    x = W.decode_kv_padded(cfg, lay, W.T_K, device="cuda")[:, 0].contiguous()
    cache = fa4.quantize_paged_mla(x, ctx, pt, lay.num_pages)
    del x
    torch.cuda.empty_cache()
    q = W.decode_query(cfg).cuda()
    run = fa4.DecodeMlaRunner(q, cache, pt, ctx, cfg.softmax_scale)
    _warm(run.run, warmup)
    step_ms = _time_loop(run.run, steps)
    kern_ms = _time_loop(run.attention, steps)
    # one latent row per token: d/2 code bytes + d/32 E8M0 bytes
    kv_bytes = float(lay.ctx_len.double().sum()) * (cfg.d // 2 + cfg.d // 32)
    return step_ms, kern_ms, kv_bytes, int(lay.ctx_len.sum())


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


def cpu_baseline(cfg, heads):
    """The oracle as it stands on `heads` query heads of the workload (quantize + attend every row)."""
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    from oracle_cases import prefill_reference
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        cores = os.cpu_count()
    t = time.time()
    prefill_reference(cfg, 0, [(0, h) for h in range(heads)], np.arange(cfg.Lq))
    secs = time.time() - t
    flops = prefill_flops(cfg) * heads / (cfg.B * cfg.Hq)
    return {"value": flops / secs / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": f"{heads} of {cfg.Hq} heads, all {cfg.Lq} query rows (quantize Q/K/V + attention), "
                      f"{secs:.1f} s"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=W.C1.name,
                    choices=[c.name for c in W.WORKLOADS + [W.C1_MX8, W.C1_V4] if isinstance(c, W.Prefill)])
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-p4", action="store_true", help="skip the decode steps with NVFP4 probabilities")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-heads", type=int, default=32)
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

    cfg = next(c for c in W.WORKLOADS + [W.C1_MX8, W.C1_V4] if c.name == args.workload)
    select = (5, 100) if cfg.select else None
    if args.copy_probe:
        copy_probe()
    step_ms, attn_ms = time_prefill(fa4, cfg, args.steps, args.warmup, select)
    flops = prefill_flops(cfg)
    achieved = flops / (attn_ms * 1e-3) / 1e12
    peak = FP8_PEAK_TFLOPS if cfg.qk_fmt == "mxfp8" else MXFP4_PEAK_TFLOPS
    line = {
        "metric": METRIC,
        "value": flops / (step_ms * 1e-3) / 1e12,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": step_ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.qk_fmt + ("+fp4v" if cfg.v_fmt == "mxfp4k" else "+fp8"),
        "data": "synthetic",
        "config": {"workload": cfg.name, "B": cfg.B, "Hq": cfg.Hq, "Hkv": cfg.Hkv, "Lq": cfg.Lq, "Lk": cfg.Lk,
                   "d": cfg.d, "causal": cfg.causal, "qk_format": cfg.qk_fmt, "hadamard": cfg.hadamard,
                   "bf16_tiles": "5%" if select else "none", "algorithmic_flops": flops},
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": peak, "unit": "TFLOP/s",
                     "frac": achieved / peak, "traffic": recorded_traffic("attn_fwd_kernel")
                     if cfg.name == W.C1.name else None, "kernel": "attn_fwd_kernel",
                     "kernel_ms": attn_ms},
    }
    print(f"[bench] prefill {cfg.name}: step {step_ms:.4f} ms, attention {attn_ms:.4f} ms", file=sys.stderr,
          flush=True)
    if not args.no_decode:
        dec = [("decode", W.C3), ("decode_mxfp4", W.C3_MX)]
        if not args.no_p4:
            dec += [("decode_p4", W.C3_P4), ("decode_mxfp4_p4", W.C3_MX_P4)]
        for key, dcfg in dec:
            d_step, d_kern, kv_bytes, tokens = time_decode(fa4, dcfg, args.steps, args.warmup)
            gbs = kv_bytes / (d_kern * 1e-3) / 1e9
            kname = "decode_split_kernel<%d, %d>" % (dcfg.kv_fmt == "nvfp4", dcfg.p_fmt == "nvfp4")
            line[key] = {
                "metric": "decode KV GB/s", "workload": dcfg.name, "value": kv_bytes / (d_step * 1e-3) / 1e9,
                "unit": "GB/s", "ms_per_step": d_step, "kv_bytes": kv_bytes, "context_tokens": tokens,
                "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                             "frac": gbs / HBM_PEAK_GBS, "traffic": recorded_traffic(kname),
                             "traffic_kernel": kname, "kernel": "decode_split+combine", "kernel_ms": d_kern}}
            print(f"[bench] {key} ({dcfg.kv_fmt}, P {dcfg.p_fmt}): step {d_step:.4f} ms, kernels {d_kern:.4f} ms, {gbs:.0f} GB/s",
                  file=sys.stderr, flush=True)
            torch.cuda.empty_cache()
        dcfg = W.C5_MLA
        d_step, d_kern, kv_bytes, tokens = time_decode_mla(fa4, dcfg, args.steps, args.warmup)
        gbs = kv_bytes / (d_kern * 1e-3) / 1e9
        line["decode_mla"] = {
            "metric": "decode KV GB/s", "workload": dcfg.name, "value": kv_bytes / (d_step * 1e-3) / 1e9,
            "unit": "GB/s", "ms_per_step": d_step, "kv_bytes": kv_bytes, "context_tokens": tokens,
            "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": gbs / HBM_PEAK_GBS, "traffic": recorded_traffic("decode_mla_kernel"),
                         "traffic_kernel": "decode_mla_kernel", "kernel": "decode_mla+combine", "kernel_ms": d_kern}}
        print(f"[bench] decode_mla (mxfp4): step {d_step:.4f} ms, kernels {d_kern:.4f} ms, {gbs:.0f} GB/s",
              file=sys.stderr, flush=True)
        torch.cuda.empty_cache()
    if args.outlier:
        line["k_quant"] = time_k_quant(fa4, args.steps, args.warmup)
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(cfg, min(args.cpu_heads, cfg.Hq))
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
