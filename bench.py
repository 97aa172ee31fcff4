#!/usr/bin/env python3
"""Benchmark: one decode-attention layer step over a long KV cache on one MI355X.

A step is one pass of the whole path over one batch: kvd_decode_partial
(split-KV partial attention for every request, KV head and shard) followed by
kvd_lse_merge (exact merge of the shards), both through the C ABI on one HIP
stream, with the synthetic cache already resident in HBM.  The default
workload is the Helix Figure-1 dense shape on one GPU: B=8 requests, 128
query heads on 8 KV heads, Hsz=128, S=2^20 tokens each, fp8 E4M3 cache with
one fp32 scale per (request, KV head), bf16 queries, KVP=32 shards.

Prints one JSON line.  `value` is KV-read GB/s: the algorithmic cache bytes of
one step (every cached element read once) divided by the measured time per
step.  The roofline object is for the dominant kernel (the partial pass),
timed with HIP events on the stream it runs on; its `traffic` field comes from
rocprofv3 counters recorded separately (null when no counter run matches the
current kernel).  The cpu_baseline object times the float64 CPU oracle on a
bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

HERE = os.path.dirname(os.path.abspath(__file__))
if HERE not in sys.path:
    sys.path.insert(0, HERE)

METRIC = "KV-read HBM GB/s (% of 8 TB/s peak) + µs per layer decode step, B=8 S=1M GQA"

# HBM bytes per launch of the partial kernel measured with rocprofv3 counters
# (FETCH_SIZE and WRITE_SIZE, each scaled by the same counter on a plain 1 GiB
# copy), keyed by (workload, cache layout (paged: with its block length),
# kvp, query tokens, sha256 prefix of the kernel code the
# counters were taken on).  Changed kernel code no longer matches, and the
# bench then reports traffic as null.  Summaries are under profiles/.
TRAFFIC = {
    ("helix_fp8", "contiguous", 32, 1, "1d5f897ac7d074ca"): 17210454343,
    ("helix_fp8", "contiguous", 128, 1, "1d5f897ac7d074ca"): 17279497781,
    ("helix_fp8", "contiguous", 32, 4, "36a0b514422612bd"): 17248988135,
    ("helix_fp8", "contiguous", 32, 3, "36a0b514422612bd"): 17231752584,
    ("helix_fp8", "contiguous", 128, 4, "36a0b514422612bd"): 17452535621,
    ("helix_mxfp4", "contiguous", 32, 1, "1d5f897ac7d074ca"): 9157645548,
    ("helix_mxfp4", "contiguous", 128, 1, "1d5f897ac7d074ca"): 9228298482,
    ("gqa_bf16_varlen", "contiguous", 16, 1, "1d5f897ac7d074ca"): 3495787310,
    ("mla_bf16", "contiguous", 32, 1, "86eb417c08c25790"): 4905784948,
}
# Fraction of the partial kernel's SIMD cycles with the matrix cores busy,
# SQ_VALU_MFMA_BUSY_CYCLES / (1024 SIMDs x GRBM_GUI_ACTIVE / 8 XCDs), from a
# rocprofv3 --pmc run; same keys as TRAFFIC.
MFMA_BUSY = {
    ("mla_bf16", "contiguous", 32, 1, "86eb417c08c25790"): 0.4151,
    ("helix_mxfp4", "contiguous", 32, 1, "1d5f897ac7d074ca"): 0.2206,
    ("helix_fp8", "contiguous", 32, 1, "1d5f897ac7d074ca"): 0.1314,
    ("helix_fp8", "contiguous", 32, 4, "36a0b514422612bd"): 0.3408,
}
_GQA_SOURCES = ("partial_gqa_mfma.hip", "gqa_mfma_kernel.hpp", "partial_gqa_mfma_tokens.hip")
KERNEL_SOURCES = {"bf16": _GQA_SOURCES, "fp8": _GQA_SOURCES, "mxfp4": _GQA_SOURCES,
                  "fp8_tokens": ("partial_gqa_tokens32.hip", "partial_gqa_mfma.hip"),
                  "f32": ("partial_valu.hip",), "latent": ("partial_mla_mfma.hip",)}


def kernel_hash(fam):
    """sha256 prefix of the code of kernel family `fam` (a KERNEL_SOURCES key:
    its source files, the launcher that routes to it, and the shared device
    header), with // comments and blank space removed, so that comment edits
    keep the recorded counters."""
    import hashlib
    import re
    names = KERNEL_SOURCES[fam]
    h = hashlib.sha256()
    for f in names + ("kvd_device.hpp",):
        with open(os.path.join(HERE, "long_context_decode_split_amd", "csrc", f)) as fh:
            code = re.sub(r"//[^\n]*", "", fh.read())
        h.update(" ".join(code.split()).encode())
    return h.hexdigest()[:16]


def median(xs):
    ys = sorted(xs)
    n = len(ys)
    return ys[n // 2] if n % 2 else 0.5 * (ys[n // 2 - 1] + ys[n // 2])


def log(msg):
    print("[bench] " + msg, file=sys.stderr, flush=True)


def cpu_baseline(w, target_s=15.0):
    """Time the float64 oracle on whole (request, KV head) slabs until ~target_s
    of CPU work, and scale to KV GB/s."""
    import numpy as np

    import kvgen
    import oracle
    from long_context_decode_split_amd import roofline

    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # noqa: BLE001
        blas_threads = 1
    cores = len(os.sched_getaffinity(0))
    T = w.q_tokens
    q = kvgen.gen_q(w).reshape(w.B, T, w.Hq, w.Dqk)
    seq = kvgen.gen_seq_lens(w)
    p = oracle.Problem.from_workload(w)
    G = w.G
    done_bytes, elapsed, slabs = 0, 0.0, 0
    pairs = [(b, h) for b in range(w.B) for h in range(w.Hkv)]
    for (b, kvh) in pairs:
        kd, ks = kvgen.gen_kv_slab(w, "k", b, kvh)
        vd, vs = (None, None) if w.v_aliases_k else kvgen.gen_kv_slab(w, "v", b, kvh)
        L = int(seq[b])
        t0 = time.perf_counter()
        if w.kv_dtype == "mxfp4":
            k = oracle.dequant("mxfp4", kd[:L], ks[:L], w.Dqk)
            v = k[:, :w.Dv] if w.v_aliases_k else oracle.dequant("mxfp4", vd[:L], vs[:L], w.Dv)
        else:
            k = oracle.dequant(w.kv_dtype, kd[:L], ks, w.Dqk)
            v = k[:, :w.Dv] if w.v_aliases_k else oracle.dequant(w.kv_dtype, vd[:L], vs, w.Dv)
        for t in range(T):
            # query t sees the first L - T + 1 + t tokens (causal among new tokens)
            n = max(0, min(L, L - T + 1 + t))
            qf = oracle.q_to_f64(q[b, t, kvh * G:(kvh + 1) * G], w.q_dtype)
            oracle.attend(qf, k[:n], v[:n], p.sm_scale)
        elapsed += time.perf_counter() - t0
        done_bytes += roofline.kv_bytes(1, [L], w.Dqk, w.Dv, w.kv_dtype, w.v_aliases_k)
        slabs += 1
        del k, v
        if elapsed >= target_s:
            break
    return {"value": done_bytes / elapsed / 1e9, "unit": "GB/s", "cores": int(max(cores, blas_threads)),
            "blas_threads": int(blas_threads), "host_cpus": int(cores), "kind": "oracle",
            "sample": "%d of %d (request, KV head) slabs of %s, full length each, %d query token(s), "
                      "float64 dequant + attention, %.1f s" % (slabs, len(pairs), w.name, T, elapsed),
            "seconds": elapsed, "bytes": int(done_bytes)}


# How each kernel family computes, for the bench line (keyed by kv format;
# "latent" for the 576/512 latent-head kernel), and the arithmetic types of
# its products ("dtype").
ARITH = {
    "f32": "fp32 vector ALU: logits, softmax and P.V in fp32",
    "bf16": "bf16 MFMA logits (16x16x32) on the bf16 cache; P.V on bf16 MFMA with P as a bf16 hi+lo pair; "
            "fp32 accumulation and softmax",
    "fp8": "bf16 MFMA logits (16x16x32) on K decoded exactly from E4M3 (the fp32 slab scale folded into the "
           "log2 multiplier); V decoded exactly to fp16, P.V on fp16 MFMA with P = 2^(s - m + 7) rounded to "
           "fp16 and normalized by the sum of those fp16 weights (one more MFMA); fp32 accumulation, softmax "
           "and log-sum-exp",
    "fp8_tokens": "bf16 MFMA logits (32x32x16, the columns are (query token, head) pairs) on K decoded exactly "
                  "from E4M3 once for all tokens; V decoded exactly to fp16, P.V on fp16 MFMA (32x32x16) with "
                  "P = 2^(s - m + 7) rounded to fp16 and normalized by the sum of those fp16 weights; fp32 "
                  "accumulation, softmax and log-sum-exp",
    "mxfp4": "bf16 MFMA logits (16x16x32) on K decoded exactly from E2M1 with its E8M0 block exponents; V "
             "decoded exactly to fp16 with its block scales, P.V on fp16 MFMA with P = 2^(s - m + 7) rounded to "
             "fp16 and normalized by the sum of those fp16 weights (tiles whose V exponents leave fp16's range: "
             "bf16 V against P as a bf16 hi+lo pair); fp32 accumulation, softmax and log-sum-exp",
    "latent": "bf16 MFMA logits (32x32x16) over the 576-wide latent rows; P.V over their first 512 columns on "
              "fp16 MFMA (32x32x16) with V converted exactly from bf16 and P = 2^(s - m + 7) rounded to fp16, "
              "normalized by the sum of those fp16 weights; tiles staged through an LDS ring, the weights "
              "exchanged between the 4 waves through LDS; fp32 accumulation, softmax and log-sum-exp",
}
DTYPE = {"f32": "f32", "bf16": "bf16", "fp8": "bf16+fp16", "fp8_tokens": "bf16+fp16", "mxfp4": "bf16+fp16",
         "latent": "bf16+fp16"}
# Executed P.V flops per algorithmic ones on the latent kernel (one fp16
# product).
LATENT_PV_PASSES = 1

# Workloads measured next to the headline by a default run (the MXFP4 Helix
# shape and the latent-head shape, both at kvp = 32).
EXTRA = (("helix_mxfp4", 32), ("mla_bf16", 32))


def measure(args, name, kvp_req, T, layout, block_len, timing_extras=True):
    """One workload: generate it into device memory, time `args.steps` steps
    after `args.warmup`, and return the result fields (no cpu_baseline)."""
    import torch

    import kvgen
    from kvgen.device import generate_on_device
    from long_context_decode_split_amd import kvd, roofline

    w = kvgen.WORKLOADS[name].with_(q_tokens=T)
    kvp = kvp_req or (32 if 32 in w.kvp else w.kvp[0])
    torch.cuda.set_device(0)
    log("generating %s (kvp=%d) into device memory" % (w.name, kvp))
    t0 = time.time()
    dev = generate_on_device(w, progress=log)
    log("inputs ready in %.1f s" % (time.time() - t0))

    S_cache = w.S_max
    paging = {}
    if layout == "paged":
        bl = block_len
        if w.S_max % bl:
            raise SystemExit("S_max %d is not a multiple of block_len %d" % (w.S_max, bl))
        max_blocks = w.S_max // bl
        num_blocks = w.B * max_blocks
        def pool_view(t, per_row):
            if t is None or not per_row:
                return t
            return t.view((num_blocks, w.Hkv, bl) + tuple(t.shape[3:]))
        mx = w.kv_dtype == "mxfp4"
        dev.k = (pool_view(dev.k[0], True), pool_view(dev.k[1], mx))
        if dev.v is not None:
            dev.v = (pool_view(dev.v[0], True), pool_view(dev.v[1], mx))
        gen = torch.Generator().manual_seed(1234)
        table = torch.randperm(num_blocks, generator=gen).to(torch.int32).view(w.B, max_blocks).cuda()
        paging = dict(block_len=bl, max_blocks=max_blocks, num_blocks=num_blocks, block_table=table)
    elif layout != "contiguous":
        # the same generated bytes viewed as kvp shards of S/kvp rows each
        if w.S_max % kvp:
            raise SystemExit("S_max %d is not a multiple of kvp %d" % (w.S_max, kvp))
        S_cache = w.S_max // kvp
        def shard_view(t, per_row_scale):
            if t is None:
                return None
            if not per_row_scale:
                return t
            return t.view((kvp, w.B, w.Hkv, S_cache) + tuple(t.shape[3:]))
        mx = w.kv_dtype == "mxfp4"
        dev.k = (shard_view(dev.k[0], True), shard_view(dev.k[1], mx))
        if dev.v is not None:
            dev.v = (shard_view(dev.v[0], True), shard_view(dev.v[1], mx))
    p = kvd.problem(w.B, w.Hq, w.Hkv, w.Dqk, w.Dv, S_cache, kvp, w.q_dtype, w.kv_dtype, 0.0, w.v_aliases_k,
                    layout=layout, q_tokens=T, **paging)
    f32 = dict(dtype=torch.float32, device="cuda")
    o_part = torch.empty((kvp, w.B, T, w.Hq, w.Dv), **f32)
    lse_part = torch.empty((kvp, w.B, T, w.Hq), **f32)
    o = torch.empty((w.B, T, w.Hq, w.Dv), **f32)
    lse = torch.empty((w.B, T, w.Hq), **f32)
    rows = w.B * T * w.Hq
    stream = torch.cuda.Stream()
    seq = dev.seq_lens.cpu().numpy()
    kv_bytes = roofline.kv_bytes(w.Hkv, seq, w.Dqk, w.Dv, w.kv_dtype, w.v_aliases_k)
    flops = roofline.attention_flops_tokens(w.Hq, seq, T, w.Dqk, w.Dv)

    def step(ev0=None, ev1=None, ev2=None):
        if ev0 is not None:
            ev0.record(stream)
        kvd.kvd_decode_partial(p, dev.q, dev.k, dev.v, dev.seq_lens, o_part, lse_part, stream)
        if ev1 is not None:
            ev1.record(stream)
        kvd.kvd_lse_merge(kvp, rows, w.Dv, o_part, lse_part, o, lse, stream)
        if ev2 is not None:
            ev2.record(stream)

    with torch.cuda.stream(stream):
        for _ in range(args.warmup):
            step()
        torch.cuda.synchronize()
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        start.record(stream)
        for i in range(args.steps):
            step(*evs[i])
        end.record(stream)
        torch.cuda.synchronize()
    total_ms = start.elapsed_time(end)
    ms_per_step = total_ms / args.steps
    partial_ms = [e[0].elapsed_time(e[1]) for e in evs]
    merge_ms = [e[1].elapsed_time(e[2]) for e in evs]
    partial_avg = sum(partial_ms) / len(partial_ms)
    step_ms = [a_ + b_ for a_, b_ in zip(partial_ms, merge_ms)]
    assert torch.isfinite(o).all().item() and torch.isfinite(lse).all().item(), "non-finite output"
    log("%s kvp=%d T=%d: partial %.1f us, step %.1f us" % (w.name, kvp, T, partial_avg * 1e3, ms_per_step * 1e3))

    value = kv_bytes / (ms_per_step * 1e-3) / 1e9
    achieved = kv_bytes / (partial_avg * 1e-3) / 1e9
    peak = roofline.HBM_BYTES_PER_S / 1e9
    fam = "latent" if w.v_aliases_k else w.kv_dtype
    if fam == "fp8" and T in (3, 4) and w.Hq == 16 * w.Hkv and kvp * w.B * w.Hkv >= 1024:
        fam = "fp8_tokens"   # the one-wave kernel with the tokens as matrix-core columns
    khash = kernel_hash(fam)
    lay_key = layout + (str(block_len) if layout == "paged" else "")
    traffic = TRAFFIC.get((w.name, lay_key, kvp, T, khash))
    res = {
        "value": round(value, 2),
        "unit": "GB/s",
        "ms_per_step": round(ms_per_step, 5),
        "us_per_step": round(ms_per_step * 1e3, 2),
        "hbm_peak_frac": round(value / peak, 4),
        "dtype": DTYPE[fam],
        "arith": ARITH[fam],
        "config": {"workload": w.name, "layout": layout,
                   "block_len": block_len if layout == "paged" else None, "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv,
                   "Hsz": w.Dqk, "Dv": w.Dv, "S": w.S_max, "kvp": kvp, "q_tokens": T, "kv_dtype": w.kv_dtype,
                   "q_dtype": w.q_dtype, "kv_bytes": kv_bytes, "flops": flops},
        "partial_us": round(partial_avg * 1e3, 2),
        "partial_us_median": round(median(partial_ms) * 1e3, 2),
        "partial_us_min": round(min(partial_ms) * 1e3, 2),
        "merge_us": round(sum(merge_ms) / len(merge_ms) * 1e3, 2),
        "step_us_median": round(median(step_ms) * 1e3, 2),
        "step_us_min": round(min(step_ms) * 1e3, 2),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": peak, "unit": "GB/s",
                     "frac": round(achieved / peak, 4), "traffic": traffic,
                     "kernel": "kvd partial pass", "kernel_source_hash": khash,
                     "bytes_per_launch": kv_bytes,
                     "tflops": round(flops / (partial_avg * 1e-3) / 1e12, 2)},
    }
    # With several query tokens the same bytes feed T times the arithmetic:
    # the pass is bound by whichever ideal time is longer.
    fpeak = roofline.VALU_FP32_FLOPS if w.kv_dtype == "f32" else roofline.MFMA_BF16_FLOPS
    if flops / fpeak > kv_bytes / roofline.HBM_BYTES_PER_S:
        ach = flops / (partial_avg * 1e-3) / 1e12
        res["roofline"].update({"bound": "alu" if w.kv_dtype == "f32" else "mfma", "achieved": round(ach, 2),
                                "peak": fpeak / 1e12, "unit": "TFLOP/s", "frac": round(ach / (fpeak / 1e12), 4),
                                "flops_per_launch": flops, "hbm_frac": round(achieved / peak, 4)})
    if w.v_aliases_k:
        # latent heads run on bf16 MFMA: report the matrix-core share of the
        # partial pass, algorithmic and as executed
        executed = roofline.attention_flops_tokens(w.Hq, seq, T, w.Dqk, LATENT_PV_PASSES * w.Dv)
        t = partial_avg * 1e-3
        res["roofline"]["mfma"] = {
            "busy_frac_counter": MFMA_BUSY.get((w.name, lay_key, kvp, T, khash)),
            "peak_tflops": roofline.MFMA_BF16_FLOPS / 1e12,
            "algorithmic_tflops": round(flops / t / 1e12, 2),
            "algorithmic_frac": round(flops / t / roofline.MFMA_BF16_FLOPS, 4),
            "executed_tflops": round(executed / t / 1e12, 2),
            "executed_frac": round(executed / t / roofline.MFMA_BF16_FLOPS, 4),
            "executed_flops": executed}
    if timing_extras and not args.no_append:
        # one step's KV write: T new fp32 token rows per (request, KV head),
        # appended at the last T positions of every request
        kn = torch.randn((w.B, T, w.Hkv, w.Dqk), dtype=torch.float32, device="cuda")
        vn = None if w.v_aliases_k else torch.randn((w.B, T, w.Hkv, w.Dv), dtype=torch.float32, device="cuda")
        pos = torch.full((w.B,), w.S_max - T, dtype=torch.int32, device="cuda")
        app = []
        with torch.cuda.stream(stream):
            for i in range(args.warmup + args.steps):
                e = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
                e[0].record(stream)
                kvd.kvd_append_kv(p, kn, vn, pos, dev.k, dev.v, stream)
                e[1].record(stream)
                torch.cuda.synchronize()
                if i >= args.warmup:
                    app.append(e[0].elapsed_time(e[1]))
        res["append_us_median"] = round(median(app) * 1e3, 2)
    if timing_extras and args.graph:
        # The same step captured once and replayed: launch overhead leaves the
        # timed region (it matters for the small, latency-bound workloads).
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            step()
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            for _ in range(args.warmup):
                g.replay()
            torch.cuda.synchronize()
            gs, ge = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            gs.record(stream)
            for _ in range(args.steps):
                g.replay()
            ge.record(stream)
            torch.cuda.synchronize()
        g_ms = gs.elapsed_time(ge) / args.steps
        res["graph"] = {"us_per_step": round(g_ms * 1e3, 2), "value": round(kv_bytes / (g_ms * 1e-3) / 1e9, 2),
                        "unit": "GB/s", "note": "the step replayed from a HIP graph; 'value' above is eager"}
        del g
    if timing_extras and args.cold:
        # Each step starts after a 1 GiB write that evicts the cache from the
        # 256 MB last-level cache; only the step itself is inside the events.
        flush = torch.empty(1 << 28, dtype=torch.float32, device="cuda")
        cold_p, cold_s = [], []
        with torch.cuda.stream(stream):
            for i in range(args.steps):
                flush.fill_(float(i))
                e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
                step(*e)
                torch.cuda.synchronize()
                cold_p.append(e[0].elapsed_time(e[1]))
                cold_s.append(e[0].elapsed_time(e[2]))
        del flush
        res["cold"] = {"partial_us_median": round(median(cold_p) * 1e3, 2),
                       "step_us_median": round(median(cold_s) * 1e3, 2),
                       "step_us_min": round(min(cold_s) * 1e3, 2),
                       "value": round(kv_bytes / (median(cold_s) * 1e-3) / 1e9, 2), "unit": "GB/s",
                       "note": "each step after a 1 GiB flush write; 'value' and us_per_step above "
                               "are warm (back-to-back steps)"}
    del dev, o_part, lse_part, o, lse
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return w, res


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=50,
                    help="untimed steps first: the clocks settle over the first few dozen launches")
    ap.add_argument("--workload", default="helix_fp8")
    ap.add_argument("--kvp", type=int, default=None)
    ap.add_argument("--layout", default="contiguous", choices=["contiguous", "striped", "staggered16", "paged"],
                    help="cache layout; a sharded layout views the generated cache as kvp shards of "
                         "S/kvp rows, the paged layout as a pool of blocks handed to the requests in "
                         "a seeded random order (same bytes, same per-step traffic)")
    ap.add_argument("--block-len", type=int, default=16, help="tokens per block of the paged layout")
    ap.add_argument("--q-tokens", type=int, default=1,
                    help="query tokens per request (a multi-token turn, causal among the new tokens; "
                         "the cache's last T tokens are the new ones)")
    ap.add_argument("--no-append", action="store_true", help="skip timing kvd_append_kv")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true",
                    help="measure only the selected workload (a default run also measures the MXFP4 Helix "
                         "shape and the latent-head shape, reported under 'workloads')")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--graph", action="store_true",
                    help="also time the step (partial pass + merge) captured once into a HIP graph "
                         "and replayed; reported under 'graph'")
    ap.add_argument("--cold", action="store_true",
                    help="also time steps that each start with the last-level cache flushed "
                         "(for workloads whose cache fits in it); reported under 'cold'")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="only run a plain device-to-device copy of BYTES, 5 times (the "
                         "reference kernel for scaling HBM byte counters), and exit")
    args = ap.parse_args()

    if args.gpus != 1:
        print("bench.py measures one GPU's share of the split-KV path; the library runs on one GPU "
              "and has no multi-GPU path (--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch

    if args.copy_calibration:
        src = torch.ones(args.copy_calibration // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": args.copy_calibration, "launches": 5}))
        return

    T = args.q_tokens
    w, head = measure(args, args.workload, args.kvp, T, args.layout, args.block_len)
    res = {"metric": METRIC, "value": head["value"], "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": head["ms_per_step"], "us_per_step": head["us_per_step"],
           "hbm_peak_frac": head["hbm_peak_frac"], "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": head["dtype"], "arith": head["arith"],
           "data": "synthetic (seeded N(0,1), encoded to the cache format)"}
    res.update({k: v for k, v in head.items() if k not in res})
    default_run = (args.workload == "helix_fp8" and args.kvp in (None, 32) and T == 1
                   and args.layout == "contiguous")
    if default_run and not args.no_extra:
        res["workloads"] = {}
        for name, kvp in EXTRA:
            _, sub = measure(args, name, kvp, 1, "contiguous", args.block_len, timing_extras=False)
            res["workloads"][name] = sub
    if not args.no_cpu_baseline:
        log("timing the float64 oracle on a bounded sample")
        res["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
