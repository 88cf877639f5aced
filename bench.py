#!/usr/bin/env python3
"""Benchmark of the block-sparse video-DiT attention path on one MI355X.

Default workload: Wan-2.1-14B-shaped single-layer attention at 6x training
length (T = 126 latent frames of 30x52 tokens, N = 196560, 40 heads,
d = 128, bf16) with the LVSA frame mask (C = 21, W = 5, T_per = 8): the
largest of the workloads that fits one GPU. One step = one pass of
the path: build the LVSA mask for denoising step s (s advances every step)
and run the block-sparse attention over it. Inputs are seeded synthetic
tensors with the workload's shapes, resident in HBM before timing starts.

Prints ONE JSON line. value = effective TFLOP/s over the timed steps,
counting 4*d FLOP per visited (query, key) pair. The dense attention at the
same shape is timed beside it for the sparse-vs-dense speedup, and the CPU
oracle is timed on a bounded sample as a reported baseline.

  python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import dataclasses
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6  # MI355X dense bf16 MFMA: 256 CU x 2.4 GHz x 4096 FLOP/clk
PEAK_FP8_TFLOPS = 5033.2   # dense fp8 MFMA: twice the bf16 rate
PEAK_HBM_GBS = 8000.0
METRIC = "block-sparse attn ms/call + effective TFLOP/s (% bf16 MFMA peak), 1 MI355X"
ATTN_SRC = os.path.join(ROOT, "video_diffusion_transformer_lvsa_amd", "csrc", "attn_bf16.hip")
ATTN_FP8_SRC = os.path.join(ROOT, "video_diffusion_transformer_lvsa_amd", "csrc", "attn_fp8.hip")
ATTN_GRP_SRC = os.path.join(ROOT, "video_diffusion_transformer_lvsa_amd", "csrc", "attn_grp.hip")
# A bf16 LVSA call launches the full 128-row tiles of every frame
# (attn_bf16.hip) and then the short frame tails, four frames per workgroup
# (attn_grp.hip).
LVSA_SRCS = (ATTN_SRC, ATTN_GRP_SRC)
LVSA_KERNELS = ("bsa_fwd_d128_kernel<MODE_LIST, false, 8>", "bsa_fwd_d128_grp_kernel<MODE_TAIL, true>")
DRAFT_SRC = os.path.join(ROOT, "video_diffusion_transformer_lvsa_amd", "csrc", "draft.hip")

WORKLOAD_NAMES = {
    "wan1.3b-6x": "wan2.1-1.3b-6x-lvsa",
    "wan1.3b-1x": "wan2.1-1.3b-1x-lvsa-full",
    "wan14b-6x": "wan2.1-14b-6x-lvsa",
    "hunyuan-draft": "hunyuanvideo-draft-90pct",
    "hunyuan-lvsa-2x": "hunyuanvideo-2x-lvsa",
    "hunyuan-lvsa-1.5x": "hunyuanvideo-1.5x-lvsa",
}


def src_hash(*paths: str) -> str:
    """Hash of the code of one or more kernel sources (a record of a call that
    launches kernels from several files names them all): comments and
    whitespace removed, so a counter record stays valid across edits that
    change no code."""
    text = ""
    for path in paths:
        with open(path) as f:
            t = f.read()
        t = re.sub(r"/\*.*?\*/", " ", t, flags=re.S)
        t = re.sub(r"//[^\n]*", " ", t)
        text += re.sub(r"\s+", "", t)
    return hashlib.sha256(text.encode()).hexdigest()[:16]


def log(msg: str):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def lvsa_pairs(w, kv_cnt_host) -> int:
    """Visited (query, key) pairs of one LVSA call, all heads."""
    return int(w.heads) * w.P * w.P * int(kv_cnt_host.sum())


def _record(kind: str, workload: str, kernel_src):
    """A committed rocprofv3 summary (profiles/<kind>_<workload>.json) and a note
    of where it came from, if it was taken on the current kernel code; else
    (None, None). Its figures come from separate profiled runs, not this one."""
    rel = os.path.join("profiles", f"{kind}_{workload}.json")
    path = os.path.join(ROOT, rel)
    if not os.path.exists(path):
        return None, None
    with open(path) as f:
        t = json.load(f)
    srcs = (kernel_src,) if isinstance(kernel_src, str) else tuple(kernel_src)
    if t.get("kernel_code_sha256_16") != src_hash(*srcs):
        return None, None
    return t, {"file": rel, "kernel_code_sha256_16": t["kernel_code_sha256_16"],
               "measured": "separate rocprofv3 runs of the commands in the file, not this run"}


def traffic_for(workload: str, kernel_src):
    """(HBM bytes per launch, source) from the committed rocprofv3 --pmc summary."""
    t, src = _record("traffic", workload, kernel_src)
    return (None, None) if t is None else (t.get("hbm_bytes_per_launch"), src)


def oracle_threads() -> int:
    """Threads the oracle's BLAS uses (else the affinity count)."""
    try:
        from threadpoolctl import threadpool_info

        return max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # threadpoolctl missing: report the affinity count
        return len(os.sched_getaffinity(0))


def counters_for(workload: str, kernel_src):
    """(counter figures, source): clock, MFMA busy, L2 hit from the committed
    rocprofv3 summary, if it was taken on the current kernel code."""
    t, src = _record("counters", workload, kernel_src)
    if t is None:
        return None
    return dict(t.get("metrics", {}), source=src)


def median(xs):
    ys = sorted(xs)
    m = len(ys) // 2
    return ys[m] if len(ys) % 2 else 0.5 * (ys[m - 1] + ys[m])


def cpu_baseline_lvsa(w, q, k, v, budget_s: float):
    """Time the fp64 oracle on whole query frames of the workload until ~budget_s."""
    import numpy as np

    import oracle

    threads = oracle_threads()
    idx, cnt = oracle.lvsa_mask(w.T, w.C, w.window, w.T_per, 0)
    rng = np.random.default_rng(0)
    frames = rng.permutation(w.T)
    pairs = 0
    t0 = time.perf_counter()
    done = 0
    for f in frames:
        for h in range(w.heads):
            rows = np.arange(f * w.P, (f + 1) * w.P)
            oracle.block_sparse_attention(q, k, v, w.P, w.P, idx, cnt, rows=rows, heads=[h])
            pairs += w.P * int(cnt[f]) * w.P
            done += 1
            if time.perf_counter() - t0 > budget_s:
                break
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    flops = 4.0 * w.d * pairs
    return {
        "value": flops / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": f"{done} (head, query-frame) pairs of {w.P} rows x {w.C} frames of keys, LVSA s=0, fp64 numpy, "
                  f"{dt:.1f} s",
        "seconds": dt,
        "ms_per_call_extrapolated": dt / pairs * (lvsa_pairs(w, cnt)) * 1e3,
    }


def cpu_baseline_draft(w, q, k, v, sparsity: float, pool: str, budget_s: float):
    """Time the oracle on the Draft workload: the whole mask (pool, map, top-k)
    for one head, then fp64 attention on whole query blocks of that head in
    token order until ~budget_s."""
    import numpy as np

    import oracle
    from video_diffusion_transformer_lvsa_amd import synth

    threads = oracle_threads()
    g = oracle.draft_grid(w.T, w.H, w.W, w.pool_h, w.pool_w)
    perm, inv, bv = oracle.draft_permutation(g)
    h = 0
    t0 = time.perf_counter()
    kv, cnt, *_ = oracle.draft_mask(synth.bf16_to_f32(q[h : h + 1]), synth.bf16_to_f32(k[h : h + 1]), g, sparsity,
                                    pool=pool)
    mask_s = time.perf_counter() - t0
    rng = np.random.default_rng(0)
    blocks = rng.permutation(g.nb)
    pairs = 0
    done = 0
    t1 = time.perf_counter()
    for b in blocks:
        slots = perm[b * g.block_size : b * g.block_size + int(bv[b])]
        oracle.draft_attention_original_order(q[h : h + 1], k[h : h + 1], v[h : h + 1], perm, inv, bv, g.block_size,
                                              kv, cnt, rows=slots)
        pairs += int(bv[b]) * int(sum(int(bv[x]) for x in kv[0, b, : cnt[0, b]]))
        done += 1
        if time.perf_counter() - t1 > budget_s:
            break
    dt = time.perf_counter() - t1
    return {
        "value": 4.0 * w.d * pairs / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": f"attention on {done} query blocks of head 0 (valid pairs, fp64 numpy, {dt:.1f} s); the mask "
                  f"(pool, map, top-k) of one head timed separately",
        "mask_seconds_per_head": round(mask_s, 3),
        "seconds": dt + mask_s,
    }


def calibrate_copy(mib: int):
    """Plain copy of known size: token_permute with the identity map over a
    [1, rows, 128] bf16 tensor of `mib` MiB (reads and writes mib MiB)."""
    import torch

    from video_diffusion_transformer_lvsa_amd import _lib

    rows = mib * (1 << 20) // 256
    src = torch.ones((1, rows, 128), dtype=torch.bfloat16, device="cuda:0")
    dst = torch.empty_like(src)
    ident = torch.arange(rows, dtype=torch.int32, device="cuda:0")
    for _ in range(3):
        _lib.token_permute(src, ident, out=dst)
    torch.cuda.synchronize()
    log(f"copy calibration: {rows} rows x 256 B = {rows * 256} bytes read and written per launch")
    del src, dst, ident
    torch.cuda.empty_cache()


def run_lvsa(args, w):
    import numpy as np
    import torch

    from video_diffusion_transformer_lvsa_amd import _lib, synth

    own_budget = w.C == synth.WORKLOADS[w.name].C
    log(f"generating inputs for {w.name}")
    q, k, v = synth.video_qkv(w.seed, w.heads, w.T, w.H, w.W, w.d)
    dev = torch.device("cuda:0")

    def up(a):
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)

    dq, dk, dv = up(q), up(k), up(v)
    o = torch.empty((w.heads, w.N, w.d), dtype=torch.float32, device=dev)
    cap = max(_lib.lvsa_mask_capacity(w.T, w.C, w.window, w.T_per, s) for s in range(w.T_per))
    kv_idx = torch.empty((w.T, cap), dtype=torch.int32, device=dev)
    kv_cnt = torch.empty((w.T,), dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream()

    fp8 = bool(args.fp8)
    if fp8:
        # E4M3 codes (V transposed) and per-head scales, refreshed every step
        q8 = torch.empty((w.heads, w.N, w.d), dtype=torch.uint8, device=dev)
        k8 = torch.empty_like(q8)
        vt8 = torch.empty((w.heads, w.d, _lib.fp8_pitch(w.N)), dtype=torch.uint8, device=dev)
        sc = torch.empty((3, w.heads), dtype=torch.float32, device=dev)

    def quantize():
        _lib.quantize_fp8_e4m3(dq, out=q8, scales=sc[0])
        _lib.quantize_fp8_e4m3(dk, out=k8, scales=sc[1])
        _lib.quantize_fp8_e4m3(dv, transpose=True, out=vt8, scales=sc[2])

    def attn():
        if fp8:
            _lib.block_sparse_attn_fwd_fp8(q8, k8, vt8, sc[0], sc[1], sc[2], w.P, w.P, kv_idx, kv_cnt, out=o)
        else:
            _lib.block_sparse_attn_fwd(dq, dk, dv, w.P, w.P, kv_idx, kv_cnt, out=o)

    def dense():
        if fp8:
            _lib.dense_attn_fwd_fp8(q8, k8, vt8, sc[0], sc[1], sc[2], out=o)
        else:
            _lib.dense_attn_fwd(dq, dk, dv, out=o)

    def step(i):
        if fp8:
            quantize()
        _lib.lvsa_mask(w.T, w.C, w.window, w.T_per, i % w.T_per, cap=cap, kv_idx=kv_idx, kv_cnt=kv_cnt)
        attn()

    log("warmup")
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    pairs = []
    for s in range(w.T_per):
        _lib.lvsa_mask(w.T, w.C, w.window, w.T_per, s, cap=cap, kv_idx=kv_idx, kv_cnt=kv_cnt)
        pairs.append(lvsa_pairs(w, kv_cnt.cpu().numpy()))
    torch.cuda.synchronize()

    log(f"timing {args.steps} steps")
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    total_pairs = 0
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    qev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    for i in range(args.steps):
        s = (args.warmup + i) % w.T_per
        if fp8:
            qev[i][0].record(stream)
            quantize()
            qev[i][1].record(stream)
        _lib.lvsa_mask(w.T, w.C, w.window, w.T_per, s, cap=cap, kv_idx=kv_idx, kv_cnt=kv_cnt)
        ev[i][0].record(stream)
        attn()
        ev[i][1].record(stream)
        total_pairs += pairs[s]
    t1.record(stream)
    torch.cuda.synchronize()
    ms_total = t0.elapsed_time(t1)
    attn_ms = [a.elapsed_time(b) for a, b in ev]
    ms_per_step = ms_total / args.steps
    flops_total = 4.0 * w.d * total_pairs
    value = flops_total / (ms_total * 1e-3) / 1e12
    attn_avg = sum(attn_ms) / len(attn_ms)
    flop_per_launch = flops_total / args.steps
    achieved = flop_per_launch / (attn_avg * 1e-3) / 1e12
    quant_ms = sum(a.elapsed_time(b) for a, b in qev) / args.steps if fp8 else 0.0
    mask_ms = ms_per_step - attn_avg - quant_ms
    peak = PEAK_FP8_TFLOPS if fp8 else PEAK_BF16_TFLOPS

    res = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8-e4m3" if fp8 else "bf16",
        "data": "synthetic",
        "config": {
            "workload": WORKLOAD_NAMES[w.name] + ("" if own_budget else f"-C{w.C}") + ("-fp8" if fp8 else ""),
            "T": w.T, "H": w.H, "W": w.W, "tokens": w.N, "heads": w.heads, "d": w.d,
            "C": w.C, "window": w.window, "T_per": w.T_per, "steps_s": "s = step mod T_per",
            "flop_per_call": flop_per_launch,
        },
        "attn_ms_per_call": round(attn_avg, 4),
        "attn_ms_median": round(median(attn_ms), 4),
        "attn_ms_min": round(min(attn_ms), 4),
        "mask_build_ms": round(max(mask_ms, 0.0), 4),
        "pct_bf16_peak": round(100.0 * achieved / PEAK_BF16_TFLOPS, 2),
    }
    if fp8:
        res["quantize_ms"] = round(quant_ms, 4)
        res["pct_fp8_peak"] = round(100.0 * achieved / PEAK_FP8_TFLOPS, 2)
    # the counter records were taken at the workload's own frame budget
    traffic, tsrc = traffic_for(w.name + ("-fp8" if fp8 else ""), ATTN_FP8_SRC if fp8 else LVSA_SRCS) \
        if own_budget else (None, None)
    res["roofline"] = {
        "bound": "mfma",
        "achieved": round(achieved, 2),
        "peak": peak,
        "unit": "TFLOP/s",
        "frac": round(achieved / peak, 4),
        "traffic": traffic,
        "kernel": "bsa_fwd_fp8_kernel<MODE_LIST, 4>" if fp8 else LVSA_KERNELS[0],
    }
    if not fp8:
        # achieved and traffic are per call: both launches of the call
        res["roofline"]["launches_per_call"] = list(LVSA_KERNELS)
    if tsrc is not None:
        res["roofline"]["traffic_source"] = tsrc
    ctr = counters_for(w.name + ("-fp8" if fp8 else ""), ATTN_FP8_SRC if fp8 else LVSA_SRCS) if own_budget else None
    if ctr is not None:
        res["counters"] = ctr

    if not args.no_dense:
        log("timing dense attention at the same shape")
        dense()
        torch.cuda.synchronize()
        d0 = torch.cuda.Event(enable_timing=True)
        d1 = torch.cuda.Event(enable_timing=True)
        nd = args.dense_steps
        d0.record(stream)
        for _ in range(nd):
            dense()
        d1.record(stream)
        torch.cuda.synchronize()
        dense_ms = d0.elapsed_time(d1) / nd
        dense_flops = 4.0 * w.d * w.heads * float(w.N) * w.N
        res["dense_ms_per_call"] = round(dense_ms, 3)
        res["dense_tflops"] = round(dense_flops / (dense_ms * 1e-3) / 1e12, 2)
        res["speedup_vs_dense"] = round(dense_ms / attn_avg, 3)
        res["dense_dtype"] = "fp8-e4m3" if fp8 else "bf16"

    if not args.no_cpu_baseline:
        log(f"timing the CPU oracle for ~{args.cpu_seconds} s")
        res["cpu_baseline"] = cpu_baseline_lvsa(w, q, k, v, args.cpu_seconds)
    return res


def run_draft(args, w):
    import numpy as np
    import torch

    from video_diffusion_transformer_lvsa_amd import _lib, synth

    log(f"generating inputs for {w.name}")
    q, k, v = synth.video_qkv(w.seed, w.heads, w.T, w.H, w.W, w.d)
    dev = torch.device("cuda:0")

    def up(a):
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)

    dq, dk, dv = up(q), up(k), up(v)
    bs = w.pool_h * w.pool_w
    stream = torch.cuda.current_stream()
    sparsity = w.sparsity if args.sparsity is None else args.sparsity
    pool = args.pool

    reorder = not args.no_reorder
    fp8 = bool(args.fp8)
    o_raster = None if reorder else torch.empty((w.heads, w.N, w.d), dtype=torch.float32, device=dev)
    f8 = {}

    def mask():
        return _lib.draft_mask_and_perm(dq, dk, dv, w.T, w.H, w.W, w.pool_h, w.pool_w, sparsity, pool=pool,
                                        reorder=reorder)

    def quantize(out):
        # E4M3 codes of the tensors the attention reads (reordered or raster)
        src = (out["q_perm"], out["k_perm"], out["v_perm"]) if reorder else (dq, dk, dv)
        n = src[0].shape[1]
        if not f8:
            f8["q8"] = torch.empty((w.heads, n, w.d), dtype=torch.uint8, device=dev)
            f8["k8"] = torch.empty_like(f8["q8"])
            f8["vt8"] = torch.empty((w.heads, w.d, _lib.fp8_pitch(n)), dtype=torch.uint8, device=dev)
            f8["sc"] = torch.empty((3, w.heads), dtype=torch.float32, device=dev)
        _lib.quantize_fp8_e4m3(src[0], out=f8["q8"], scales=f8["sc"][0])
        _lib.quantize_fp8_e4m3(src[1], out=f8["k8"], scales=f8["sc"][1])
        _lib.quantize_fp8_e4m3(src[2], transpose=True, out=f8["vt8"], scales=f8["sc"][2])

    def attn(out):
        if fp8:
            c = (f8["q8"], f8["k8"], f8["vt8"], f8["sc"][0], f8["sc"][1], f8["sc"][2])
            if reorder:
                return _lib.block_sparse_attn_fwd_fp8(*c, bs, bs, out["kv_idx"], out["kv_cnt"], mask_heads=w.heads,
                                                      block_valid=out["block_valid"])
            return _lib.draft_attn_fwd_fp8(*c, w.T, w.H, w.W, w.pool_h, w.pool_w, out["kv_idx"], out["kv_cnt"],
                                           out=o_raster)
        if reorder:
            return _lib.block_sparse_attn_fwd(out["q_perm"], out["k_perm"], out["v_perm"], bs, bs, out["kv_idx"],
                                              out["kv_cnt"], mask_heads=w.heads, block_valid=out["block_valid"])
        return _lib.draft_attn_fwd(dq, dk, dv, w.T, w.H, w.W, w.pool_h, w.pool_w, out["kv_idx"], out["kv_cnt"],
                                   out=o_raster)

    def step():
        out = mask()
        if fp8:
            quantize(out)
        op = attn(out)
        o = _lib.token_permute(op, out["inv_perm"]) if reorder else op
        return out, op, o

    for _ in range(args.warmup):
        out, op, o = step()
    torch.cuda.synchronize()
    kv = out["kv_idx"].cpu().numpy()
    bv = out["block_valid"].cpu().numpy().astype(np.int64)
    pairs = int(sum((bv * bv[kv[h]].sum(axis=1)).sum() for h in range(w.heads)))
    cnt_all = out["kv_cnt"].cpu().numpy().astype(np.int64)
    flops_area = 4.0 * w.d * bs * bs * float(cnt_all.sum())
    e = [torch.cuda.Event(enable_timing=True) for _ in range(5)]
    times = {"mask": [], "attn": [], "scatter": []}
    if fp8:
        times["quantize"] = []
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for _ in range(args.steps):
        e[0].record(stream)
        out = mask()
        e[1].record(stream)
        if fp8:
            quantize(out)
        e[4].record(stream)
        op = attn(out)
        e[2].record(stream)
        if reorder:
            _lib.token_permute(op, out["inv_perm"])
        e[3].record(stream)
        torch.cuda.synchronize()
        times["mask"].append(e[0].elapsed_time(e[1]))
        if fp8:
            times["quantize"].append(e[1].elapsed_time(e[4]))
        times["attn"].append(e[4].elapsed_time(e[2]))
        times["scatter"].append(e[2].elapsed_time(e[3]))
    t1.record(stream)
    torch.cuda.synchronize()
    ms_total = t0.elapsed_time(t1)
    attn_avg = sum(times["attn"]) / len(times["attn"])
    attn_med = median(times["attn"])
    flops = 4.0 * w.d * pairs
    res = {
        "metric": METRIC,
        "value": round(flops * args.steps / (ms_total * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_total / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8-e4m3" if fp8 else "bf16",
        "data": "synthetic",
        "config": {"workload": f"hunyuanvideo-draft-{round(100 * sparsity)}pct" + ("-maxpool" if pool == "max" else "")
                               + ("" if reorder else "-raster") + ("-fp8" if fp8 else ""),
                   "T": w.T, "H": w.H, "W": w.W, "heads": w.heads, "d": w.d, "pool": [w.pool_h, w.pool_w],
                   "pooling": pool, "sparsity": sparsity, "top_k": int(kv.shape[-1]), "flop_per_call": flops,
                   "flop_block_area_per_call": flops_area},
        "stage_ms": {k2: round(sum(v2) / len(v2), 4) for k2, v2 in times.items()},
        "attn_ms_median": round(attn_med, 4),
        "roofline": {"bound": "mfma", "achieved": round(flops / (attn_avg * 1e-3) / 1e12, 2),
                     "peak": PEAK_FP8_TFLOPS if fp8 else PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(flops / (attn_avg * 1e-3) / 1e12 / (PEAK_FP8_TFLOPS if fp8 else PEAK_BF16_TFLOPS), 4),
                     "traffic": None,
                     "kernel": ("bsa_fwd_fp8_kernel<MODE_LIST, 4>" if reorder else "bsa_fwd_fp8_kernel<MODE_T2D, 4>")
                     if fp8 else ("bsa_fwd_d128_grp_kernel<MODE_GRP, true>" if reorder
                                  else "bsa_fwd_d128_grp_kernel<MODE_T2DG, false>")},
    }
    # the counter records were taken at the workload's own sparsity with mean
    # pooling, one record per path; other settings move other bytes
    if sparsity == w.sparsity and pool == "mean":
        key = w.name + ("" if reorder else "-raster") + ("-fp8" if fp8 else "")
        traffic, tsrc = traffic_for(key, ATTN_FP8_SRC if fp8 else ATTN_GRP_SRC)
        res["roofline"]["traffic"] = traffic
        if tsrc is not None:
            res["roofline"]["traffic_source"] = tsrc
        ctr = counters_for(key, ATTN_FP8_SRC if fp8 else ATTN_GRP_SRC)
        if ctr is not None:
            res["counters"] = ctr
    if not args.no_dense:
        # dense attention over the unpadded raster tokens at the same shape
        # and arithmetic (FP8 codes of the raster tensors for an FP8 line)
        log("timing dense attention at the same shape")
        od = torch.empty((w.heads, w.N, w.d), dtype=torch.float32, device=dev)
        if fp8:
            c8 = _lib.quantize_qkv_fp8(dq, dk, dv)

            def dense():
                _lib.dense_attn_fwd_fp8(c8["q8"], c8["k8"], c8["vt8"], c8["q_scale"], c8["k_scale"], c8["v_scale"],
                                        out=od)
        else:
            def dense():
                _lib.dense_attn_fwd(dq, dk, dv, out=od)
        dense()
        torch.cuda.synchronize()
        d0 = torch.cuda.Event(enable_timing=True)
        d1 = torch.cuda.Event(enable_timing=True)
        d0.record(stream)
        for _ in range(args.dense_steps):
            dense()
        d1.record(stream)
        torch.cuda.synchronize()
        dense_ms = d0.elapsed_time(d1) / args.dense_steps
        res["dense_ms_per_call"] = round(dense_ms, 3)
        res["dense_tflops"] = round(4.0 * w.d * w.heads * float(w.N) * w.N / (dense_ms * 1e-3) / 1e12, 2)
        res["speedup_vs_dense"] = round(dense_ms / attn_avg, 3)
        res["speedup_vs_dense_pipeline"] = round(dense_ms / (ms_total / args.steps), 3)
        res["dense_dtype"] = "fp8-e4m3" if fp8 else "bf16"
        del od
    if not args.no_cpu_baseline:
        log(f"timing the CPU oracle for ~{args.cpu_seconds} s")
        res["cpu_baseline"] = cpu_baseline_draft(w, q, k, v, sparsity, pool, args.cpu_seconds)
    return res


# ---------------------------------------------------------------------------
# Summaries of rocprofv3 output (run on the host after the profiled runs):
#   python3 bench.py --summarize traffic --workload W [--fp8] --fetch DIR --write DIR [--calib-copy-mb 1024]
#   python3 bench.py --summarize counters --workload W [--fp8] --passes DIR DIR
#   python3 bench.py --summarize trace --trace DIR --title T --cmd C --out FILE.md
# traffic/counters write profiles/traffic_<key>.json / profiles/counters_<key>.json
# with the code hash of the kernel source they were taken on.
# ---------------------------------------------------------------------------
def _csv_in(d: str, suffix: str):
    import csv

    for dirpath, _, files in os.walk(d):
        for f in sorted(files):
            if f.endswith(suffix):
                with open(os.path.join(dirpath, f)) as fh:
                    return list(csv.DictReader(fh))
    raise FileNotFoundError(f"no *{suffix} under {d}")


def _kernel_key(name: str) -> str:
    for a in ("void ", "lvsa::(anonymous namespace)::", "lvsa::"):
        name = name.replace(a, "")
    return name.split("(")[0]


def _per_kernel(rows, counter: str):
    """{kernel: [value per dispatch]} for one counter."""
    out = {}
    for r in rows:
        if r["Counter_Name"] == counter and "lvsa::" in r["Kernel_Name"]:
            out.setdefault(_kernel_key(r["Kernel_Name"]), []).append(float(r["Counter_Value"]))
    return out


def _profiled_kernel(workload: str, fp8: bool, raster: bool = False):
    """(sources, kernel key in traces, label, traffic/counter key, algorithmic
    bytes per call, keys of the call's other launches)."""
    from video_diffusion_transformer_lvsa_amd import synth

    w = synth.WORKLOADS[workload]
    if w.kind == "draft" and not raster:
        nb = w.T * (-(-w.H // w.pool_h)) * (-(-w.W // w.pool_w))
        n = nb * w.pool_h * w.pool_w
    else:
        n = w.N
    elem = 1 if fp8 else 2
    alg = 3 * w.heads * n * w.d * elem + w.heads * n * w.d * 4
    key = w.name + ("-raster" if raster else "") + ("-fp8" if fp8 else "")
    if fp8:
        mode = ("3", "MODE_T2D") if raster else ("1", "MODE_LIST")
        return (ATTN_FP8_SRC,), f"bsa_fwd_fp8_kernel<{mode[0]}, 4>", f"bsa_fwd_fp8_kernel<{mode[1]}, 4>", key, alg, ()
    if w.kind == "draft":
        tmpl, label = (("bsa_fwd_d128_grp_kernel<5, false>", "bsa_fwd_d128_grp_kernel<MODE_T2DG, false>") if raster
                       else ("bsa_fwd_d128_grp_kernel<4, true>", "bsa_fwd_d128_grp_kernel<MODE_GRP, true>"))
        return (ATTN_GRP_SRC,), tmpl, label, key, alg, ()
    return LVSA_SRCS, "bsa_fwd_d128_kernel<1, false, 8>", LVSA_KERNELS[0], key, alg, ("bsa_fwd_d128_grp_kernel<6, true>",)


def summarize(argv) -> int:
    sp = argparse.ArgumentParser(prog="bench.py --summarize")
    sp.add_argument("what", choices=("traffic", "counters", "trace"))
    sp.add_argument("--workload", default="wan14b-6x")
    sp.add_argument("--fp8", action="store_true")
    sp.add_argument("--no-reorder", action="store_true", help="Draft: records of the raster path")
    sp.add_argument("--fetch")
    sp.add_argument("--write")
    sp.add_argument("--calib-copy-mb", type=int, default=1024)
    sp.add_argument("--passes", nargs="+")
    sp.add_argument("--trace")
    sp.add_argument("--title")
    sp.add_argument("--cmd", action="append", default=[])
    sp.add_argument("--note", action="append", default=[])
    sp.add_argument("--out")
    a = sp.parse_args(argv)
    if a.what == "trace":
        rows = _csv_in(a.trace, "kernel_stats.csv")
        lines = [f"# {a.title}", "", "Command (on one MI355X, from the repository root):", "", "```", *a.cmd, "```", "",
                 "| kernel | calls | avg ms | min ms | max ms | % time |", "|---|---|---|---|---|---|"]
        for r in rows[:10]:
            lines.append(f"| `{_kernel_key(r['Name'])}` | {r['Calls']} | {float(r['AverageNs']) / 1e6:.4f} | "
                         f"{float(r['MinNs']) / 1e6:.4f} | {float(r['MaxNs']) / 1e6:.4f} | "
                         f"{float(r['Percentage']):.2f} |")
        lines += ["", *a.note] if a.note else []
        with open(a.out, "w") as f:
            f.write("\n".join(lines) + "\n")
        return 0
    src, key, label, tkey, alg, extra = _profiled_kernel(a.workload, a.fp8, a.no_reorder)
    if a.what == "traffic":
        fr, wr = _per_kernel(_csv_in(a.fetch, "counter_collection.csv"), "FETCH_SIZE"), \
            _per_kernel(_csv_in(a.write, "counter_collection.csv"), "WRITE_SIZE")
        rows = a.calib_copy_mb * (1 << 20) // 256
        known_r, known_w = (rows * 256 + rows * 4) / 1024, rows * 256 / 1024
        cal = "token_permute_kernel"
        # the first three copy launches are the calibration (identity map over a known size)
        cf = sum(fr[cal][:3]) / 3
        cw = sum(wr[cal][:3]) / 3
        ff, fw = known_r / cf, known_w / cw
        mean = lambda v: sum(v) / len(v)
        calls = (key,) + tuple(e for e in extra if e in fr and e in wr)
        t = {"kernel": label, "workload": WORKLOAD_NAMES[a.workload] + ("-raster" if a.no_reorder else "")
             + ("-fp8" if a.fp8 else ""),
             "kernel_code_sha256_16": src_hash(*src),
             "fetch_size_kib_raw": mean(fr[key]), "write_size_kib_raw": mean(wr[key]),
             "copy_calibration": {"kernel": f"token_permute_kernel (identity map, {a.calib_copy_mb} MiB)",
                                  "read_kib_known": known_r, "fetch_size_kib": cf, "write_kib_known": known_w,
                                  "write_size_kib": cw, "fetch_factor": ff, "write_factor": fw},
             # per call: the dominant kernel plus the call's other launches
             "hbm_fetch_bytes_per_launch": sum(mean(fr[k]) for k in calls) * ff * 1024,
             "hbm_write_bytes_per_launch": sum(mean(wr[k]) for k in calls) * fw * 1024,
             "algorithmic_bytes_per_launch": alg,
             "note": "FETCH_SIZE counts L2 misses, served by MALL or HBM",
             "other_kernels_bytes_per_launch": {
                 k: {"read": mean(fr[k] if k != cal else fr[k][3:] or fr[k]) * ff * 1024,
                     "write": mean(wr[k] if k != cal else wr[k][3:] or wr[k]) * fw * 1024}
                 for k in sorted(set(fr) & set(wr)) if k not in calls and (k != cal or len(fr[k]) > 3)},
             "commands": a.cmd}
        if len(calls) > 1:
            t["launches_per_call"] = {k: {"read": mean(fr[k]) * ff * 1024, "write": mean(wr[k]) * fw * 1024}
                                      for k in calls}
        t["hbm_bytes_per_launch"] = t["hbm_fetch_bytes_per_launch"] + t["hbm_write_bytes_per_launch"]
        out = a.out or os.path.join(ROOT, "profiles", f"traffic_{tkey}.json")
    else:
        def metrics(kname):
            got = {}
            for d in a.passes:
                rows = _csv_in(d, "counter_collection.csv")
                for r in rows:
                    if _kernel_key(r["Kernel_Name"]) != kname:
                        continue
                    did = (d, r["Dispatch_Id"])
                    e = got.setdefault(r["Counter_Name"], {})
                    e[did] = float(r["Counter_Value"])
                    got.setdefault("_dur", {})[did] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-9
            if not got:
                return None
            m = {c: sum(v.values()) / len(v) for c, v in got.items()}
            xcd, simds = 8, 1024
            clk = m["GRBM_GUI_ACTIVE"] / xcd / m["_dur"]
            cyc = m["GRBM_GUI_ACTIVE"] / xcd
            mops = "SQ_INSTS_VALU_MFMA_MOPS_F8" if a.fp8 else "SQ_INSTS_VALU_MFMA_MOPS_BF16"
            met = {"duration_ms_under_counters": round(m["_dur"] * 1e3, 2), "shader_clock_ghz": round(clk / 1e9, 3)}
            if "SQ_VALU_MFMA_BUSY_CYCLES" in m:
                met["mfma_busy_frac"] = round(m["SQ_VALU_MFMA_BUSY_CYCLES"] / simds / cyc, 4)
            if mops in m:
                met["matrix_core_flop_per_launch"] = m[mops] * 512
            if "SQ_INSTS_MFMA" in m:
                met["mfma_insts_per_launch"] = m["SQ_INSTS_MFMA"]
                if "SQ_INSTS_VALU" in m:
                    met["other_valu_per_mfma"] = round((m["SQ_INSTS_VALU"] - m["SQ_INSTS_MFMA"]) / m["SQ_INSTS_MFMA"], 3)
            if "SQ_WAIT_INST_ANY" in m and "SQ_WAVE_CYCLES" in m:
                met["dependency_wait_frac"] = round(m["SQ_WAIT_INST_ANY"] / m["SQ_WAVE_CYCLES"], 4)
            if "SQ_VALU_MFMA_COEXEC_CYCLES" in m:
                met["valu_mfma_coexec_frac"] = round(m["SQ_VALU_MFMA_COEXEC_CYCLES"] / simds / cyc, 4)
            if "TCC_HIT_sum" in m and "TCC_MISS_sum" in m:
                met["l2_hit_rate"] = round(m["TCC_HIT_sum"] / (m["TCC_HIT_sum"] + m["TCC_MISS_sum"]), 4)
            if "SQ_LDS_BANK_CONFLICT" in m:
                met["lds_bank_conflicts"] = m["SQ_LDS_BANK_CONFLICT"]
            if "SQ_INSTS_LDS" in m:
                met["lds_insts_per_launch"] = m["SQ_INSTS_LDS"]
            return met

        met = metrics(key)
        mops = "SQ_INSTS_VALU_MFMA_MOPS_F8" if a.fp8 else "SQ_INSTS_VALU_MFMA_MOPS_BF16"
        t = {"kernel": label, "workload": WORKLOAD_NAMES[a.workload] + ("-raster" if a.no_reorder else "")
             + ("-fp8" if a.fp8 else ""),
             "kernel_code_sha256_16": src_hash(*src), "metrics": met,
             "derivation": {"shader_clock_ghz": "GRBM_GUI_ACTIVE / 8 XCDs / dispatch duration",
                            "mfma_busy_frac": "SQ_VALU_MFMA_BUSY_CYCLES / 1024 SIMDs / (GRBM_GUI_ACTIVE / 8)",
                            "matrix_core_flop_per_launch": mops + " x 512",
                            "other_valu_per_mfma": "(SQ_INSTS_VALU - SQ_INSTS_MFMA) / SQ_INSTS_MFMA",
                            "dependency_wait_frac": "SQ_WAIT_INST_ANY / SQ_WAVE_CYCLES",
                            "valu_mfma_coexec_frac": "SQ_VALU_MFMA_COEXEC_CYCLES / 1024 / (GRBM_GUI_ACTIVE / 8)",
                            "l2_hit_rate": "TCC_HIT_sum / (TCC_HIT_sum + TCC_MISS_sum)"},
             "commands": a.cmd}
        others = {e: metrics(e) for e in extra}
        others = {e: v for e, v in others.items() if v is not None}
        if others:
            t["other_launches_per_call"] = others
        out = a.out or os.path.join(ROOT, "profiles", f"counters_{tkey}.json")
    with open(out, "w") as f:
        json.dump(t, f, indent=1)
        f.write("\n")
    print(f"wrote {out}")
    return 0


def main(argv=None) -> int:
    argv = sys.argv[1:] if argv is None else argv
    if argv and argv[0] == "--summarize":
        return summarize(argv[1:])
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=16)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="wan14b-6x", choices=sorted(WORKLOAD_NAMES))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-dense", action="store_true")
    ap.add_argument("--sparsity", type=float, default=None, help="Draft workload: override the 90%% sparsity")
    ap.add_argument("--budget", type=int, default=None, help="LVSA workloads: override the frame budget C")
    ap.add_argument("--pool", choices=("mean", "max"), default="mean", help="Draft workload: pooling of Q and K")
    ap.add_argument("--no-reorder", action="store_true",
                    help="Draft workload: attend on the raster layout (draft_attn_fwd) instead of reordering")
    ap.add_argument("--dense-steps", type=int, default=3)
    ap.add_argument("--fp8", action="store_true",
                    help="quantize Q, K, V (Draft: the tensors the attention reads) to E4M3 each step and run the "
                         "FP8 attention")
    ap.add_argument("--calib-copy-mb", type=int, default=0,
                    help="first run a plain row copy (token_permute, identity map) over this many MiB, 3 times, "
                         "so HBM counters can be scaled by a kernel of known traffic")
    args = ap.parse_args(argv)

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path (attention shards by heads with "
              "no exchange; see the design notes). Run with --gpus 1.", file=sys.stderr)
        return 2

    from video_diffusion_transformer_lvsa_amd import synth

    w = synth.WORKLOADS[args.workload]
    if args.budget is not None:
        if w.kind != "lvsa" or args.budget < 1:
            print("--budget takes a frame count >= 1 and applies to the LVSA workloads only", file=sys.stderr)
            return 2
        w = dataclasses.replace(w, C=args.budget)

    import torch

    from video_diffusion_transformer_lvsa_amd import _lib

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    _lib.load()
    if args.calib_copy_mb > 0:
        calibrate_copy(args.calib_copy_mb)
    res = run_draft(args, w) if w.kind == "draft" else run_lvsa(args, w)
    print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
