#!/usr/bin/env python3
"""Benchmark of the batch-invariant paged attention path on one MI355X.

One step = one pass of the whole path over one batch of synthetic input: the page update of
the step's new tokens, then attention (a decode step is `bi_attn_decode_append`, whose split
kernel also writes the new tokens into their pages, then the combine). The headline workload is the bf16 decode sweep at its
largest batch (64 sequences, 32 query heads, 4 KV heads, head_dim 128, context lengths
U[128, 8192], 16-token pages in a shuffled pool, fixed split size 256); ``value`` is its
algorithmic HBM GB/s. The chunked-prefill workload (16 sequences, 64/4 heads, cached prefix
U[0, 16384], new chunk U[1, 2048]) is measured in the same run and reported under
``prefill`` in TFLOP/s, the long-context decode (8 x 131072 tokens, q x 4) under
``long_decode`` and the 64-step mixed continuous-batching trace under ``mixed_trace``.
Times are reported as medians with p10/p90 beside the whole-run averages. Every figure counts
only because the same run checks bitwise batch invariance first and, in the host leg, parity
against the fp64 oracle (the headline decode rows, sampled prefill and long-context rows).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--no-prefill]
                       [--no-long] [--no-trace]
       (profiling: --profile-run, --prefill-only, --long-only, --next-rows-only, --copy-calib-mb)
"""

from __future__ import annotations

import argparse
import json
import math
import os
import platform
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import invariant_attention_amd as bi  # noqa: E402
from synth import CONFIG_SHAPES, SeqSpec, build_batch  # noqa: E402

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0    # MI355X dense bf16 MFMA, published
METRIC = "decode attn HBM GB/s + prefill attn TFLOP/s at bitwise batch invariance"


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


KERNEL_SOURCES = ("invariant_attention_amd/csrc/bi_attn.hip", "invariant_attention_amd/csrc/core.hpp",
                  "include/bi_attn.h")
NORM_SOURCES = ("invariant_attention_amd/csrc/bi_norm.hip", "include/bi_norm.h")
GEMM_SOURCES = ("invariant_attention_amd/csrc/bi_gemm.hip", "include/bi_gemm.h")


def kernel_sha256(sources=KERNEL_SOURCES):
    import hashlib
    h = hashlib.sha256()
    for rel in sources:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def profiled_traffic(kernel, sources=KERNEL_SOURCES):
    """HBM bytes per launch from the committed rocprofv3 counter summaries, if they were taken
    on the kernel sources as they are now (else None)."""
    import glob
    import re
    sha = kernel_sha256(sources)
    for path in sorted(glob.glob(os.path.join(ROOT, "profiles", "*.md"))):
        for m in re.finditer(r"<!-- traffic: (\{.*?\}) -->", open(path).read()):
            rec = json.loads(m.group(1))
            if rec.get("kernel_sha256") == sha and kernel in rec:
                return rec[kernel]
    return None


def dev(x, dt):
    return torch.from_numpy(np.ascontiguousarray(x)).cuda().to(dt)


def cfg_of(shape, policy=bi.BI_SPLIT_FIXED):
    return bi.AttnConfig(shape.num_q_heads, shape.num_kv_heads, shape.head_dim, shape.page_size,
                         shape.split_size, bi.BI_BF16, 0.0, policy)


def stats_ms(samples):
    """median / p10 / p90 / mean of per-iteration times, in microseconds."""
    a = np.asarray(samples, np.float64) * 1e3
    return {"median_us": float(np.median(a)), "p10_us": float(np.percentile(a, 10)),
            "p90_us": float(np.percentile(a, 90)), "mean_us": float(a.mean()), "n": int(a.size)}


def host_cpu():
    """CPU model and thread counts of the host (for the oracle's timing)."""
    model = platform.processor() or platform.machine()
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return model


class Timer:
    """HIP events on torch's current stream (the stream every call below is launched on)."""

    def __init__(self, n):
        self.ev = [torch.cuda.Event(enable_timing=True) for _ in range(n)]

    def mark(self, i):
        self.ev[i].record()

    def ms(self, i, j):
        return self.ev[i].elapsed_time(self.ev[j])


# ----------------------------------------------------------------------------- decode
def decode_workload(seed=2026, batch=64):
    shape = CONFIG_SHAPES["decode_bf16"]
    rng = np.random.default_rng(seed)
    lens = [int(x) for x in rng.integers(128, 8193, batch)]
    seqs = [SeqSpec(i, L - 1, 1) for i, L in enumerate(lens)]
    return shape, build_batch(shape, seqs, seed=seed, page_seed=seed + 1)


def decode_bytes(shape, lens):
    """Algorithmic bytes of one decode step: K and V once (the new token's rows read from the
    new-token arrays), the new token's K and V written to its slot, q in, fp32 out, the page
    table. The split kernel moves all but the output."""
    D, Hq, Hkv = shape.head_dim, shape.num_q_heads, shape.num_kv_heads
    lens = np.asarray(lens, np.int64)
    kv = int((lens * Hkv * D * 2 * 2).sum())
    slot_writes = len(lens) * Hkv * D * 2 * 2
    pages = int(((lens + 15) // 16).sum()) * 4
    q_in = len(lens) * Hq * D * 2
    out = len(lens) * Hq * D * 4
    return dict(total=kv + slot_writes + pages + q_in + out,
                split_kernel=kv + slot_writes + pages + q_in, kv=kv)


def run_decode_bench(args, result):
    shape, bt = decode_workload()
    cfg = cfg_of(shape)
    B = bt.batch
    log(f"decode workload: B={B}, KV {decode_bytes(shape, bt.seq_lens)['kv'] / 1e6:.0f} MB")
    q, kn, vn = (dev(bt.q, torch.bfloat16), dev(bt.k_new, torch.bfloat16), dev(bt.v_new, torch.bfloat16))
    pt, sl = dev(bt.page_table, torch.int32), dev(bt.seq_lens, torch.int32)
    qs = dev(bt.q_starts, torch.int32)
    mx = bt.max_seq_len
    # R copies of the pool so no step finds its KV in the 256 MB last-level cache
    R = args.rotate
    pools = [(dev(bt.k_pool, torch.bfloat16), dev(bt.v_pool, torch.bfloat16)) for _ in range(R)]
    ws = torch.empty(bi.bi_attn_workspace_bytes(cfg, B, mx) // 4 + 64, device="cuda")
    out = torch.empty((B, shape.num_q_heads, shape.head_dim), device="cuda")
    for kc, vc in pools:
        bi.bi_kv_page_update(cfg, kn, vn, qs, sl, pt, kc, vc)

    # --- parity and invariance, in this run, before any timing
    bi.bi_attn_decode(cfg, q, pools[0][0], pools[0][1], pt, sl, mx, out, ws)
    ref_bits = out.clone()
    for p in (0, 17, 63):
        it = torch.tensor([p], device="cuda", dtype=torch.long)
        o1 = torch.empty((1, shape.num_q_heads, shape.head_dim), device="cuda")
        bi.bi_attn_decode(cfg, q[it].contiguous(), pools[0][0], pools[0][1], pt[it].contiguous(),
                          sl[it].contiguous(), mx, o1, ws)
        assert torch.equal(o1.view(torch.int32), ref_bits[p:p + 1].view(torch.int32)), \
            f"decode invariance broken for sequence {p} (B=1 vs B={B})"
    # the same batch in reversed order: every row's bits unchanged
    rev = torch.arange(B - 1, -1, -1, device="cuda")
    o_rev = torch.empty_like(out)
    bi.bi_attn_decode(cfg, q[rev].contiguous(), pools[1 % R][0], pools[1 % R][1],
                      pt[rev].contiguous(), sl[rev].contiguous(), mx, o_rev, ws)
    assert torch.equal(o_rev[rev].view(torch.int32), ref_bits.view(torch.int32)), "order invariance"
    result["invariance"] = {"decode": "bitwise: B=1 vs B=64 for sequences 0, 17, 63; "
                                      "reversed batch order; all rows equal"}
    gpu_out = ref_bits.cpu().double().numpy()

    # --- the non-invariant comparison variants (split count chosen by batch: about 2 splits
    # per CU, and enough to fill the 8 resident waves per CU)
    cfg_v = cfg_of(shape, bi.BI_SPLIT_BY_BATCH)
    cfg_f = cfg_of(shape, bi.BI_SPLIT_BY_BATCH_FILL)
    ws_v = torch.empty(max(bi.bi_attn_workspace_bytes(c, B, mx) for c in (cfg_v, cfg_f)) // 4 + 64,
                       device="cuda")

    # One step: the page update folded into the split kernel (bi_attn_decode_append: the new
    # token's K/V written to its slot, split partials, combine; two launches). The per-kernel
    # pass runs the same step as its two phases with events between them.
    def step(i, c, w, tm=None):
        kc, vc = pools[i % R]
        if tm is None:
            bi.bi_attn_decode_append(c, q, kn, vn, kc, vc, pt, sl, mx, out, w)
            return
        tm.mark(0)
        bi.bi_attn_decode_append_partials(c, q, kn, vn, kc, vc, pt, sl, mx, w)
        tm.mark(1)
        bi.bi_attn_decode_combine(c, sl, mx, out, w)
        tm.mark(2)

    def whole_run(c, w):
        for i in range(args.warmup):
            step(i, c, w)
        tm = Timer(2)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        tm.mark(0)
        for i in range(args.steps):
            step(i, c, w)
        tm.mark(1)
        torch.cuda.synchronize()
        return tm.ms(0, 1) / args.steps, (time.perf_counter() - t0) / args.steps

    # the step folded in one call matches the separate page update + decode bit for bit
    step(0, cfg, ws)
    assert torch.equal(out.view(torch.int32), ref_bits.view(torch.int32)), \
        "decode with the folded page update differs from page update + decode"
    # the timed steps: one call per step (events only around the whole run)
    gpu_step, wall = whole_run(cfg, ws)
    # per-kernel breakdown in a separate pass with events between the two phases
    timers = [Timer(3) for _ in range(args.steps)]
    for i in range(args.steps):
        step(i, cfg, ws, timers[i])
    torch.cuda.synchronize()
    comb = [t.ms(1, 2) for t in timers]
    steps_ms = [t.ms(0, 2) for t in timers]
    # the dominant kernel alone: back-to-back launches on the same stream (rotating the pools),
    # events around each launch and around the whole run (the average excludes the records)
    tk = Timer(2)
    torch.cuda.synchronize()
    tk.mark(0)
    for i in range(args.steps):
        kc, vc = pools[i % R]
        bi.bi_attn_decode_append_partials(cfg, q, kn, vn, kc, vc, pt, sl, mx, ws)
    tk.mark(1)
    torch.cuda.synchronize()
    part = tk.ms(0, 1) / args.steps
    part_each = []
    for i in range(args.steps):
        kc, vc = pools[i % R]
        t1 = Timer(2)
        t1.mark(0)
        bi.bi_attn_decode_append_partials(cfg, q, kn, vn, kc, vc, pt, sl, mx, ws)
        t1.mark(1)
        part_each.append(t1)
    torch.cuda.synchronize()
    part_each = [t.ms(0, 1) for t in part_each]
    # the separate page update kernel, for reference (not part of the step)
    tpu = Timer(2)
    torch.cuda.synchronize()
    tpu.mark(0)
    for i in range(args.steps):
        kc, vc = pools[i % R]
        bi.bi_kv_page_update(cfg, kn, vn, qs, sl, pt, kc, vc)
    tpu.mark(1)
    torch.cuda.synchronize()
    pu_alone = tpu.ms(0, 1) / args.steps

    # variant timing (same step shape)
    var_step = fill_step = None
    if not args.profile_run:
        var_step = whole_run(cfg_v, ws_v)[0]
        fill_step = whole_run(cfg_f, ws_v)[0]

    nb = decode_bytes(shape, bt.seq_lens)
    step_ms = max(wall * 1e3, gpu_step)
    result.update(
        value=nb["total"] / (step_ms * 1e-3) / 1e9,
        ms_per_step=step_ms,
        config={"workload": "decode_bf16: batch 64, 1 query token each, Hq 32, Hkv 4, D 128, "
                            "context U[128,8192], page 16 (shuffled), split 256",
                "global_batch": B, "seq_len": int(np.mean(bt.seq_lens)), "parallelism": "none"},
    )
    split_gbs = nb["split_kernel"] / (part * 1e-3) / 1e9
    result["roofline"] = {"bound": "hbm", "kernel": "decode_split_kernel<bf16,128,1,append>",
                          "achieved": split_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                          "frac": split_gbs / HBM_PEAK_GBS,
                          "traffic": profiled_traffic("decode_split_kernel"),
                          "bytes_per_launch": nb["split_kernel"], "avg_launch_ms": part}
    result["decode_breakdown_ms"] = {"append_partials": part, "combine": float(np.mean(comb)),
                                     "step_events": gpu_step, "step_wall": wall * 1e3,
                                     "separate_page_update_not_in_step": pu_alone}
    result["decode_stats"] = {"step_with_events": stats_ms(steps_ms),
                              "append_partials": stats_ms(part_each), "combine": stats_ms(comb),
                              "step_GBps_median": nb["total"] / (np.median(steps_ms) * 1e-3) / 1e9}
    result["variant_slowdown"] = {
        "definition": "t(invariant) / t(variant) - 1 on the same step (page update folded into "
                      "the split kernel, combine); variants pick the split count from the batch",
        "decode_vs_2_per_cu": gpu_step / var_step - 1.0 if var_step else None,
        "decode_vs_fill_8_per_cu": gpu_step / fill_step - 1.0 if fill_step else None,
        "decode_ms": {"invariant": gpu_step, "split_by_batch_2_per_cu": var_step,
                      "split_by_batch_fill_8_per_cu": fill_step}}

    # --- sweep over batch sizes (first B sequences of the same workload)
    sweep = []
    for Bs in (() if args.profile_run else (1, 2, 4, 8, 16, 32, 64)):
        idx = torch.arange(Bs, device="cuda")
        qb, ptb, slb = q[idx].contiguous(), pt[idx].contiguous(), sl[idx].contiguous()
        ob = torch.empty((Bs, shape.num_q_heads, shape.head_dim), device="cuda")
        mxb = int(bt.seq_lens[:Bs].max())
        n = max(args.steps, 20)
        for i in range(5):
            bi.bi_attn_decode(cfg, qb, pools[i % R][0], pools[i % R][1], ptb, slb, mxb, ob, ws)
        tm = Timer(2)
        torch.cuda.synchronize()
        tm.mark(0)
        for i in range(n):
            bi.bi_attn_decode(cfg, qb, pools[i % R][0], pools[i % R][1], ptb, slb, mxb, ob, ws)
        tm.mark(1)
        torch.cuda.synchronize()
        ms = tm.ms(0, 1) / n
        byt = decode_bytes(shape, bt.seq_lens[:Bs])["total"]
        sweep.append({"batch": Bs, "us": ms * 1e3, "GBps": byt / (ms * 1e-3) / 1e9})
    result["decode_sweep"] = sweep
    return bt, gpu_out


# ----------------------------------------------------------------------------- prefill
def prefill_workload(seed=2027):
    shape = CONFIG_SHAPES["prefill_bf16"]
    rng = np.random.default_rng(seed)
    specs = [SeqSpec(i, int(rng.integers(0, 16385)), int(rng.integers(1, 2049))) for i in range(16)]
    return shape, build_batch(shape, specs, seed=seed, page_seed=seed + 1)


def prefill_flops(bt):
    D, Hq = bt.shape.head_dim, bt.shape.num_q_heads
    tot = 0
    for s in bt.seqs:
        n = s.n_new
        tot += 4 * D * Hq * (n * (s.cached + 1) + n * (n - 1) // 2)
    return tot


def run_prefill_bench(args, result):
    shape, bt = prefill_workload()
    cfg = cfg_of(shape)
    log(f"prefill workload: {bt.total_tokens} new tokens, {prefill_flops(bt) / 1e12:.2f} TFLOP")
    q, kn, vn = (dev(bt.q, torch.bfloat16), dev(bt.k_new, torch.bfloat16), dev(bt.v_new, torch.bfloat16))
    kc, vc = dev(bt.k_pool, torch.bfloat16), dev(bt.v_pool, torch.bfloat16)
    pt, sl, qs = dev(bt.page_table, torch.int32), dev(bt.seq_lens, torch.int32), dev(bt.q_starts, torch.int32)
    out = torch.empty((bt.total_tokens, shape.num_q_heads, shape.head_dim), device="cuda")
    bi.bi_kv_page_update(cfg, kn, vn, qs, sl, pt, kc, vc)
    bi.bi_attn_prefill(cfg, q, kc, vc, pt, qs, sl, bt.max_q_len, bt.max_seq_len, out)
    ref = out.clone()
    # invariance: last token of every sequence through decode must match bitwise
    last = torch.tensor([int(bt.q_starts[b + 1]) - 1 for b in range(bt.batch)], device="cuda")
    od = torch.empty((bt.batch, shape.num_q_heads, shape.head_dim), device="cuda")
    ws = torch.empty(bi.bi_attn_workspace_bytes(cfg, bt.batch, bt.max_seq_len) // 4 + 64, device="cuda")
    bi.bi_attn_decode(cfg, q[last].contiguous(), kc, vc, pt, sl, bt.max_seq_len, od, ws)
    assert torch.equal(od.view(torch.int32), ref[last].view(torch.int32)), "prefill vs decode bits"
    result.setdefault("invariance", {})["prefill"] = ("bitwise: last token of each of the 16 "
                                                      "sequences, prefill vs decode")

    def run(c, n, warm):
        for _ in range(warm):
            bi.bi_attn_prefill(c, q, kc, vc, pt, qs, sl, bt.max_q_len, bt.max_seq_len, out)
        tms = [Timer(3) for _ in range(n)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(n):
            tms[i].mark(0)
            bi.bi_kv_page_update(c, kn, vn, qs, sl, pt, kc, vc)
            tms[i].mark(1)
            bi.bi_attn_prefill(c, q, kc, vc, pt, qs, sl, bt.max_q_len, bt.max_seq_len, out)
            tms[i].mark(2)
        torch.cuda.synchronize()
        wall = (time.perf_counter() - t0) / n * 1e3
        kern = [t.ms(1, 2) for t in tms]
        return float(np.median(kern)), float(np.mean([t.ms(0, 2) for t in tms])), wall, kern

    n = max(10, args.steps // 2)
    kern, step_ms, wall, kern_all = run(cfg, n, max(2, args.warmup // 3))
    kern_v = kern_f = None
    if not args.profile_run:
        kern_v = run(cfg_of(shape, bi.BI_SPLIT_BY_BATCH), n, 2)[0]
        kern_f = run(cfg_of(shape, bi.BI_SPLIT_BY_BATCH_FILL), n, 2)[0]
    fl = prefill_flops(bt)
    tf = fl / (kern * 1e-3) / 1e12
    ks = stats_ms(kern_all)
    result["prefill"] = {
        "value": fl / (max(step_ms, wall) * 1e-3) / 1e12, "unit": "TFLOP/s",
        "kernel_tflops": tf, "ms_per_step": max(step_ms, wall), "kernel_ms": kern,
        "kernel_stats": ks,
        "kernel_tflops_p10_p90": [fl / (ks["p90_us"] * 1e-6) / 1e12, fl / (ks["p10_us"] * 1e-6) / 1e12],
        "flops_per_step": fl,
        "config": {"workload": "prefill_bf16: 16 sequences, Hq 64, Hkv 4, D 128, cached prefix "
                               "U[0,16384], chunk U[1,2048], page 16, split 256",
                   "new_tokens": bt.total_tokens},
    }
    result["roofline_prefill"] = {"bound": "mfma", "kernel": "prefill_kernel<bf16,128,2>",
                                  "achieved": tf, "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                                  "frac": tf / BF16_PEAK_TFLOPS, "kernel_ms_median": kern,
                                  "traffic": profiled_traffic("prefill_kernel")}
    vs = result.setdefault("variant_slowdown", {})
    vs["prefill_vs_2_per_cu"] = kern / kern_v - 1.0 if kern_v else None
    vs["prefill_vs_fill_8_per_cu"] = kern / kern_f - 1.0 if kern_f else None
    vs["prefill_ms"] = {"invariant": kern, "split_by_batch_2_per_cu": kern_v,
                        "split_by_batch_fill_8_per_cu": kern_f}
    run_varlen_bench(args, result, shape, bt, cfg, q, kc, vc, pt, ref)
    return bt, ref


def run_varlen_bench(args, result, shape, bt, cfg, q, kc, vc, pt, ref):
    """The same prefill workload through bi_attn_varlen (dense [rows][Hkv][D] keys and values,
    the trainer's layout): bits against the paged prefill, and kernel time."""
    ks, vs = [], []
    for b in range(bt.batch):
        L = int(bt.seq_lens[b])
        npg = (L + 15) // 16
        pages = pt[b, :npg].long()
        for cache, dst in ((kc, ks), (vc, vs)):
            blk = cache[pages]
            dst.append(blk.permute(0, 2, 1, 3).reshape(npg * 16, shape.num_kv_heads, shape.head_dim)[:L])
    kd, vd = torch.cat(ks).contiguous(), torch.cat(vs).contiguous()
    k_starts = dev(np.concatenate([[0], np.cumsum(bt.seq_lens)]).astype(np.int32), torch.int32)
    qs = dev(bt.q_starts, torch.int32)
    out = torch.empty_like(ref)
    bi.bi_attn_varlen(cfg, q, kd, vd, qs, k_starts, bt.max_q_len, bt.max_seq_len, out)
    assert torch.equal(out.view(torch.int32), ref.view(torch.int32)), "varlen vs paged prefill bits"
    n = max(3, args.steps // 5)
    for _ in range(2):
        bi.bi_attn_varlen(cfg, q, kd, vd, qs, k_starts, bt.max_q_len, bt.max_seq_len, out)
    tm = Timer(2)
    torch.cuda.synchronize()
    tm.mark(0)
    for _ in range(n):
        bi.bi_attn_varlen(cfg, q, kd, vd, qs, k_starts, bt.max_q_len, bt.max_seq_len, out)
    tm.mark(1)
    torch.cuda.synchronize()
    ms = tm.ms(0, 1) / n
    tf = prefill_flops(bt) / (ms * 1e-3) / 1e12
    result["varlen"] = {"kernel_tflops": tf, "kernel_ms": ms,
                        "unit": "TFLOP/s",
                        "roofline": {"bound": "mfma", "kernel": "prefill_kernel<bf16,128,...,DENSE=true>",
                                     "achieved": tf, "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                                     "frac": tf / BF16_PEAK_TFLOPS,
                                     "traffic": profiled_traffic("prefill_kernel_dense")},
                        "bits": "all rows equal to the paged prefill of the same keys and values",
                        "config": {"workload": "the prefill workload with dense keys and values "
                                               "[rows][Hkv][D] (bi_attn_varlen)"}}
    log(f"varlen (dense K/V): {result['varlen']['kernel_tflops']:.1f} TFLOP/s, same bits as paged")


# ----------------------------------------------------------------------------- long decode
def run_long_decode_bench(args, result):
    """Long-context decode: 8 sequences of 131072 tokens, 64/4 heads, q x 4 (peaked softmax);
    each split kernel launch reads 2.15 GB of K/V, far more than the last-level cache."""
    shape = CONFIG_SHAPES["long_decode_bf16"]
    cfg = cfg_of(shape)
    L, B = 131072, 8
    bt = build_batch(shape, [SeqSpec(i, L - 1, 1) for i in range(B)], seed=2028, page_seed=2029,
                     q_scale=4.0)
    log(f"long decode workload: B={B} x {L}, KV {decode_bytes(shape, bt.seq_lens)['kv'] / 1e9:.2f} GB")
    q, kn, vn = dev(bt.q, torch.bfloat16), dev(bt.k_new, torch.bfloat16), dev(bt.v_new, torch.bfloat16)
    kc, vc = dev(bt.k_pool, torch.bfloat16), dev(bt.v_pool, torch.bfloat16)
    pt, sl, qs = dev(bt.page_table, torch.int32), dev(bt.seq_lens, torch.int32), dev(bt.q_starts, torch.int32)
    ws = torch.empty(bi.bi_attn_workspace_bytes(cfg, B, L) // 4 + 64, device="cuda")
    out = torch.empty((B, shape.num_q_heads, shape.head_dim), device="cuda")
    bi.bi_kv_page_update(cfg, kn, vn, qs, sl, pt, kc, vc)
    bi.bi_attn_decode(cfg, q, kc, vc, pt, sl, L, out, ws)
    ref = out.clone()
    for b in (0, 5):        # each sequence alone at batch size 1: the same bits
        it = torch.tensor([b], device="cuda")
        o1 = torch.empty((1, shape.num_q_heads, shape.head_dim), device="cuda")
        bi.bi_attn_decode(cfg, q[it].contiguous(), kc, vc, pt[it].contiguous(), sl[it].contiguous(), L, o1, ws)
        assert torch.equal(o1.view(torch.int32), ref[b:b + 1].view(torch.int32)), "long decode B=1 vs B=8"

    # the same step as the decode workload's: page update folded into the split kernel
    def step(tm=None):
        if tm is None:
            bi.bi_attn_decode_append(cfg, q, kn, vn, kc, vc, pt, sl, L, out, ws)
            return
        tm.mark(0)
        bi.bi_attn_decode_append_partials(cfg, q, kn, vn, kc, vc, pt, sl, L, ws)
        tm.mark(1)
        bi.bi_attn_decode_combine(cfg, sl, L, out, ws)
        tm.mark(2)

    for _ in range(3):
        step()
    n = max(10, args.steps // 2)
    whole = Timer(2)
    torch.cuda.synchronize()
    whole.mark(0)
    for _ in range(n):
        step()
    whole.mark(1)
    torch.cuda.synchronize()
    step_ms = whole.ms(0, 1) / n
    assert torch.equal(out.view(torch.int32), ref.view(torch.int32)), "long decode: folded step"
    tms = [Timer(3) for _ in range(n)]
    for t in tms:
        step(t)
    torch.cuda.synchronize()
    part = [t.ms(0, 1) for t in tms]
    nb = decode_bytes(shape, bt.seq_lens)
    gbs = nb["split_kernel"] / (np.median(part) * 1e-3) / 1e9
    result["long_decode"] = {
        "value": nb["total"] / (step_ms * 1e-3) / 1e9, "unit": "GB/s", "ms_per_step": step_ms,
        "step_stats": stats_ms([t.ms(0, 2) for t in tms]), "append_partials_stats": stats_ms(part),
        "combine_stats": stats_ms([t.ms(1, 2) for t in tms]),
        "roofline": {"bound": "hbm", "kernel": "decode_split_kernel<bf16,128,1,append>", "achieved": gbs,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": gbs / HBM_PEAK_GBS,
                     "traffic": profiled_traffic("decode_split_kernel_long"),
                     "bytes_per_launch": nb["split_kernel"], "avg_launch_ms": float(np.median(part))},
        "invariance": "bitwise: sequences 0 and 5 alone at B=1 equal to the B=8 call",
        "config": {"workload": "long_decode_bf16: 8 sequences x 131072 tokens, Hq 64, Hkv 4, D 128, "
                               "q x 4, page 16 (shuffled), split 256 (512 splits folded in order)"}}
    log(f"long decode: step {result['long_decode']['value']:.0f} GB/s, split kernel {gbs:.0f} GB/s")
    return bt, ref


# ----------------------------------------------------------------------------- mixed trace
def run_trace_bench(args, result):
    """The mixed continuous-batching trace: 256 requests, 64 steps of at most 8192 tokens, decode
    tokens first then FCFS prompt chunks, 64/4 heads; each step is the page update, one decode
    call for the decode tokens and one prefill call for the chunks. Inputs are generated on the
    device for all steps before timing."""
    from synth import mixed_trace
    from synth.device import normal_tokens
    from synth.workloads import PageAllocator
    HQ, HKV, D, P = 64, 4, 128, 16
    cfg = bi.AttnConfig(HQ, HKV, D, P, 256, bi.BI_BF16)
    seed = 2029
    tr = mixed_trace(seed)
    num_pages = 48 * 1024
    kc = torch.zeros((num_pages, HKV, P, D), dtype=torch.bfloat16, device="cuda")
    vc = torch.zeros_like(kc)
    alloc = PageAllocator(num_pages, seed=seed)
    steps = []
    for st in tr.steps:
        dec = [(r, pos, 1) for r, pos in st.decode]
        pre = [(r, s0, n) for r, s0, n in st.prefill]
        ent = dec + pre
        req = torch.tensor([r for r, s0, n in ent for _ in range(n)], device="cuda")
        pos = torch.tensor([p for r, s0, n in ent for p in range(s0, s0 + n)], device="cuda")
        pages = [alloc.ensure(r, s0 + n, P) for r, s0, n in ent]
        mp = max(len(pg) for pg in pages)
        table = torch.full((len(ent), mp), -1, dtype=torch.int32)
        for i, pg in enumerate(pages):
            table[i, :len(pg)] = torch.tensor(pg, dtype=torch.int32)
        sl = [s0 + n for r, s0, n in ent]
        qs = [0] + list(np.cumsum([n for _, _, n in ent]))
        nd = len(dec)
        d = {"q": normal_tokens(seed, req, "q", pos, HQ, D),
             "kn": normal_tokens(seed, req, "k", pos, HKV, D),
             "vn": normal_tokens(seed, req, "v", pos, HKV, D),
             "table": table.cuda(), "sl": torch.tensor(sl, dtype=torch.int32, device="cuda"),
             "qs": torch.tensor(qs, dtype=torch.int32, device="cuda"), "nd": nd,
             "dec_bytes": decode_bytes(CONFIG_SHAPES["mixed_trace_bf16"], sl[:nd])["total"] if nd else 0,
             "pre_flops": sum(4 * D * HQ * (n * (s0 + 1) + n * (n - 1) // 2) for _, s0, n in pre),
             "pre_tokens": sum(n for _, _, n in pre)}
        if nd:
            d["dq"] = d["q"][:nd].contiguous()
            d["dtable"] = d["table"][:nd].contiguous()
            d["dsl"] = d["sl"][:nd].contiguous()
            d["dmx"] = max(sl[:nd])
            d["dws"] = torch.empty(bi.bi_attn_workspace_bytes(cfg, nd, d["dmx"]) // 4 + 64, device="cuda")
            d["dout"] = torch.empty((nd, HQ, D), device="cuda")
        if pre:
            d["pq"] = d["q"][nd:].contiguous()
            d["ptable"] = d["table"][nd:].contiguous()
            d["psl"] = d["sl"][nd:].contiguous()
            d["pqs"] = (d["qs"][nd:] - nd).contiguous()
            d["pmxq"] = max(n for _, _, n in pre)
            d["pmx"] = max(sl[nd:])
            d["pout"] = torch.empty((d["pre_tokens"], HQ, D), device="cuda")
        steps.append(d)
        for r in st.finished:
            alloc.release(r)

    def run_step(d, tm=None):
        if tm: tm.mark(0)
        bi.bi_kv_page_update(cfg, d["kn"], d["vn"], d["qs"], d["sl"], d["table"], kc, vc)
        if tm: tm.mark(1)
        if d["nd"]:
            bi.bi_attn_decode(cfg, d["dq"], kc, vc, d["dtable"], d["dsl"], d["dmx"], d["dout"], d["dws"])
        if tm: tm.mark(2)
        if "pq" in d:
            bi.bi_attn_prefill(cfg, d["pq"], kc, vc, d["ptable"], d["pqs"], d["psl"], d["pmxq"], d["pmx"], d["pout"])
        if tm: tm.mark(3)

    # the trace once untimed (fills the cache), then timed: the steps write the same K/V again
    for d in steps:
        run_step(d)
    torch.cuda.synchronize()
    # route check on one mixed step: one prefill call with the decode tokens as 1-token chunks
    # gives the bits of the decode call plus the prefill call
    d = next(x for x in steps if x["nd"] and "pq" in x)
    run_step(d)
    T = int(d["qs"][-1])
    o1 = torch.empty((T, HQ, D), device="cuda")
    bi.bi_attn_prefill(cfg, d["q"], kc, vc, d["table"], d["qs"], d["sl"], max(d["pmxq"], 1),
                       max(d["pmx"], d["dmx"]), o1)
    assert torch.equal(o1[:d["nd"]].view(torch.int32), d["dout"].view(torch.int32)), "trace decode route"
    assert torch.equal(o1[d["nd"]:].view(torch.int32), d["pout"].view(torch.int32)), "trace prefill route"
    tms = [Timer(4) for _ in steps]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for d, t in zip(steps, tms):
        run_step(d, t)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    step_ms = [t.ms(0, 3) for t in tms]
    dec_ms = sum(t.ms(1, 2) for t, d in zip(tms, steps) if d["nd"])
    pre_ms = sum(t.ms(2, 3) for t, d in zip(tms, steps) if "pq" in d)
    dec_bytes = sum(d["dec_bytes"] for d in steps)
    pre_flops = sum(d["pre_flops"] for d in steps)
    toks = sum(int(d["qs"][-1]) for d in steps)
    result["mixed_trace"] = {
        "value": toks / (sum(step_ms) * 1e-3), "unit": "tokens/s", "steps": len(steps), "tokens": toks,
        "step_stats": stats_ms(step_ms), "wall_s": wall,
        "decode": {"GBps": dec_bytes / (dec_ms * 1e-3) / 1e9, "ms": dec_ms, "bytes": dec_bytes},
        "prefill": {"TFLOPs": pre_flops / (pre_ms * 1e-3) / 1e12, "ms": pre_ms, "flops": pre_flops},
        "invariance": "bitwise: one mixed step as one prefill call (decode tokens as 1-token chunks) "
                      "equal to its decode call plus prefill call",
        "config": {"workload": "mixed_trace_bf16: 256 requests, 64 steps, <= 8192 tokens per step, "
                               "prompts floor(exp U[ln 64, ln 32768]), outputs U[16, 1024], Hq 64, "
                               "Hkv 4, D 128, page 16, split 256"}}
    log(f"mixed trace: {toks} tokens in {sum(step_ms):.1f} ms of steps (median step "
        f"{result['mixed_trace']['step_stats']['median_us']:.0f} us); decode "
        f"{result['mixed_trace']['decode']['GBps']:.0f} GB/s, prefill {result['mixed_trace']['prefill']['TFLOPs']:.0f} TFLOP/s")
    del steps, kc, vc


# ----------------------------------------------------------------------------- RMSNorm
def run_rmsnorm_bench(args, result):
    """Batch-invariant RMSNorm of a 16384-token activation block (hidden 4096, bf16): HBM GB/s
    (x read once, y written once, the weight once), and row bits at 1 vs 16384 rows."""
    from synth import norm_inputs
    rows, hidden = 16384, 4096
    x, w = norm_inputs(2030, rows, hidden, "bf16")
    xs = [dev(x, torch.bfloat16) for _ in range(2)]     # two copies, alternated across launches
    wd = dev(w, torch.bfloat16)
    y = torch.empty_like(xs[0])
    bi.bi_rmsnorm(xs[0], wd, y, 1e-6)
    y1 = torch.empty((1, hidden), dtype=torch.bfloat16, device="cuda")
    for r in (0, 7777, rows - 1):
        bi.bi_rmsnorm(xs[0][r:r + 1].contiguous(), wd, y1, 1e-6)
        assert torch.equal(y1.view(torch.int16), y[r:r + 1].view(torch.int16)), "rmsnorm row bits"
    n = max(10, args.steps)
    for i in range(3):
        bi.bi_rmsnorm(xs[i % 2], wd, y, 1e-6)
    tm = Timer(2)
    torch.cuda.synchronize()
    tm.mark(0)
    for i in range(n):
        bi.bi_rmsnorm(xs[i % 2], wd, y, 1e-6)
    tm.mark(1)
    torch.cuda.synchronize()
    ms = tm.ms(0, 1) / n
    nbytes = 2 * rows * hidden * 2 + hidden * 2
    gbs = nbytes / (ms * 1e-3) / 1e9
    result["rmsnorm"] = {"value": gbs, "unit": "GB/s", "ms": ms, "bytes": nbytes,
                         "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS,
                                      "unit": "GB/s", "frac": gbs / HBM_PEAK_GBS,
                                      "traffic": profiled_traffic("rmsnorm_kernel", NORM_SOURCES)},
                         "bits": "rows 0, 7777, 16383 alone equal to the 16384-row call",
                         "config": {"workload": "rmsnorm_bf16: 16384 rows x hidden 4096, eps 1e-6"}}
    log(f"rmsnorm: {gbs:.0f} GB/s ({ms * 1e3:.1f} us for {nbytes / 1e6:.0f} MB)")


# ----------------------------------------------------------------------------- GEMM
def run_gemm_bench(args, result):
    """Batch-invariant GEMM C = A W^T on a linear-layer shape (8192 tokens, 4096 -> 8192, bf16),
    against torch.matmul (hipBLASLt) on the same tensors; row bits at M = 1 vs M = 8192."""
    m, n, k = 8192, 8192, 4096
    g = torch.Generator(device="cuda").manual_seed(2031)
    a = torch.randn((m, k), device="cuda", generator=g).to(torch.bfloat16)
    w = (torch.randn((n, k), device="cuda", generator=g) / 64).to(torch.bfloat16)
    c = torch.empty((m, n), device="cuda", dtype=torch.bfloat16)
    bi.bi_gemm(a, w, c)
    c1 = torch.empty((1, n), device="cuda", dtype=torch.bfloat16)
    for r in (0, 4097, m - 1):
        bi.bi_gemm(a[r:r + 1].contiguous(), w, c1)
        assert torch.equal(c1.view(torch.int16), c[r:r + 1].view(torch.int16)), "gemm row bits"
    ref_full = torch.matmul(a, w.t())
    vendor_same = all(torch.equal(torch.matmul(a[r:r + 1], w.t()).view(torch.int16),
                                  ref_full[r:r + 1].view(torch.int16)) for r in (0, 4097, m - 1))

    def timed(fn, n_it):
        for _ in range(3):
            fn()
        tm = Timer(2)
        torch.cuda.synchronize()
        tm.mark(0)
        for _ in range(n_it):
            fn()
        tm.mark(1)
        torch.cuda.synchronize()
        return tm.ms(0, 1) / n_it

    n_it = max(10, args.steps // 2)
    ms = timed(lambda: bi.bi_gemm(a, w, c), n_it)
    ms_v = timed(lambda: torch.matmul(a, w.t(), out=c), n_it)
    fl = 2.0 * m * n * k
    tf, tf_v = fl / (ms * 1e-3) / 1e12, fl / (ms_v * 1e-3) / 1e12
    # token counts of decode and small prefill chunks (other kernels: 64 x 64 tiles, skinny);
    # W rotated over four copies so it is not cache resident, bandwidth of W
    small = {}
    for sm, sn, sk in ((1, 4096, 4096), (64, 8192, 4096), (128, 14336, 4096), (1, 8192, 14336)):
        sa = torch.randn((sm, sk), device="cuda", generator=g).to(torch.bfloat16)
        sws = [(torch.randn((sn, sk), device="cuda", generator=g) / 64).to(torch.bfloat16) for _ in range(4)]
        sc = torch.empty((sm, sn), device="cuda", dtype=torch.bfloat16)
        it = iter(range(1 << 30))
        t_b = timed(lambda: bi.bi_gemm(sa, sws[next(it) % 4], sc), 20)
        t_v = timed(lambda: torch.matmul(sa, sws[next(it) % 4].t(), out=sc), 20)
        small[f"{sm}x{sn}x{sk}"] = {"us": t_b * 1e3, "w_gbs": sn * sk * 2 / (t_b * 1e-3) / 1e9,
                                    "hipblaslt_us": t_v * 1e3, "ratio": t_v / t_b}
        del sa, sws, sc
    result["gemm"] = {"value": tf, "unit": "TFLOP/s", "ms": ms,
                      "roofline": {"bound": "mfma", "achieved": tf, "peak": BF16_PEAK_TFLOPS,
                                   "unit": "TFLOP/s", "frac": tf / BF16_PEAK_TFLOPS,
                                   "traffic": profiled_traffic("gemm_kernel", GEMM_SOURCES)},
                      "bytes": 2 * (m * k + n * k + m * n),
                      "vs_hipblaslt": {"hipblaslt_tflops": tf_v, "ratio": tf / tf_v,
                                       "hipblaslt_rows_same_bits_at_m1": vendor_same},
                      "bits": "rows 0, 4097, 8191 at M = 1 equal to the M = 8192 call",
                      "small_m": small,
                      "config": {"workload": "gemm_bf16: C[8192][8192] = A[8192][4096] W[8192][4096]^T, "
                                             "bf16 in and out, fp32 accumulation"}}
    log(f"gemm: {tf:.0f} TFLOP/s ({tf / tf_v:.2f}x hipBLASLt {tf_v:.0f}; hipBLASLt rows same bits "
        f"at M = 1: {vendor_same}); small M: " +
        ", ".join(f"{kk} {v['us']:.1f} us ({v['ratio']:.2f}x)" for kk, v in small.items()))


# ----------------------------------------------------------------------------- CPU baseline
def cpu_baseline(result, bt_dec, gpu_dec, samples, pf=None, long=None):
    """Time the fp64 oracle on the host on a bounded sample of the headline decode workload and
    use its outputs for the parity check; also check sampled rows of the prefill and long-context
    workloads (``pf``, ``long``: (batch, GPU output)) against the oracle."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        threads = os.cpu_count()
    kc, vc = bt_dec.k_pool.copy(), bt_dec.v_pool.copy()
    oracle.kv_page_update(bt_dec.k_new, bt_dec.v_new, bt_dec.q_starts, bt_dec.seq_lens,
                          bt_dec.page_table, kc, vc)
    n = min(samples, bt_dec.batch)
    t0 = time.perf_counter()
    reps = 0
    while True:
        ref = oracle.paged_attention(bt_dec.q[:n], kc, vc, bt_dec.page_table[:n],
                                     bt_dec.q_starts[: n + 1], bt_dec.seq_lens[:n],
                                     bt_dec.shape.num_kv_heads)
        reps += 1
        if time.perf_counter() - t0 > 10.0 or reps >= 64:   # about 10 s of host work
            break
    dt = (time.perf_counter() - t0) / reps
    byt = decode_bytes(bt_dec.shape, bt_dec.seq_lens[:n])["total"]
    err = np.abs(gpu_dec[:n] - ref)
    parity = {"decode_rows": int(n * bt_dec.shape.num_q_heads), "max_abs": float(err.max()),
              "mean_abs": float(err.mean())}
    assert err.max() <= 2e-3 and err.mean() <= 2e-4, parity

    def sampled(bt, out, rows, in_place=False):
        kc2, vc2 = (bt.k_pool, bt.v_pool) if in_place else (bt.k_pool.copy(), bt.v_pool.copy())
        oracle.kv_page_update(bt.k_new, bt.v_new, bt.q_starts, bt.seq_lens, bt.page_table, kc2, vc2)
        want = oracle.paged_attention_rows(bt.q, kc2, vc2, bt.page_table, bt.q_starts, bt.seq_lens,
                                           bt.shape.num_kv_heads, rows)
        got = np.stack([out[t, h].double().cpu().numpy() for t, h in rows])
        e = np.abs(got - want)
        rec = {"rows": len(rows), "max_abs": float(e.max()), "mean_abs": float(e.mean())}
        assert e.max() <= 2e-3 and e.mean() <= 2e-4, rec
        return rec

    if pf is not None:
        bt_pf, out_pf = pf
        T, Hq = bt_pf.total_tokens, bt_pf.shape.num_q_heads
        rows = [(int(t), int(h)) for t in np.linspace(0, T - 1, 16).astype(int) for h in (0, 21, 42, Hq - 1)]
        parity["prefill_sample"] = sampled(bt_pf, out_pf, rows)
    if long is not None:
        bt_l, out_l = long
        rows = [(b, h) for b in (0, 3, 7) for h in (0, 17, 40, 63)]
        parity["long_decode_sample"] = sampled(bt_l, out_l, rows, in_place=True)
    result["parity"] = parity
    result["cpu_baseline"] = {"value": byt / dt / 1e9, "unit": "GB/s", "cores": int(threads),
                              "kind": "oracle",
                              "sample": f"decode_bf16, first {n} of 64 sequences (all 32 heads), "
                                        f"fp64 numpy, {reps} rep(s), {dt:.2f} s each, "
                                        f"{dt * reps:.1f} s in all",
                              "host": host_cpu(), "host_cpus": os.cpu_count()}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--rotate", type=int, default=4, help="KV pool copies cycled across steps")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-long", action="store_true", help="skip the long-context decode workload")
    ap.add_argument("--no-trace", action="store_true", help="skip the mixed-trace workload")
    ap.add_argument("--long-only", action="store_true",
                    help="measure the long-context decode workload alone (no headline value; for "
                         "profiling its kernels)")
    ap.add_argument("--prefill-only", action="store_true",
                    help="measure the prefill workload alone (no headline value)")
    ap.add_argument("--cpu-samples", type=int, default=64)
    ap.add_argument("--profile-run", action="store_true",
                    help="only the headline decode steps and the prefill workload, paged and dense (no "
                         "split-by-batch variant, no batch sweep), so a profiler sees one workload "
                         "per kernel")
    ap.add_argument("--next-rows-only", action="store_true",
                    help="only the RMSNorm and GEMM legs (no headline value; for profiling those kernels)")
    ap.add_argument("--copy-calib-mb", type=int, default=0,
                    help="also run a plain device copy of this many MiB (counter calibration)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: this path is built and timed on a single device "
              "(the library has no multi-GPU path); run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    bi.load()
    torch.cuda.set_device(0)
    result = {"metric": METRIC, "value": None, "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
              "warmup": args.warmup, "ms_per_step": None, "higher_is_better": True,
              "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
              "data": "synthetic (seeded N(0,1), bf16-rounded; no model weights)"}
    if args.copy_calib_mb:
        # a plain copy kernel of known size: reads and writes exactly n bytes each
        n = args.copy_calib_mb << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        result["copy_calib_bytes"] = n
        del src, dst
    if args.next_rows_only:
        run_rmsnorm_bench(args, result)
        run_gemm_bench(args, result)
        print(json.dumps(result), flush=True)
        return
    if args.long_only:
        run_long_decode_bench(args, result)
        print(json.dumps(result), flush=True)
        return
    if args.prefill_only:
        result["variant_slowdown"] = {}
        run_prefill_bench(args, result)
        log(f"prefill: {result['prefill']['kernel_tflops']:.1f} TFLOP/s (kernel)")
        print(json.dumps(result), flush=True)
        return
    bt_dec, gpu_dec = run_decode_bench(args, result)
    log(f"decode: {result['value']:.0f} GB/s per step, split kernel "
        f"{result['roofline']['achieved']:.0f} GB/s")
    pf = lg = None
    if not args.no_prefill:
        pf = run_prefill_bench(args, result)
        log(f"prefill: {result['prefill']['kernel_tflops']:.1f} TFLOP/s (kernel)")
    if not args.profile_run:
        if not args.no_long:
            lg = run_long_decode_bench(args, result)
        if not args.no_trace:
            run_trace_bench(args, result)
        run_rmsnorm_bench(args, result)
        run_gemm_bench(args, result)
    if not args.no_cpu_baseline:
        cpu_baseline(result, bt_dec, gpu_dec, args.cpu_samples, pf, lg)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
