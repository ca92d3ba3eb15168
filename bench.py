"""Benchmark of MLA decode over a paged latent KV cache on one MI355X.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--configs 2,3,4,5]

A step is one pass of the decode path over one batch: the scheduler kernel
(mla_get_metadata) and the decode call (split-KV decode + lse combine).  The
headline workload is the memory-bound dense BF16 decode (B=64, h_q=128,
seqlen 4096, block 64, shuffled pages); the other workloads (dense s_q=2
compute-bound, sparse FP8 top-2048, skewed long-context sparse FP8) are
measured the same way and reported under "workloads".  All inputs are seeded
synthetic data resident in HBM before timing.

Counting: FLOPs = 2 (576 + 512) per query row per attended token; bytes = KV
bytes of the attended tokens (1152 B per bf16 token, 656 B per FP8 token) +
q + o.  Peaks: 8.0 TB/s HBM, 2.5 PFLOP/s dense bf16 MFMA.

Prints one JSON line.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0
PEAK_BF16_TFLOPS = 2500.0
METRIC = "decode TFLOP/s + HBM GB/s vs MI355X roofline; dense bf16 & sparse fp8 MLA"
HEADLINE = 2


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--configs", default="2,3,4,5")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cold", action="store_true", help="also time each step after overwriting 1 GiB (cold caches)")
    return ap.parse_args()


def measure(cfg: int, steps: int, warmup: int, cold: bool):
    import torch

    import mla_inputs as mi
    import mla_paged_kv_get_amd as mla

    t0 = time.time()
    prob = mi.config(cfg)
    gen_s = time.time() - t0
    dev = torch.device("cuda:0")
    q = prob.q.to(dev)
    kv = prob.kvcache.to(dev)
    bt = prob.block_table.to(dev)
    sl = prob.cache_seqlens.to(dev)
    idx = None if prob.indices is None else prob.indices.to(dev)
    topk = prob.topk
    meta = mla.mla_get_metadata(sl, prob.s_q, prob.h_q, 1, topk, prob.is_fp8)
    ws = torch.empty(meta.workspace_bytes, dtype=torch.uint8, device=dev)
    o = torch.empty((prob.B, prob.s_q, prob.h_q, 512), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((prob.B, prob.s_q, prob.h_q), dtype=torch.float32, device=dev)

    def step():
        m = mla.mla_get_metadata(sl, prob.s_q, prob.h_q, 1, topk, prob.is_fp8)
        mla.mla_decode_with_kvcache(q, kv, bt, sl, 512, m, idx, prob.is_fp8, prob.softmax_scale, ws, o, lse)

    def decode_only():
        mla.mla_decode_with_kvcache(q, kv, bt, sl, 512, meta, idx, prob.is_fp8, prob.softmax_scale, ws, o, lse)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    step_ms = e0.elapsed_time(e1) / steps

    # decode call alone (metadata reused, as across layers), per-launch events
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for a, b in evs:
        a.record(stream)
        decode_only()
        b.record(stream)
    torch.cuda.synchronize()
    dec = sorted(a.elapsed_time(b) for a, b in evs)
    dec_ms = sum(dec) / len(dec)
    res = dict(config=cfg, name=prob.name, gen_s=round(gen_s, 2), flops=prob.flops(), bytes=prob.bytes(),
               num_workers=meta.num_workers, step_ms=step_ms, decode_ms=dec_ms, decode_ms_median=dec[len(dec) // 2])
    if cold:
        junk = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        times = []
        for _ in range(steps):
            junk.fill_(1)
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            decode_only()
            b.record(stream)
            torch.cuda.synchronize()
            times.append(a.elapsed_time(b))
        times.sort()
        res["decode_ms_cold_median"] = times[len(times) // 2]
        del junk
    res["tflops"] = prob.flops() / (dec_ms * 1e-3) / 1e12
    res["gbps"] = prob.bytes() / (dec_ms * 1e-3) / 1e9
    res["frac_hbm"] = res["gbps"] / PEAK_HBM_GBS
    res["frac_mfma"] = res["tflops"] / PEAK_BF16_TFLOPS
    del q, kv, bt, sl, idx, ws, o, lse
    torch.cuda.empty_cache()
    return prob, res


def cpu_baseline(prob):
    """The float64 oracle on the host cores over the whole headline workload."""
    import numpy as np

    import oracle

    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    rows = None
    t0 = time.perf_counter()
    oracle.problem_decode(prob, rows)
    dt = time.perf_counter() - t0
    _ = np
    return dict(value=prob.flops() / dt / 1e12, unit="TFLOP/s", cores=threads, kind="oracle",
                sample="all %d query rows of the headline workload (%.1f GFLOP, %.1f s)" % (
                    prob.B * prob.s_q * prob.h_q, prob.flops() / 1e9, dt),
                seconds=round(dt, 2), gbps=prob.bytes() / dt / 1e9)


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py runs on one GPU only: this build has no multi-GPU path (run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    import torch

    import mla_paged_kv_get_amd as mla

    mla.lib()
    cfgs = [int(c) for c in args.configs.split(",") if c]
    if HEADLINE not in cfgs:
        cfgs = [HEADLINE] + cfgs
    results = {}
    head_prob = None
    for c in cfgs:
        prob, r = measure(c, args.steps, args.warmup, args.cold)
        results[c] = r
        print("[bench] config %d %s: decode %.1f us, %.1f TFLOP/s, %.0f GB/s (W=%d)" % (
            c, prob.name, r["decode_ms"] * 1e3, r["tflops"], r["gbps"], r["num_workers"]), file=sys.stderr, flush=True)
        if c == HEADLINE:
            head_prob = prob
    h = results[HEADLINE]
    roofline = dict(bound="hbm", achieved=round(h["gbps"], 1), peak=PEAK_HBM_GBS, unit="GB/s",
                    frac=round(h["gbps"] / PEAK_HBM_GBS, 4), traffic=None,
                    kernel="decode call (split-KV decode + combine), per-launch HIP events")
    line = dict(metric=METRIC, value=round(head_prob.flops() / (h["step_ms"] * 1e-3) / 1e12, 2), unit="TFLOP/s",
                n_gpus=1, steps=args.steps, warmup=args.warmup, ms_per_step=round(h["step_ms"], 5),
                higher_is_better=True, scaling="weak", vs_baseline=None, dtype="bf16", data="synthetic",
                config=dict(workload=head_prob.name, B=head_prob.B, s_q=head_prob.s_q, h_q=head_prob.h_q,
                            seq_len=int(head_prob.cache_seqlens[0]), block_size=64, kv="bf16"),
                hbm_gbps=round(head_prob.bytes() / (h["step_ms"] * 1e-3) / 1e9, 1),
                roofline=roofline,
                workloads={str(c): {k: (round(v, 5) if isinstance(v, float) else v) for k, v in r.items()}
                           for c, r in results.items()})
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(head_prob)
    print(json.dumps(line))


if __name__ == "__main__":
    main()
