"""Benchmark of MLA decode over a paged latent KV cache on one MI355X.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--workloads 2,3,4,5]
                [--no-cpu-baseline] [--calibrate-copy] [--prefill] [--merge]

A step is one pass of the whole decode path over one batch of synthetic input
already resident in HBM: the scheduler kernel (mla_get_metadata) and the decode
call (mla_decode_with_kvcache: the split-KV decode kernel, then the lse combine
kernel).  The headline workload is the memory-bound dense BF16 decode (B=64,
s_q=1, h_q=128, seqlen 4096 for all, block 64, pages a random permutation of
the pool); its step rate is the line's value.  By default the line also
carries, under "workloads", the compute-bound dense s_q=2 decode (3), the sparse
FP8 top-2048 decode (4) and the skewed long-context sparse FP8 decode (5),
measured the same way, each with a roofline of its own: the fraction of the
HBM peak for the memory-bound ones (2, 5: intensity below the ridge point) and
of the dense bf16 MFMA peak for the compute-bound ones (3, 4).

Counting (per decode call): FLOPs = 2 (576 + 512) per query row per attended
token; algorithmic bytes = KV bytes of the attended tokens (1152 B per bf16
token, 656 B per FP8 token) + q + o.  Peaks: 8.0 TB/s HBM, 2.5 PFLOP/s dense
bf16 MFMA.

roofline: the dominant kernel is the split-KV decode kernel; its duration is
taken per launch over the timed steps with HIP events recorded on its stream
right around it (mla_set_decode_kernel_events).  Every timed region starts
behind a short GPU spin (torch.cuda._sleep), so the host has queued the work
before the GPU reaches it and the events measure GPU time, not launch overhead.  "traffic" is the HBM bytes per
launch that rocprofv3 FETCH_SIZE + WRITE_SIZE measured for that kernel on this
workload (scaled by the same counters' reading of a plain copy of known size),
read from profiles/; it is null when the kernel sources changed since.

--calibrate-copy runs only a plain 1 GiB device-to-device copy (8 times), the
known-size reference the traffic counters are scaled by.

Prints one JSON line.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
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
KERNEL_SOURCES = ["mla_paged_kv_get_amd/csrc/mla_decode.hip", "mla_paged_kv_get_amd/csrc/mla_decode_dense.hip",
                  "mla_paged_kv_get_amd/csrc/mla_decode_fp8.hip", "mla_paged_kv_get_amd/csrc/mla_device.hpp",
                  "mla_paged_kv_get_amd/csrc/mla_common.hpp"]
# copy-calibrated FETCH_SIZE + WRITE_SIZE summaries of the decode kernel, per workload
TRAFFIC_FILES = {
    2: "traffic_mla_decode_dense_kernel_bf16_b64_h128_s4096.json",
    3: "traffic_mla_decode_dense_kernel_bf16_b128_sq2_h128_varlen.json",
    4: "traffic_mla_decode_fp8_kernel_sparse_b64_h128_topk2048.json",
    5: "traffic_mla_decode_fp8_kernel_sparse_skewed_b8_sq2_h64.json",
}
RIDGE = PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9)  # FLOP per byte


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workloads", default="2,3,4,5",
                    help="comma list of configurations; 2 (the headline) is always run")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy", action="store_true")
    ap.add_argument("--prefill", action="store_true",
                    help="also time the sparse prefill call (s_q 2048 query tokens, h_q 128, s_kv 8192, topk 2048)")
    ap.add_argument("--no-headline", action="store_true",
                    help="run only the --workloads listed (the first one is reported); for per-workload profiles")
    ap.add_argument("--merge", action="store_true",
                    help="also compare where split results are merged (combine kernel / decode kernel's last split) "
                         "on small shapes and workloads 1 and 4, with the two modes' calls alternated")
    ap.add_argument("--no-calls", action="store_true",
                    help="skip the separate warm/cold call timings (for kernel traces of the timed steps alone)")
    return ap.parse_args()


def kernel_source_sha() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(cfg: int):
    """HBM bytes per launch of the decode kernel on workload cfg, if the committed
    counter summary was taken on the current kernel sources."""
    if cfg not in TRAFFIC_FILES:
        return None
    try:
        with open(os.path.join(ROOT, "profiles", TRAFFIC_FILES[cfg])) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_sha256") != kernel_source_sha():
        return None
    return t.get("hbm_bytes_per_launch")


def calibrate_copy():
    import torch

    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda:0")
    b = torch.empty(n, dtype=torch.uint8, device="cuda:0")
    a.fill_(1)
    torch.cuda.synchronize()
    for _ in range(8):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "copies": 8}))


def measure(cfg: int, steps: int, warmup: int, calls: bool = True):
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
    stream = torch.cuda.current_stream()

    def decode_call(m):
        mla.mla_decode_with_kvcache(q, kv, bt, sl, 512, m, idx, prob.is_fp8, prob.softmax_scale, ws, o, lse)

    def step():
        decode_call(mla.mla_get_metadata(sl, prob.s_q, prob.h_q, 1, topk, prob.is_fp8, out=meta.tensor))

    def hold_gpu(us: float):
        # keep the GPU busy while the host queues the timed work behind it, so
        # events time the GPU and not the host's launch overhead
        torch.cuda._sleep(int(us * 2500))

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()

    # timed steps (scheduler + decode call); the decode kernel of each step is
    # bracketed by its own pair of HIP events on its stream
    timer = mla.DecodeKernelTimer()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    hold_gpu(400.0 * steps + 2000.0)
    e0.record(stream)
    for _ in range(steps):
        timer.record(step)
    e1.record(stream)
    torch.cuda.synchronize()
    step_ms = e0.elapsed_time(e1) / steps
    kern = sorted(timer.durations_ms())
    kernel_ms = sum(kern) / len(kern)

    # decode call alone (metadata reused, as across layers), one call per
    # iteration, alternately: the whole call (decode + combine) by an event pair
    # around it, and the decode kernel alone by the library's events (the events
    # it records between the two kernels add ~2-3 us, so calls are timed without
    # them).  Warm: back to back over
    # the same inputs.  Cold: 1 GiB read between calls (a sum over a scratch
    # buffer), so neither L2 nor the 256 MB MALL holds the KV pool and no dirty
    # lines are left to be written back inside the timed call.  cold_write: the
    # same with 1 GiB written instead (the write-back of those dirty lines then
    # lands inside the timed call).
    junk = torch.ones(1 << 28, dtype=torch.float32, device=dev) if calls else None

    def timed_calls(mode: str):
        calls_ms = []
        kt = mla.DecodeKernelTimer()
        for i in range(2 * steps):
            if mode == "cold":
                junk.sum()
            elif mode == "cold_write":
                junk.fill_(1)
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            hold_gpu(500.0)
            a.record(stream)
            if i % 2:
                kt.record(lambda: decode_call(meta))
            else:
                decode_call(meta)
            b.record(stream)
            torch.cuda.synchronize()
            if i % 2 == 0:
                calls_ms.append(a.elapsed_time(b))
        kd = sorted(kt.durations_ms())
        calls_ms.sort()
        return calls_ms[len(calls_ms) // 2], kd[len(kd) // 2]

    # (skipped with --no-calls, so that a kernel trace of the run holds only the
    # warmup and timed steps and its mean decode duration is the one reported)
    nan = (float("nan"), float("nan"))
    call_warm, kern_warm = timed_calls("warm") if calls else nan
    call_cold, kern_cold = timed_calls("cold") if calls else nan
    call_cold_w, kern_cold_w = timed_calls("cold_write") if calls else nan
    del junk
    # the scheduler kernel alone
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    hold_gpu(100.0 * steps + 2000.0)
    a.record(stream)
    for _ in range(steps):
        mla.mla_get_metadata(sl, prob.s_q, prob.h_q, 1, topk, prob.is_fp8, out=meta.tensor)
    b.record(stream)
    torch.cuda.synchronize()
    sched_ms = a.elapsed_time(b) / steps

    flops, nbytes = prob.flops(), prob.bytes()
    us = lambda ms: round(ms * 1e3, 2)
    res = dict(config=cfg, name=prob.name, gen_s=round(gen_s, 2), flops=flops, bytes=nbytes,
               intensity=round(flops / nbytes, 1), num_workers=meta.num_workers, splits=meta.total_splits(),
               step_us=us(step_ms), decode_kernel_us=us(kernel_ms),
               decode_kernel_us_median=us(kern[len(kern) // 2]),
               decode_kernel_us_warm_median=us(kern_warm), decode_kernel_us_cold_median=us(kern_cold),
               decode_kernel_us_cold_write_median=us(kern_cold_w),
               decode_call_us_warm_median=us(call_warm), decode_call_us_cold_median=us(call_cold),
               decode_call_us_cold_write_median=us(call_cold_w), scheduler_us=us(sched_ms),
               step_tflops=round(flops / (step_ms * 1e-3) / 1e12, 2),
               kernel_tflops=round(flops / (kernel_ms * 1e-3) / 1e12, 2),
               kernel_gbps=round(nbytes / (kernel_ms * 1e-3) / 1e9, 1),
               call_cold_tflops=round(flops / (call_cold * 1e-3) / 1e12, 2),
               call_cold_gbps=round(nbytes / (call_cold * 1e-3) / 1e9, 1))
    for k, v in list(res.items()):  # timings skipped with --no-calls
        if isinstance(v, float) and v != v:
            res[k] = None
    res["kernel_frac_hbm"] = round(res["kernel_gbps"] / PEAK_HBM_GBS, 4)
    res["kernel_frac_mfma"] = round(res["kernel_tflops"] / PEAK_BF16_TFLOPS, 4)
    # the roofline this workload sits under: HBM below the ridge point, MFMA above
    mem_bound = flops / nbytes < RIDGE
    res["roofline"] = dict(
        bound="hbm" if mem_bound else "mfma",
        achieved=res["kernel_gbps"] if mem_bound else res["kernel_tflops"],
        peak=PEAK_HBM_GBS if mem_bound else PEAK_BF16_TFLOPS, unit="GB/s" if mem_bound else "TFLOP/s",
        frac=res["kernel_frac_hbm"] if mem_bound else res["kernel_frac_mfma"],
        traffic=measured_traffic(cfg),
        per_launch=dict(algorithmic_bytes=nbytes, flops=flops, kernel_us=res["decode_kernel_us"]))
    if calls and topk == 0 and prob.s_q > 1:
        # speculative query tokens with the causal mask (query token s of s_q sees
        # positions <= seqlen - s_q + s): the same decode kernel, timed the same way
        ct = mla.DecodeKernelTimer()
        for _ in range(warmup):
            mla.mla_decode_with_kvcache(q, kv, bt, sl, 512, meta, idx, prob.is_fp8, prob.softmax_scale, ws, o, lse,
                                        causal=True)
        torch.cuda.synchronize()
        hold_gpu(400.0 * steps + 2000.0)
        for _ in range(steps):
            ct.record(lambda: mla.mla_decode_with_kvcache(q, kv, bt, sl, 512, meta, idx, prob.is_fp8,
                                                          prob.softmax_scale, ws, o, lse, causal=True))
        cd = ct.durations_ms()
        c_ms = sum(cd) / len(cd)
        lens = prob.cache_seqlens.tolist()
        c_flops = sum(prob.h_q * max(0, L - prob.s_q + s + 1) for L in lens for s in range(prob.s_q)) * 2 * (576 + 512)
        res["causal_decode_kernel_us"] = round(c_ms * 1e3, 2)
        res["causal_kernel_tflops"] = round(c_flops / (c_ms * 1e-3) / 1e12, 2)
    del q, kv, bt, sl, idx, ws, o, lse
    torch.cuda.empty_cache()
    return prob, res


def cpu_baseline(prob):
    """The float64 oracle (as it stands) on the host cores: all query rows of the
    headline workload."""
    import oracle

    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    cpu_model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    cpu_model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    t0 = time.perf_counter()
    oracle.problem_decode(prob, None)
    dt = time.perf_counter() - t0
    return dict(value=round(prob.flops() / dt / 1e12, 5), unit="TFLOP/s", cores=threads, kind="oracle",
                sample="all %d query rows of the headline workload (%.1f GFLOP, %.1f MB algorithmic), %.1f s" % (
                    prob.B * prob.s_q * prob.h_q, prob.flops() / 1e9, prob.bytes() / 1e6, dt),
                seconds=round(dt, 2), gbps=round(prob.bytes() / dt / 1e9, 3), cpu_model=cpu_model,
                host_cpus=os.cpu_count())


PREFILL_SHAPE = dict(s_q=2048, h_q=128, s_kv=8192, topk=2048, n_invalid=102)


def measure_prefill(steps: int, warmup: int):
    """Whole sparse prefill calls (set-up, schedule, decode path, combine) back to
    back, timed by one event pair; FLOPs = 2 (576 + 512) per row per attended token."""
    import torch

    import mla_inputs as mi
    import mla_paged_kv_get_amd as mla

    sh = PREFILL_SHAPE
    prob = mi.make_prefill_problem("sparse prefill (s_q %d, h_q %d, s_kv %d, topk %d)" % (
        sh["s_q"], sh["h_q"], sh["s_kv"], sh["topk"]), sh["s_q"], sh["h_q"], sh["s_kv"], sh["topk"], seed=7,
        n_invalid=sh["n_invalid"])
    dev = torch.device("cuda:0")
    q = prob.q[0].to(dev)
    kv = prob.kvcache.reshape(-1, 576)[:sh["s_kv"]].contiguous().to(dev)
    idx = prob.indices[0].to(dev)
    o = torch.empty((sh["s_q"], sh["h_q"], 512), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((sh["s_q"], sh["h_q"]), dtype=torch.float32, device=dev)
    need = ctypes.c_size_t(0)
    mla.lib().mla_sparse_prefill_workspace_size(sh["s_q"], sh["h_q"], 1, sh["s_kv"], sh["topk"], 0,
                                                ctypes.byref(need), None)
    ws = torch.empty(need.value, dtype=torch.uint8, device=dev)
    call = lambda: mla.mla_sparse_prefill(q, kv, idx, workspace=ws, out=o, lse=lse)
    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda._sleep(int((3000.0 * steps + 2000.0) * 2500))
    e0.record()
    for _ in range(steps):
        call()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    flops = prob.flops()
    tflops = flops / (ms * 1e-3) / 1e12
    return dict(name=prob.name, call_us=round(ms * 1e3, 1), flops=flops, tflops=round(tflops, 1),
                frac_mfma=round(tflops / PEAK_BF16_TFLOPS, 4))


MERGE_SHAPES = [
    dict(name="dense bf16 B=4 h_q=64 300 tokens", B=4, s_q=1, h_q=64, seqlens=[300] * 4),
    dict(name="dense bf16 B=8 h_q=128 512 tokens", B=8, s_q=1, h_q=128, seqlens=[512] * 8),
    dict(name="dense fp8 B=16 h_q=128 640 tokens", B=16, s_q=1, h_q=128, seqlens=[640] * 16, is_fp8=True),
    dict(name="sparse fp8 B=32 h_q=128 topk 512", B=32, s_q=1, h_q=128, seqlens=[8192] * 32, topk=512, is_fp8=True),
]


def measure_merge(rounds: int = 30, per: int = 3):
    """Decode calls with the combine kernel (MLA_MERGE_OFF) and with the decode
    kernel merging (MLA_MERGE_ON), alternated in groups of `per` calls so that
    both modes share the clock state; median call time of each (an event pair
    around each group, behind a GPU spin), and whether the outputs are
    bit-identical."""
    import torch

    import mla_inputs as mi
    import mla_paged_kv_get_amd as mla

    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    probs = [mi.config(1)]
    for sh in MERGE_SHAPES:
        c = dict(sh)
        probs.append(mi.make_problem(c.pop("name"), seed=7, **c))
    probs.append(mi.config(4))
    out = []
    for prob in probs:
        q, kv, bt, sl = prob.q.to(dev), prob.kvcache.to(dev), prob.block_table.to(dev), prob.cache_seqlens.to(dev)
        idx = None if prob.indices is None else prob.indices.to(dev)
        meta = mla.mla_get_metadata(sl, prob.s_q, prob.h_q, 1, prob.topk, prob.is_fp8)
        ws = torch.empty(meta.workspace_bytes, dtype=torch.uint8, device=dev)
        o_buf = torch.empty((prob.B, prob.s_q, prob.h_q, 512), dtype=torch.bfloat16, device=dev)
        l_buf = torch.empty((prob.B, prob.s_q, prob.h_q), dtype=torch.float32, device=dev)
        res, times = {}, {0: [], 1: []}

        def call():
            return mla.mla_decode_with_kvcache(q, kv, bt, sl, 512, meta, idx, prob.is_fp8, prob.softmax_scale, ws,
                                               o_buf, l_buf)

        try:
            for mode in (0, 1):
                mla.mla_set_merge_mode(mode)
                o, l = call()
                torch.cuda.synchronize()
                res[mode] = (o.clone(), l.clone())
            for r in range(rounds):
                for mode in ((0, 1) if r % 2 == 0 else (1, 0)):
                    mla.mla_set_merge_mode(mode)
                    torch.cuda._sleep(int(300 * per * 2500))
                    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                    e0.record(stream)
                    for _ in range(per):
                        call()
                    e1.record(stream)
                    torch.cuda.synchronize()
                    times[mode].append(e0.elapsed_time(e1) * 1e3 / per)
        finally:
            mla.mla_set_merge_mode(mla.MLA_MERGE_OFF)
        same = torch.equal(res[0][0], res[1][0]) and torch.equal(res[0][1], res[1][1])
        med = {m: sorted(t)[len(t) // 2] for m, t in times.items()}
        out.append(dict(name=prob.name, call_us_combine_kernel=round(med[0], 2), call_us_merged=round(med[1], 2),
                        splits=meta.total_splits(), bit_identical=same))
        del q, kv, bt, sl, idx, ws, o_buf, l_buf
        torch.cuda.empty_cache()
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU: the decode path here has no multi-GPU mode (run with --gpus 1)",
              file=sys.stderr)
        sys.exit(2)
    if args.calibrate_copy:
        calibrate_copy()
        return
    import torch  # noqa: F401

    import mla_paged_kv_get_amd as mla

    mla.lib()
    listed = [int(c) for c in args.workloads.split(",") if c]
    cfgs = listed if args.no_headline else [HEADLINE] + [c for c in listed if c != HEADLINE]
    head = cfgs[0]
    results = {}
    head_prob = None
    for c in cfgs:
        prob, r = measure(c, args.steps, args.warmup, calls=not args.no_calls)
        results[c] = r
        print("[bench] config %d %s: step %.1f us, decode kernel %.1f us (%.1f TFLOP/s, %.0f GB/s, %.1f %% of the %s "
              "roofline); kernel warm / cold / cold-after-writes %s / %s / %s us; call warm / cold %s / %s us; "
              "scheduler %.1f us, W=%d, %d splits" % (
                  c, prob.name, r["step_us"], r["decode_kernel_us"], r["kernel_tflops"], r["kernel_gbps"],
                  100 * r["roofline"]["frac"], r["roofline"]["bound"], r["decode_kernel_us_warm_median"],
                  r["decode_kernel_us_cold_median"], r["decode_kernel_us_cold_write_median"],
                  r["decode_call_us_warm_median"], r["decode_call_us_cold_median"], r["scheduler_us"],
                  r["num_workers"], r["splits"]), file=sys.stderr, flush=True)
        if "causal_decode_kernel_us" in r:
            print("[bench] config %d causal mask: decode kernel %.1f us (%.1f TFLOP/s)" % (
                c, r["causal_decode_kernel_us"], r["causal_kernel_tflops"]), file=sys.stderr, flush=True)
        if c == head:
            head_prob = prob
    h = results[head]
    roofline = dict(h["roofline"])
    roofline.pop("per_launch")
    kname = ("mla_decode_fp8_kernel" if head_prob.is_fp8 else
             "mla_decode_dense_kernel" if head_prob.topk == 0 else "mla_decode_kernel")
    roofline.update(kernel=kname + " (split-KV decode), mean of per-launch HIP events over the timed steps",
                    hbm_frac=h["kernel_frac_hbm"], mfma_frac=h["kernel_frac_mfma"])
    line = dict(metric=METRIC, value=h["step_tflops"], unit="TFLOP/s", n_gpus=1, steps=args.steps,
                warmup=args.warmup, ms_per_step=round(h["step_us"] / 1e3, 5), higher_is_better=True, scaling="weak",
                vs_baseline=None, dtype="bf16", data="synthetic",
                config=dict(workload=head_prob.name, B=head_prob.B, s_q=head_prob.s_q, h_q=head_prob.h_q, h_kv=1,
                            seqlen=int(head_prob.cache_seqlens[0]), block_size=64,
                            kv="fp8-656B" if head_prob.is_fp8 else "bf16", topk=head_prob.topk, d_qk=576, d_v=512),
                hbm_gbps_step=round(head_prob.bytes() / (h["step_us"] * 1e-6) / 1e9, 1),
                roofline=roofline,
                workloads={str(c): r for c, r in results.items()})
    if args.prefill:
        pf = measure_prefill(max(3, min(args.steps, 20)), 2)
        print("[bench] %s: call %.1f us (%.1f TFLOP/s, %.1f %% of MFMA peak)" % (
            pf["name"], pf["call_us"], pf["tflops"], 100 * pf["frac_mfma"]), file=sys.stderr, flush=True)
        line["workloads"]["prefill"] = pf
    if args.merge:
        mg = measure_merge()
        for m in mg:
            print("[bench] merge %s: decode call %.2f us with the combine kernel, %.2f us merged in the decode kernel "
                  "(%d splits, %s)" % (m["name"], m["call_us_combine_kernel"], m["call_us_merged"], m["splits"],
                                       "bit-identical" if m["bit_identical"] else "OUTPUTS DIFFER"),
                  file=sys.stderr, flush=True)
        line["merge"] = mg
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(head_prob)
    print(json.dumps(line))


if __name__ == "__main__":
    main()
