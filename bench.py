"""Throughput of one decode step of paged attention on one MI355X.

A step is one pass of the whole hot path over one batch: append the new
token's K/V to every cache group (paged_kv_append), then, for every logical
layer, decode attention over that layer's group cache -- work-balanced
(paged_decode_attention_balanced, which merges cut units itself) or fixed
splits (paged_decode_attention + split_context_reduce).  Single-layer
workloads have one layer and one group; the fp8 workload has 36 layers over
9 groups.  Workloads with several new tokens per sequence (draft-token
verification) write them with paged_kv_write and attend them causally
with paged_multiquery_attention.  Inputs are seeded synthetic arrays
already resident in HBM.

Prints ONE JSON line.  value = KV-read GB/s of the whole step (ideal KV
bytes 2 * sum(ctx) * Hkv * D * bytes_per_elem per layer call, times the
layers, / step time), the step time being the host wall clock over exactly
--steps steps bracketed by a device synchronisation on both sides.  The same
timed region is also measured on the device, by two HIP events recorded on
the stream the steps run on; roofline = the algorithmic bytes of one
attention call over that device span per call (the call's merge or reduce
launch included).  In the default run the line also carries the other
target workloads (8B shape, 32k-token split context with a shared prefix,
fp8 over 36 layers in 9 groups), each timed over at least 50 ms of steps,
and the plain streaming-read probe's GB/s.  cpu_baseline = the CPU oracle on
a bounded sample of the same workload, on this machine's host cores.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "achieved KV-read GB/s (% of HBM peak) + decode tokens/s, paged decode attn 1 GPU"
HBM_PEAK_GBS = 8000.0
MFMA_PEAK_TFLOPS = 2500.0    # dense bf16

DEFAULT_WORKLOAD = "llama70b_b64_ragged1k_16k_bs32"
# measured beside the headline in the default run: the 8B shape, the 32k
# split-context workload with its shared prefix, and the fp8 36-layer step
EXTRA_WORKLOADS = ("llama8b_b32_ctx4096_bs16", "llama70b_b4_ctx32k_split512_prefix2k",
                   "fp8_36layers_groups4_b32_ctx2k_8k")
MIN_TIMED_S = 0.05           # timed device work of each secondary workload


def _args():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    # steady state: a short loop (50 steps, ~18 ms of device work) reads the
    # clocks still ramping (fp8 70B batch 5.79 TB/s over 50 steps, 6.29 over
    # 2000; steps timed one by one read the same 186 us either way)
    p.add_argument("--steps", type=int, default=1000)
    p.add_argument("--warmup", type=int, default=100)
    p.add_argument("--workload", default=DEFAULT_WORKLOAD)
    p.add_argument("--mode", default="auto",
                   choices=["auto", "balanced", "split", "single", "multiquery", "swap",
                            "blockmanager", "stream"],
                   help="attention schedule: work-balanced, fixed splits + reduce, or one "
                        "wave per (sequence, kv head); auto = the workload's own split size "
                        "if it has one, multiquery if it has several new tokens per "
                        "sequence, else balanced; swap = whole-block moves of preempted "
                        "sequences to pinned host memory and back; blockmanager = host cost "
                        "of the C++ block manager on a serving trace; stream = the plain "
                        "streaming-read probe (4 GiB)")
    p.add_argument("--kv-format", default=None,
                   choices=["bf16", "fp8", "fp8_head", "fp8_tensor", "int8"],
                   help="cache format (default: the workload's own); fp8 = one scale per "
                        "block and kv head, fp8_head / fp8_tensor = one per kv head / per "
                        "cache, int8 = per-block asymmetric scale and zero point")
    p.add_argument("--preempt", type=int, default=8,
                   help="sequences swapped out and back in (--mode swap)")
    p.add_argument("--split", type=int, default=None, help="split_tokens for --mode split")
    p.add_argument("--unfused", action="store_true",
                   help="append with paged_kv_append in its own launch instead of inside "
                        "the attention launch of each cache group's first layer")
    p.add_argument("--cold-steps", type=int, default=20,
                   help="extra event-timed steps, each after a 1 GiB write that evicts the "
                        "MALL and the L2s (cold_cache in the JSON line; 0 = skip)")
    p.add_argument("--cpu-seconds", type=float, default=24.0,
                   help="target time of the single-threaded oracle baseline (3 runs)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-extra", action="store_true",
                   help="headline workload only (skip the other workloads and the probe)")
    p.add_argument("--calibrate-copy", action="store_true",
                   help="also run a plain 1 GiB device copy (counter calibration)")
    p.add_argument("--traffic-json", default=os.path.join(ROOT, "profiles", "traffic.json"),
                   help="measured HBM bytes per attention launch (written from rocprofv3)")
    return p.parse_args()


def main():
    a = _args()
    if a.gpus != 1:
        print(f"bench.py: measures one GPU only (asked for --gpus {a.gpus}); "
              "the decode kernel has no multi-GPU path.", file=sys.stderr)
        sys.exit(2)
    from synthetic import make_workload

    if a.mode == "stream":
        return print(json.dumps(_bench_stream(a)), flush=True)
    wl = make_workload(a.workload)
    if a.mode == "swap":
        return _bench_swap(a, wl)
    if a.mode == "blockmanager":
        return _bench_block_manager(a)
    res = _run_workload(a, wl, a.mode, a.steps, a.warmup, a.cold_steps,
                        cpu=not a.no_cpu_baseline, headline=True)
    if a.workload == DEFAULT_WORKLOAD and a.mode == "auto" and not a.no_extra:
        # the other target workloads, each timed over enough steps that the
        # start and end of the timed region do not matter
        res["configs"] = {}
        for name in EXTRA_WORKLOADS:
            print(f"bench: {name}", file=sys.stderr, flush=True)
            res["configs"][name] = _run_workload(a, make_workload(name), "auto", None,
                                                 a.warmup, a.cold_steps, cpu=False,
                                                 headline=False)
        res["hbm_stream_read"] = _bench_stream(a, summary=True)
    print(json.dumps(res), flush=True)


def _check_tables(tables, lens, block_size, num_blocks):
    """The preconditions the kernels rely on (they are not checked on the
    device): every sequence fits its table row and its live entries name
    blocks of the pool."""
    import numpy as np

    nblk = (lens.astype(np.int64) + block_size - 1) // block_size
    live = np.arange(tables.shape[1])[None, :] < nblk[:, None]
    ok = (lens >= 0).all() and (nblk <= tables.shape[1]).all() and \
        (((tables >= 0) & (tables < num_blocks)) | ~live).all()
    if not ok:
        raise SystemExit("bench.py: generated block tables break the kernel preconditions")


def _timed(step, steps, warmup):
    """warmup untimed steps, then `steps` steps bracketed by a device
    synchronisation on both sides: host wall clock, and the device span
    between two HIP events recorded on the stream the steps run on."""
    import torch

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    for _ in range(steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return wall, e0.elapsed_time(e1) * 1e-3


def _run_workload(a, wl, mode_arg, steps, warmup, cold_steps, cpu, headline):
    import numpy as np
    import torch

    import paged_kv_cache_273_amd as pkv
    from synthetic import generate, generate_multiquery

    multi = wl.q_uniform != (1, 1)
    mode = mode_arg
    if mode == "auto":
        mode = "multiquery" if multi else ("split" if wl.split_tokens > 0 else "balanced")
    if (mode == "multiquery") != multi:
        print(f"bench.py: mode {mode} does not fit workload {wl.name}", file=sys.stderr)
        sys.exit(2)
    S = 0
    if mode == "split":
        S = a.split if (a.split is not None and headline) else (wl.split_tokens or 512)
    dev = torch.device("cuda:0")
    t_gen = time.time()
    mq = generate_multiquery(wl) if multi else None
    inp = mq.base if multi else generate(wl)   # every cache group of the workload
    print(f"bench: generated {wl.name} in {time.time() - t_gen:.1f} s", file=sys.stderr,
          flush=True)
    _check_tables(inp.block_tables, inp.context_lens, wl.block_size, inp.num_blocks)

    def up(x):
        x = np.ascontiguousarray(x)
        if x.dtype == np.uint16:
            x = x.view(np.int16)
        return torch.from_numpy(x).to(dev)

    live = torch.from_numpy(np.arange(wl.block_size)[None, :] < inp.live[:, None]).to(dev)

    fmt = (a.kv_format if headline else None) or wl.kv_dtype
    ebytes = 2 if fmt == "bf16" else 1

    def quant(src):
        # 1-byte cache built on the device from the bf16 source values (input
        # preparation only): fp8 scale = amax / 448 per block and kv head,
        # per kv head or per cache; int8 = asymmetric (min, max) per block
        # and kv head
        x = up(src).view(torch.bfloat16).float()
        ok = live[:, :, None, None] & torch.isfinite(x)
        if fmt == "int8":
            lo = torch.where(ok, x, torch.full_like(x, float("inf"))).amin(dim=(1, 3))
            hi = torch.where(ok, x, torch.full_like(x, float("-inf"))).amax(dim=(1, 3))
            spread = hi > lo
            sc = torch.where(spread, (hi - lo) / 255.0, torch.ones_like(hi))
            zp = torch.where(spread, torch.round(-lo / sc).clamp(0, 255), torch.zeros_like(hi))
            u = (torch.round(x / sc[:, None, :, None]) + zp[:, None, :, None]).clamp(0, 255)
            u = torch.nan_to_num(u, nan=0.0)
            return u.to(torch.uint8).contiguous(), torch.stack([sc, zp], -1).float().contiguous()
        xm = torch.where(ok, x.abs(), torch.zeros_like(x))
        if fmt == "fp8":
            amax = xm.amax(dim=(1, 3))
        elif fmt == "fp8_head":
            amax = xm.amax(dim=(0, 1, 3))
        else:
            amax = xm.amax().reshape(1)
        sc = torch.where(amax > 0, amax / 448.0, torch.ones_like(amax)).float()
        if fmt == "fp8":
            y = x / sc[:, None, :, None]
        elif fmt == "fp8_head":
            y = x / sc[None, None, :, None]
        else:
            y = x / sc
        y = y.clamp(-448, 448)
        return y.to(torch.float8_e4m3fn).view(torch.uint8).contiguous(), sc.contiguous()

    # one cache per layer group ([A] cross-layer KV sharing: layer l reads
    # group l // layers_per_group); bf16 workloads have a single group
    caches = []
    for g in range(wl.groups):
        if fmt != "bf16":
            k, ks = quant(inp.k_pool[g])
            v, vs = quant(inp.v_pool[g])
        else:
            k, v, ks, vs = up(inp.k_pool[g]), up(inp.v_pool[g]), None, None
        if multi:
            caches.append((k, v, ks, vs, up(mq.k_rows[g]), up(mq.v_rows[g])))
        else:
            caches.append((k, v, ks, vs, up(inp.k_new[g]), up(inp.v_new[g])))
    qs = [up((mq if multi else inp).query[l]) for l in range(wl.layers)]
    rows = mq.rows if multi else wl.B
    if multi:
        qstart = up(mq.query_start)
        max_q = int(mq.query_lens.max())
    bt, cl = up(inp.block_tables), up(inp.context_lens)
    ctx = inp.context_lens.astype(np.int64)
    per_layer = 2 * int(ctx.sum()) * wl.Hkv * wl.D * ebytes
    ideal = per_layer * wl.layers
    scale = float(inp.scale)

    ms = pkv.max_splits_for(int(ctx.max()), S) if S else 1
    out = torch.empty((rows, wl.Hq, wl.D), dtype=torch.float32, device=dev)
    po = torch.empty((wl.B, wl.Hq, ms, wl.D), dtype=torch.float32, device=dev) if S else None
    pl = torch.empty((wl.B, wl.Hq, ms), dtype=torch.float32, device=dev) if S else None
    ws = pkv.make_workspace(qs[0], caches[0][0], kv_dtype=fmt) if mode == "balanced" else None
    if mode == "multiquery":
        ws = pkv.make_multiquery_workspace(qs[0], caches[0][0], max_q, kv_dtype=fmt)

    # decode steps append in the attention launch of each group's first
    # layer (paged_append_decode_attention*), unless --unfused
    fused = not multi and not (a.unfused and headline)

    def step():
        for k, v, ks, vs, kn, vn in caches:
            if multi:
                pkv.paged_kv_write(kn, vn, qstart, k, v, bt, cl, max_q, k_scale=ks, v_scale=vs,
                                   kv_dtype=fmt)
            elif not fused:
                pkv.paged_kv_append(kn, vn, k, v, bt, cl, k_scale=ks, v_scale=vs, kv_dtype=fmt)
        for layer in range(wl.layers):
            k, v, ks, vs, kn, vn = caches[layer // wl.layers_per_group]
            q = qs[layer]
            new = fused and layer % wl.layers_per_group == 0
            if mode == "split" and new:
                pkv.paged_append_decode_attention(q, kn, vn, k, v, bt, cl, scale,
                                                  split_tokens=S, partial_out=po,
                                                  partial_lse=pl, k_scale=ks, v_scale=vs,
                                                  kv_dtype=fmt)
            elif mode == "split":
                pkv.paged_decode_attention(q, k, v, bt, cl, scale, split_tokens=S,
                                           partial_out=po, partial_lse=pl, k_scale=ks,
                                           v_scale=vs, kv_dtype=fmt)
            elif mode == "balanced" and new:
                pkv.paged_append_decode_attention_balanced(q, kn, vn, k, v, bt, cl, scale,
                                                           workspace=ws, out=out, k_scale=ks,
                                                           v_scale=vs, kv_dtype=fmt)
            elif mode == "balanced":
                pkv.paged_decode_attention_balanced(q, k, v, bt, cl, scale, workspace=ws,
                                                    out=out, k_scale=ks, v_scale=vs,
                                                    kv_dtype=fmt)
            elif mode == "single" and new:
                pkv.paged_append_decode_attention(q, kn, vn, k, v, bt, cl, scale, out=out,
                                                  k_scale=ks, v_scale=vs, kv_dtype=fmt)
            elif mode == "multiquery":
                pkv.paged_multiquery_attention(q, qstart, k, v, bt, cl, scale, max_q,
                                               workspace=ws, out=out, k_scale=ks, v_scale=vs,
                                               kv_dtype=fmt)
            else:
                pkv.paged_decode_attention(q, k, v, bt, cl, scale, out=out, k_scale=ks,
                                           v_scale=vs, kv_dtype=fmt)
            if mode == "split":
                pkv.split_context_reduce(po, pl, cl, S, out=out)

    if a.calibrate_copy and headline:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    if steps is None:
        # secondary workloads: enough steps for MIN_TIMED_S of device time
        _, est = _timed(step, 5, warmup)
        steps = max(a.steps, int(math.ceil(MIN_TIMED_S / max(est / 5, 1e-6))))
        warmup = 0
    wall, span = _timed(step, steps, warmup)
    step_s = wall / steps
    dev_step_s = span / steps
    call_s = dev_step_s / wl.layers           # one attention call (+ its merge / reduce)
    gbs = ideal / step_s / 1e9
    kern_gbs = per_layer / call_s / 1e9
    cold = _cold_steps(step, cold_steps, ideal, dev) if cold_steps > 0 else None
    # algorithmic flops of one attention call: q.k and p.v, 2 per multiply-add,
    # per (row or sequence, query head, visible token, head-dim element)
    if multi:
        qn = mq.query_lens.astype(np.int64)
        visible = int((qn * (ctx - qn) + qn * (qn + 1) // 2).sum())
    else:
        visible = int(ctx.sum())
    flops = 4 * wl.Hq * wl.D * visible
    mfma_bound = flops / per_layer > MFMA_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)
    kern_tflops = flops / call_s / 1e12
    key = f"{wl.name}:{mode}" + (f":{fmt}" if fmt != wl.kv_dtype else "")
    traffic = _measured_traffic(a.traffic_json, key)
    kernel = {"split": "decode_kernel (split) + reduce_kernel", "single": "decode_kernel",
              "balanced": "decode_balanced_kernel + balanced_merge_kernel",
              "multiquery": ("prefill_kernel" if mfma_bound else
                             "decode_balanced_kernel (causal columns) + balanced_merge_kernel")
              }[mode]
    step_desc = ({"split": "paged_append_decode_attention(split) + split_context_reduce",
                  "balanced": "paged_append_decode_attention_balanced (append + decode, "
                              "then log-sum-exp merge of cut units)",
                  "single": "paged_append_decode_attention"} if fused else {
                 "split": "paged_kv_append + paged_decode_attention(split) + "
                          "split_context_reduce",
                 "balanced": "paged_kv_append + paged_decode_attention_balanced "
                             "(decode + log-sum-exp merge of cut units)",
                 "single": "paged_kv_append + paged_decode_attention",
                 "multiquery": "paged_kv_write + paged_multiquery_attention (causal, "
                               "log-sum-exp merge of cut units)"})[mode]
    roofline = ({
        "bound": "mfma", "kernel": kernel,
        "achieved": round(kern_tflops, 1), "peak": MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
        "frac": round(kern_tflops / MFMA_PEAK_TFLOPS, 4), "traffic": traffic,
        "launch_us": round(call_s * 1e6, 2), "algorithmic_flops_per_launch": flops,
        "algorithmic_bytes_per_launch": per_layer,
    } if mfma_bound else {
        "bound": "hbm", "kernel": kernel,
        "achieved": round(kern_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
        "frac": round(kern_gbs / HBM_PEAK_GBS, 4), "traffic": traffic,
        "launch_us": round(call_s * 1e6, 2), "algorithmic_bytes_per_launch": per_layer,
    })
    if not headline:
        res = {
            "schedule": mode, "kv_dtype": fmt, "split_tokens": S, "layers_per_step": wl.layers,
            "steps": steps, "ms_per_step": round(step_s * 1e3, 4),
            "device_ms_per_step": round(dev_step_s * 1e3, 4), "gbs": round(gbs, 1),
            "pct_of_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
            "decode_tokens_per_s": round(wl.B / step_s, 1),
            "ideal_kv_bytes_per_step": ideal, "step": step_desc, "roofline": roofline,
            "traffic_over_algorithmic": (round(traffic / per_layer, 4) if traffic else None),
            "cold_cache": cold,
        }
        del caches, qs, out, po, pl, ws
        torch.cuda.empty_cache()
        return res

    cpu_res = None
    if cpu:
        cpu_res = _cpu_baseline(inp, wl, a.cpu_seconds, mq, fmt)

    return {
        "metric": METRIC,
        "value": round(gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(step_s * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": fmt,
        "data": "synthetic",
        "pct_of_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
        "decode_tokens_per_s": round(wl.B / step_s, 1),
        "new_tokens_per_s": round(rows / step_s, 1),
        "device_ms_per_step": round(dev_step_s * 1e3, 4),
        "config": {
            "workload": wl.name, "batch": wl.B, "Hq": wl.Hq, "Hkv": wl.Hkv, "head_dim": wl.D,
            "block_size": wl.block_size, "kv_dtype": fmt,
            "ctx_sum": int(ctx.sum()), "ctx_mean": round(float(ctx.mean()), 1),
            "ctx_min": int(ctx.min()), "ctx_max": int(ctx.max()), "schedule": mode,
            "split_tokens": S, "num_blocks": inp.num_blocks, "ideal_kv_bytes_per_step": ideal,
            "layers_per_step": wl.layers, "cache_groups": wl.groups,
            "new_tokens_per_sequence": (list(wl.q_uniform) if multi else 1),
            "new_tokens_per_step": rows,
            "step": step_desc,
        },
        "roofline": roofline,
        "attention_tflops": round(kern_tflops, 2),
        "cold_cache": cold,
        "cpu_baseline": cpu_res,
    }


def _cold_steps(step, n, ideal, dev):
    """Whole steps timed one by one with a HIP event pair, each after a
    1 GiB write on the same stream that evicts the 256 MB MALL and the L2s
    (no K/V byte of the previous step is left in a cache).  The same
    event-timed measurement of back-to-back steps without the write is
    reported beside it: the event pair's own marker packets are in both."""
    import torch

    flush = torch.empty(1 << 30, dtype=torch.uint8, device=dev)

    def timed(evict):
        pairs = []
        for i in range(n):
            if evict:
                flush.fill_(i & 0xFF)
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            step()
            e1.record()
            pairs.append((e0, e1))
        torch.cuda.synchronize()
        us = sorted(e0.elapsed_time(e1) * 1e3 for e0, e1 in pairs)
        return us[len(us) // 2], us[len(us) // 10], us[min(len(us) - 1, (9 * len(us)) // 10)]

    cold_med, cold_p10, cold_p90 = timed(True)
    warm_med, _, _ = timed(False)
    del flush
    return {
        "flush_bytes": 1 << 30, "steps": n,
        "step_us_median": round(cold_med, 2), "step_us_p10": round(cold_p10, 2),
        "step_us_p90": round(cold_p90, 2),
        "gbs_median": round(ideal / (cold_med * 1e-6) / 1e9, 1),
        "frac_median": round(ideal / (cold_med * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
        "warm_step_us_median_same_timing": round(warm_med, 2),
    }


STREAM_BYTES = 1 << 32        # 4 GiB: 16x the MALL, so the probe reads HBM


def _bench_stream(a, summary=False):
    """The plain streaming-read probe (pkv_stream_read): a 4 GiB buffer read
    once per launch by 1024 / 2048 / 4096 waves, each a contiguous chunk of
    16-byte non-temporal loads; launches back to back, timed with one HIP
    event pair around 10 of them after 3 untimed ones."""
    import torch

    import paged_kv_cache_273_amd as pkv

    dev = torch.device("cuda:0")
    buf = torch.empty(STREAM_BYTES, dtype=torch.uint8, device=dev)
    buf.fill_(1)
    sink = torch.zeros(64, dtype=torch.int32, device=dev)
    out = {}
    for waves in (1024, 2048, 4096):
        run = lambda: pkv.pkv_stream_read(buf, waves, sink)   # noqa: E731
        for _ in range(3):
            run()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(10):
            run()
        e1.record()
        torch.cuda.synchronize()
        t = e0.elapsed_time(e1) * 1e-3 / 10
        out[str(waves)] = round(STREAM_BYTES / t / 1e9, 1)
    del buf
    torch.cuda.empty_cache()
    best = max(out.values())
    res = {"bytes": STREAM_BYTES, "gbs_by_waves": out, "best_gbs": best,
           "best_frac_of_peak": round(best / HBM_PEAK_GBS, 4),
           "probe": "pkv_stream_read: each wave one contiguous chunk, 16-byte non-temporal "
                    "loads, 8 per lane in flight"}
    if summary:
        return res
    return {"metric": "streaming-read GB/s of a plain HIP probe (4 GiB)", "value": best,
            "unit": "GB/s", "n_gpus": 1, "steps": 10, "warmup": 3,
            "ms_per_step": round(STREAM_BYTES / best / 1e6, 4), "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": "u8", "data": "synthetic",
            "config": {"workload": "stream read, 4 GiB"}, **res,
            "roofline": {"bound": "hbm", "kernel": "stream_read_kernel", "achieved": best,
                         "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(best / HBM_PEAK_GBS, 4), "traffic": None},
            "cpu_baseline": None}


HOST_LINK_GBS = 64.0     # PCIe 5.0 x16, one direction


def _bench_swap(a, wl):
    """Preemption by swapping ([C] "When the cache fills"): the blocks of
    --preempt sequences are gathered into pinned host memory and scattered
    back into freshly chosen blocks of the pool; and the same gather into
    device memory (the HBM-bound form used for copy-on-write)."""
    import numpy as np
    import torch

    import paged_kv_cache_273_amd as pkv
    from synthetic import generate

    dev = torch.device("cuda:0")
    inp = generate(wl, groups=[])
    nb = inp.num_blocks
    g = torch.Generator(device=dev)
    g.manual_seed(1)
    k = torch.randn((nb, wl.block_size, wl.Hkv, wl.D), device=dev, generator=g).to(
        torch.bfloat16).view(torch.int16)
    v = torch.randn((nb, wl.block_size, wl.Hkv, wl.D), device=dev, generator=g).to(
        torch.bfloat16).view(torch.int16)
    P = min(a.preempt, wl.B)
    nblk = (inp.context_lens[:P].astype(np.int64) + wl.block_size - 1) // wl.block_size
    ids = np.concatenate([inp.block_tables[b, :nblk[b]] for b in range(P)]).astype(np.int32)
    n = ids.size
    block_bytes = wl.block_size * wl.Hkv * wl.D * 2
    moved = 2 * n * block_bytes                                  # K and V
    ids_d = torch.from_numpy(ids).to(dev)
    back = torch.from_numpy(np.random.default_rng(2).permutation(ids)).to(dev)
    host_k = torch.empty((n,) + k.shape[1:], dtype=k.dtype).pin_memory()
    host_v = torch.empty_like(host_k).pin_memory()
    dev_k = torch.empty((n,) + k.shape[1:], dtype=k.dtype, device=dev)
    dev_v = torch.empty_like(dev_k)

    def timed(fn):
        for _ in range(max(1, a.warmup)):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(a.steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e-3 / a.steps

    t_out = timed(lambda: pkv.paged_kv_gather_blocks(k, v, ids_d, host_k, host_v))
    t_in = timed(lambda: pkv.paged_kv_scatter_blocks(host_k, host_v, back, k, v))
    t_dev = timed(lambda: pkv.paged_kv_gather_blocks(k, v, ids_d, dev_k, dev_v))
    out_gbs, in_gbs = moved / t_out / 1e9, moved / t_in / 1e9
    dev_gbs = 2 * moved / t_dev / 1e9                           # read + write of HBM
    res = {
        "metric": "KV swap GB/s (blocks of preempted sequences, device <-> pinned host)",
        "value": round(moved * 2 / (t_out + t_in) / 1e9, 2), "unit": "GB/s", "n_gpus": 1,
        "steps": a.steps, "warmup": a.warmup, "ms_per_step": round((t_out + t_in) * 1e3, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "preempted_sequences": P, "blocks": n,
                   "block_bytes": block_bytes, "bytes_each_way": moved,
                   "step": "paged_kv_gather_blocks to pinned host + paged_kv_scatter_blocks "
                           "back into permuted blocks"},
        "swap_out_gbs": round(out_gbs, 2), "swap_in_gbs": round(in_gbs, 2),
        "roofline": {"bound": "host link", "kernel": "move_blocks_kernel (device <-> host)",
                     "achieved": round(max(out_gbs, in_gbs), 2), "peak": HOST_LINK_GBS,
                     "unit": "GB/s", "frac": round(max(out_gbs, in_gbs) / HOST_LINK_GBS, 4),
                     "traffic": None},
        "device_gather": {"bound": "hbm", "achieved": round(dev_gbs, 1),
                          "peak": HBM_PEAK_GBS, "unit": "GB/s",
                          "frac": round(dev_gbs / HBM_PEAK_GBS, 4),
                          "launch_us": round(t_dev * 1e6, 2),
                          "algorithmic_bytes_per_launch": 2 * moved},
        "cpu_baseline": None,
    }
    print(json.dumps(res), flush=True)


def _serving_trace(seed, n_requests, prompt_system, user_len, decode_steps, batch):
    """A seeded request stream in the shape of [B] "Prefix Caching": most
    requests open with one of a few 500-token system prompts."""
    import numpy as np

    rng = np.random.default_rng(seed)
    systems = [list(rng.integers(0, 32000, prompt_system)) for _ in range(4)]
    reqs = []
    for r in range(n_requests):
        sysp = systems[rng.integers(0, 4)] if rng.random() < 0.8 else \
            list(rng.integers(0, 32000, prompt_system))
        user = list(rng.integers(0, 32000, int(rng.integers(user_len // 2, user_len * 2))))
        gen = [int(x) for x in rng.integers(0, 32000, decode_steps)]
        reqs.append((np.asarray(sysp + user, dtype=np.int32), gen))
    return reqs


def _run_trace(mgr_add, mgr_append, mgr_release, mgr_export, reqs, batch):
    """Continuous batching ([B] "Continuous Batching"): up to `batch` live
    sequences; each iteration appends one token to each, exports the
    tables, retires finished ones and admits waiting ones."""
    live, nxt, cached, prompt = {}, 0, 0, 0
    steps = 0
    while nxt < len(reqs) or live:
        while len(live) < batch and nxt < len(reqs):
            toks, gen = reqs[nxt]
            cached += mgr_add(nxt, toks)
            prompt += len(toks)
            live[nxt] = list(gen)
            nxt += 1
        seqs = list(live)
        mgr_append(seqs, [live[s].pop() for s in seqs])
        mgr_export(seqs)
        steps += 1
        for s in [s for s, g in live.items() if not g]:
            mgr_release(s)
            del live[s]
    return steps, cached, prompt


def _bench_block_manager(a):
    """Host cost of the C++ block manager on a serving trace (admission with
    prefix lookup, one append per live sequence per step, table export),
    and the same trace through the Python reference model."""
    import numpy as np

    from paged_kv_cache_273_amd.block_manager import BlockManager

    bs, nb, batch, width = 16, 65536, 64, 128
    reqs = _serving_trace(273, 512, 500, 200, 64, batch)
    bm = BlockManager(nb, bs)

    def append_all(seqs, toks):          # one token per live sequence, one call
        bm.append_batch(seqs, np.arange(len(seqs) + 1, dtype=np.int32), toks)

    t0 = time.perf_counter()
    steps, cached, prompt = _run_trace(bm.add, append_all, bm.release,
                                       lambda seqs: bm.export(seqs, width), reqs, batch)
    el = time.perf_counter() - t0
    st = bm.stats()
    cpu = None
    if not a.no_cpu_baseline:
        import oracle.block_manager as ref

        m = ref.RefBlockManager(nb, bs)

        def export(seqs):
            return [m.table(s) for s in seqs]

        def ref_append(seqs, toks):
            for s_, t_ in zip(seqs, toks):
                m.append(s_, [t_])

        sub = reqs[:96]
        t1 = time.perf_counter()
        rsteps, _, _ = _run_trace(m.add, ref_append, m.release, export, sub, batch)
        rel = time.perf_counter() - t1
        cpu = {"value": round(rel / rsteps * 1e6, 1), "unit": "us per step", "cores": 1,
               "kind": "oracle",
               "sample": f"first 96 of 512 requests ({rsteps} steps), Python reference model"}
    res = {
        "metric": "host block-manager us per decode step (64 live sequences, prefix cache)",
        "value": round(el / steps * 1e6, 2), "unit": "us per step", "n_gpus": 1,
        "steps": steps, "warmup": 0, "ms_per_step": round(el / steps * 1e3, 5),
        "higher_is_better": False, "scaling": "weak", "vs_baseline": None, "dtype": "int32",
        "data": "synthetic",
        "config": {"workload": "serving trace: 512 requests, 80% open with one of 4 "
                               "500-token system prompts, user 100-400 tokens, 64 decode "
                               "tokens, batch 64, block 16, 65536 blocks",
                   "prompt_tokens": prompt, "cached_prompt_tokens": cached,
                   "prefix_hit_rate": round(cached / prompt, 4),
                   "prompt_block_hits": st["prompt_block_hits"],
                   "prompt_block_lookups": st["prompt_block_lookups"]},
        "total_host_seconds": round(el, 4),
        "cpu_baseline": cpu,
    }
    print(json.dumps(res), flush=True)


def _measured_traffic(path, key):
    """HBM bytes per attention launch from the rocprofv3 FETCH_SIZE /
    WRITE_SIZE passes recorded in profiles/traffic.json, or None when there
    is no record or the kernel's source file has changed since it was taken."""
    import hashlib

    try:
        rec = json.load(open(path)).get(key)
    except (OSError, ValueError):
        return None
    if not rec or not rec.get("source_file"):
        return None
    src = os.path.join(ROOT, rec["source_file"])
    try:
        sha = hashlib.sha256(open(src, "rb").read()).hexdigest()
    except OSError:
        return None
    if rec.get("source_sha256") != sha:
        return None
    return rec.get("hbm_bytes_per_launch")


def _oracle_cache(oracle, kp, vp, inp, wl, fmt):
    """Host caches of format fmt built by the oracle's own encoder."""
    if fmt == "bf16":
        return kp.copy(), vp.copy(), None, None
    args = (inp.block_tables, inp.context_lens, wl.block_size)
    if fmt == "int8":
        ks = oracle.int8_block_params(kp, *args)
        vs = oracle.int8_block_params(vp, *args)
    elif fmt == "fp8":
        ks = oracle.fp8_block_scales(kp, *args)
        vs = oracle.fp8_block_scales(vp, *args)
    else:
        ks = oracle.fp8_wide_scales(kp, *args, per_tensor=(fmt == "fp8_tensor"))
        vs = oracle.fp8_wide_scales(vp, *args, per_tensor=(fmt == "fp8_tensor"))
    return oracle.quantize_pool(kp, ks, fmt), oracle.quantize_pool(vp, vs, fmt), ks, vs


def _host_threads():
    """Host threads this process may use (its CPU affinity), at most 16: the
    share of host cores that comes with one GPU."""
    try:
        n = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _cpu_baseline(inp, wl, target_s, mq=None, fmt="bf16"):
    """The oracle (plain C, fp64) on whole sequences of the same workload:
    single-threaded on a sample of about target_s / 3 seconds, and with one
    host thread per sequence at a time on every host thread this process may
    use, on as many sequences as that takes; each the median of 3 runs of
    the same sample.  GB/s on the same ideal-byte formula; generation and
    cache preparation are not timed."""
    import concurrent.futures as cf

    import numpy as np

    import oracle

    multi = mq is not None
    base = mq.base if multi else inp
    kp, vp, ks, vs = _oracle_cache(oracle, base.k_pool[0], base.v_pool[0], base, wl, fmt)
    if multi:
        oracle.write_tokens(mq.k_rows[0], mq.v_rows[0], mq.query_start, kp, vp,
                            base.block_tables, base.context_lens, wl.block_size, kv_dtype=fmt,
                            k_scale=ks, v_scale=vs)
    else:
        oracle.append(base.k_new[0], base.v_new[0], kp, vp, base.block_tables,
                      base.context_lens, wl.block_size, kv_dtype=fmt, k_scale=ks, v_scale=vs)
    ebytes = 2 if fmt == "bf16" else 1
    seq_bytes = [2 * int(base.context_lens[b]) * wl.Hkv * wl.D * ebytes for b in range(wl.B)]
    kw = dict(block_size=wl.block_size, Hkv=wl.Hkv, kv_dtype=fmt, k_scale=ks, v_scale=vs)

    def one(b):
        bt = np.ascontiguousarray(base.block_tables[b:b + 1])
        cl = np.ascontiguousarray(base.context_lens[b:b + 1])
        if multi:
            r0, r1 = int(mq.query_start[b]), int(mq.query_start[b + 1])
            oracle.multiquery_attention(np.ascontiguousarray(mq.query[0][r0:r1]),
                                        np.array([0, r1 - r0], dtype=np.int32), kp, vp, bt, cl,
                                        base.scale, **kw)
        else:
            oracle.paged_attention(np.ascontiguousarray(base.query[0][b:b + 1]), kp, vp, bt,
                                   cl, base.scale, **kw)

    # single thread: the first sequences, up to about target_s / 3 per run
    t0 = time.perf_counter()
    n1 = 0
    while n1 < wl.B and (n1 == 0 or time.perf_counter() - t0 < target_s / 3):
        one(n1)
        n1 += 1
    runs1 = [time.perf_counter() - t0]
    for _ in range(2):
        t0 = time.perf_counter()
        for b in range(n1):
            one(b)
        runs1.append(time.perf_counter() - t0)
    single = sum(seq_bytes[:n1]) / sorted(runs1)[1] / 1e9

    # every host thread, one sequence each at a time, over about as much
    # work per thread as the single-threaded sample
    threads = _host_threads()
    nm = min(wl.B, n1 * threads)
    runs = []
    with cf.ThreadPoolExecutor(threads) as ex:      # ctypes releases the GIL
        for _ in range(3):
            t0 = time.perf_counter()
            list(ex.map(one, range(nm)))
            runs.append(time.perf_counter() - t0)
    multi_gbs = sum(seq_bytes[:nm]) / sorted(runs)[1] / 1e9
    what = "sequences" + (f" ({int(mq.query_start[nm])} new tokens)" if multi else "")
    return {"value": round(multi_gbs, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": f"first {nm} of {wl.B} {what}, all {wl.Hq} query heads, "
                      f"{sum(seq_bytes[:nm]) / 1e6:.0f} MB of KV, one sequence per host "
                      f"thread at a time on {threads} threads, median of 3 runs "
                      f"({', '.join(f'{r:.2f}' for r in runs)} s); fp64 C",
            "single_thread": {"value": round(single, 4), "unit": "GB/s", "cores": 1,
                              "sample": f"first {n1} {what}, "
                                        f"{sum(seq_bytes[:n1]) / 1e6:.0f} MB of KV, median "
                                        f"of 3 runs ({', '.join(f'{r:.2f}' for r in runs1)} s)"},
            "cpu_model": _cpu_model(), "host_threads_available": threads}


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


if __name__ == "__main__":
    main()
