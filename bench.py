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
layers, / step time).  roofline = one attention call, timed with HIP events
on the stream it is launched on.  cpu_baseline = the CPU oracle on a bounded
sample of the same workload, on this machine's host cores.
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

DEFAULT_WORKLOAD = "llama70b_b64_ragged1k_16k_bs32"


def _args():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--workload", default=DEFAULT_WORKLOAD)
    p.add_argument("--mode", default="auto",
                   choices=["auto", "balanced", "split", "single", "multiquery"],
                   help="attention schedule: work-balanced, fixed splits + reduce, or one "
                        "wave per (sequence, kv head); auto = the workload's own split size "
                        "if it has one, multiquery if it has several new tokens per "
                        "sequence, else balanced")
    p.add_argument("--split", type=int, default=None, help="split_tokens for --mode split")
    p.add_argument("--cpu-seconds", type=float, default=12.0,
                   help="target CPU time of the oracle baseline sample")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--calibrate-copy", action="store_true",
                   help="also run a plain 1 GiB device copy (counter calibration)")
    p.add_argument("--traffic-json", default=os.path.join(ROOT, "profiles", "traffic.json"),
                   help="measured HBM bytes per attention launch (written from rocprofv3)")
    return p.parse_args()


def main():
    a = _args()
    if a.gpus != 1:
        print(f"bench.py: this build measures one GPU only (asked for --gpus {a.gpus}); "
              "the decode kernel has no multi-GPU path.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import paged_kv_cache_273_amd as pkv
    from synthetic import generate, generate_multiquery, make_workload

    wl = make_workload(a.workload)
    multi = wl.q_uniform != (1, 1)
    mode = a.mode
    if mode == "auto":
        mode = "multiquery" if multi else ("split" if wl.split_tokens > 0 else "balanced")
    if (mode == "multiquery") != multi:
        print(f"bench.py: mode {mode} does not fit workload {wl.name}", file=sys.stderr)
        sys.exit(2)
    S = 0
    if mode == "split":
        S = a.split if a.split is not None else (wl.split_tokens or 512)
    dev = torch.device("cuda:0")
    t_gen = time.time()
    mq = generate_multiquery(wl) if multi else None
    inp = mq.base if multi else generate(wl)   # every cache group of the workload
    print(f"bench: generated {wl.name} in {time.time() - t_gen:.1f} s", file=sys.stderr,
          flush=True)

    def up(x):
        x = np.ascontiguousarray(x)
        if x.dtype == np.uint16:
            x = x.view(np.int16)
        return torch.from_numpy(x).to(dev)

    live = torch.from_numpy(np.arange(wl.block_size)[None, :] < inp.live[:, None]).to(dev)

    def quant(src):
        # fp8 cache built on the device from the bf16 source values (input
        # preparation only: scale = amax / 448 per block and kv head)
        x = up(src).view(torch.bfloat16).float()
        xm = torch.where(live[:, :, None, None] & torch.isfinite(x), x.abs(), torch.zeros_like(x))
        amax = xm.amax(dim=(1, 3))
        sc = torch.where(amax > 0, amax / 448.0, torch.ones_like(amax)).float()
        y = (x / sc[:, None, :, None]).clamp(-448, 448)
        return y.to(torch.float8_e4m3fn).view(torch.uint8).contiguous(), sc.contiguous()

    # one cache per layer group ([A] cross-layer KV sharing: layer l reads
    # group l // layers_per_group); bf16 workloads have a single group
    caches = []
    for g in range(wl.groups):
        if wl.kv_dtype == "fp8":
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
    per_layer = 2 * int(ctx.sum()) * wl.Hkv * wl.D * wl.bytes_per_elem
    ideal = per_layer * wl.layers
    scale = float(inp.scale)

    ms = pkv.max_splits_for(int(ctx.max()), S) if S else 1
    out = torch.empty((rows, wl.Hq, wl.D), dtype=torch.float32, device=dev)
    po = torch.empty((wl.B, wl.Hq, ms, wl.D), dtype=torch.float32, device=dev) if S else None
    pl = torch.empty((wl.B, wl.Hq, ms), dtype=torch.float32, device=dev) if S else None
    ws = pkv.make_workspace(qs[0], caches[0][0]) if mode == "balanced" else None
    if mode == "multiquery":
        ws = pkv.make_multiquery_workspace(qs[0], caches[0][0], max_q)

    ev = []  # (start, end) around each attention call in the timed region

    def step(record):
        for k, v, ks, vs, kn, vn in caches:
            if multi:
                pkv.paged_kv_write(kn, vn, qstart, k, v, bt, cl, max_q, k_scale=ks, v_scale=vs)
            else:
                pkv.paged_kv_append(kn, vn, k, v, bt, cl, k_scale=ks, v_scale=vs)
        for layer in range(wl.layers):
            k, v, ks, vs, _, _ = caches[layer // wl.layers_per_group]
            q = qs[layer]
            if record:
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record()
            if mode == "split":
                pkv.paged_decode_attention(q, k, v, bt, cl, scale, split_tokens=S,
                                           partial_out=po, partial_lse=pl, k_scale=ks,
                                           v_scale=vs)
            elif mode == "balanced":
                pkv.paged_decode_attention_balanced(q, k, v, bt, cl, scale, workspace=ws,
                                                    out=out, k_scale=ks, v_scale=vs)
            elif mode == "multiquery":
                pkv.paged_multiquery_attention(q, qstart, k, v, bt, cl, scale, max_q,
                                               workspace=ws, out=out, k_scale=ks, v_scale=vs)
            else:
                pkv.paged_decode_attention(q, k, v, bt, cl, scale, out=out, k_scale=ks,
                                           v_scale=vs)
            if record:
                e1.record()
                ev.append((e0, e1))
            if mode == "split":
                pkv.split_context_reduce(po, pl, cl, S, out=out)

    if a.calibrate_copy:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    for _ in range(a.warmup):
        step(False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(a.steps):
        step(True)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kern_s = sum(e0.elapsed_time(e1) for e0, e1 in ev) * 1e-3 / len(ev)

    step_s = wall / a.steps
    gbs = ideal / step_s / 1e9
    kern_gbs = per_layer / kern_s / 1e9
    traffic = _measured_traffic(a.traffic_json, f"{wl.name}:{mode}")

    cpu = None
    if not a.no_cpu_baseline:
        cpu = _cpu_baseline(inp, wl, a.cpu_seconds, mq)

    res = {
        "metric": METRIC,
        "value": round(gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(step_s * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.kv_dtype,
        "data": "synthetic",
        "pct_of_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
        "decode_tokens_per_s": round(wl.B / step_s, 1),
        "new_tokens_per_s": round(rows / step_s, 1),
        "config": {
            "workload": wl.name, "batch": wl.B, "Hq": wl.Hq, "Hkv": wl.Hkv, "head_dim": wl.D,
            "block_size": wl.block_size, "kv_dtype": wl.kv_dtype,
            "ctx_sum": int(ctx.sum()), "ctx_mean": round(float(ctx.mean()), 1),
            "ctx_min": int(ctx.min()), "ctx_max": int(ctx.max()), "schedule": mode,
            "split_tokens": S, "num_blocks": inp.num_blocks, "ideal_kv_bytes_per_step": ideal,
            "layers_per_step": wl.layers, "cache_groups": wl.groups,
            "new_tokens_per_sequence": (list(wl.q_uniform) if multi else 1),
            "new_tokens_per_step": rows,
            "step": {"split": "paged_kv_append + paged_decode_attention(split) + "
                              "split_context_reduce",
                     "balanced": "paged_kv_append + paged_decode_attention_balanced "
                                 "(decode + log-sum-exp merge of cut units)",
                     "single": "paged_kv_append + paged_decode_attention",
                     "multiquery": "paged_kv_write + paged_multiquery_attention (causal, "
                                   "log-sum-exp merge of cut units)"}[mode],
        },
        "roofline": {
            "bound": "hbm",
            "kernel": {"split": "decode_kernel (split)", "single": "decode_kernel",
                       "balanced": "decode_balanced_kernel + balanced_merge_kernel",
                       "multiquery": "decode_balanced_kernel (causal columns) + "
                                     "balanced_merge_kernel"}[mode],
            "achieved": round(kern_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(kern_gbs / HBM_PEAK_GBS, 4), "traffic": traffic,
            "launch_us": round(kern_s * 1e6, 2), "algorithmic_bytes_per_launch": per_layer,
        },
        "cpu_baseline": cpu,
    }
    print(json.dumps(res), flush=True)


def _measured_traffic(path, key):
    """HBM bytes per attention launch from the rocprofv3 FETCH_SIZE /
    WRITE_SIZE passes recorded in profiles/traffic.json, or None when there
    is no record or the decode source has changed since it was taken."""
    import hashlib

    try:
        rec = json.load(open(path)).get(key)
    except (OSError, ValueError):
        return None
    if not rec:
        return None
    src = os.path.join(ROOT, "paged_kv_cache_273_amd", "csrc", "decode.hip")
    sha = hashlib.sha256(open(src, "rb").read()).hexdigest()
    if rec.get("decode_source_sha256") != sha:
        return None
    return rec.get("hbm_bytes_per_launch")


def _cpu_baseline(inp, wl, target_s, mq=None):
    """The oracle (single-threaded C, fp64) on whole sequences of the same
    workload until about target_s seconds of CPU time; GB/s on the same
    ideal-byte formula."""
    if mq is not None:
        return _cpu_baseline_multiquery(mq, target_s)
    import numpy as np

    import oracle

    kp, vp = inp.k_pool[0], inp.v_pool[0]
    kind = "bf16"
    ks = vs = None
    if wl.kv_dtype == "fp8":
        ks = oracle.fp8_block_scales(kp, inp.block_tables, inp.context_lens, wl.block_size)
        vs = oracle.fp8_block_scales(vp, inp.block_tables, inp.context_lens, wl.block_size)
        kp, vp = oracle.fp8_quantize_pool(kp, ks), oracle.fp8_quantize_pool(vp, vs)
        kind = "fp8"
    oracle.append(inp.k_new[0], inp.v_new[0], kp, vp, inp.block_tables, inp.context_lens,
                  wl.block_size, kv_dtype=kind, k_scale=ks, v_scale=vs)
    done_bytes = 0
    seqs = 0
    t0 = time.perf_counter()
    for b in range(wl.B):
        sl = slice(b, b + 1)
        oracle.paged_attention(np.ascontiguousarray(inp.query[0][sl]), kp, vp,
                               np.ascontiguousarray(inp.block_tables[sl]),
                               np.ascontiguousarray(inp.context_lens[sl]), inp.scale,
                               block_size=wl.block_size, Hkv=wl.Hkv, kv_dtype=kind,
                               k_scale=ks, v_scale=vs)
        done_bytes += 2 * int(inp.context_lens[b]) * wl.Hkv * wl.D * wl.bytes_per_elem
        seqs += 1
        if time.perf_counter() - t0 >= target_s:
            break
    el = time.perf_counter() - t0
    gbs = done_bytes / el / 1e9
    return {"value": round(gbs, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"{seqs} of {wl.B} sequences (all {wl.Hq} query heads, "
                      f"{done_bytes / 1e6:.0f} MB of KV), single-threaded fp64 C, "
                      f"{el:.1f} s; {seqs / el:.3f} sequences/s",
            "cpu_model": _cpu_model(), "host_threads_available": os.cpu_count()}


def _cpu_baseline_multiquery(mq, target_s):
    """The multi-query oracle on whole sequences (bf16 or fp8 cache)."""
    import numpy as np

    import oracle

    wl, inp = mq.wl, mq.base
    kp, vp = inp.k_pool[0], inp.v_pool[0]
    kind = wl.kv_dtype
    ks = vs = None
    if kind == "fp8":
        ks = oracle.fp8_block_scales(kp, inp.block_tables, inp.context_lens, wl.block_size)
        vs = oracle.fp8_block_scales(vp, inp.block_tables, inp.context_lens, wl.block_size)
        kp, vp = oracle.fp8_quantize_pool(kp, ks), oracle.fp8_quantize_pool(vp, vs)
    else:
        kp, vp = kp.copy(), vp.copy()
    oracle.write_tokens(mq.k_rows[0], mq.v_rows[0], mq.query_start, kp, vp, inp.block_tables,
                        inp.context_lens, wl.block_size, kv_dtype=kind, k_scale=ks, v_scale=vs)
    done_bytes = rows = seqs = 0
    t0 = time.perf_counter()
    for b in range(wl.B):
        r0, r1 = int(mq.query_start[b]), int(mq.query_start[b + 1])
        oracle.multiquery_attention(np.ascontiguousarray(mq.query[0][r0:r1]),
                                    np.array([0, r1 - r0], dtype=np.int32), kp, vp,
                                    np.ascontiguousarray(inp.block_tables[b:b + 1]),
                                    np.ascontiguousarray(inp.context_lens[b:b + 1]), inp.scale,
                                    block_size=wl.block_size, Hkv=wl.Hkv, kv_dtype=kind,
                                    k_scale=ks, v_scale=vs)
        done_bytes += 2 * int(inp.context_lens[b]) * wl.Hkv * wl.D * wl.bytes_per_elem
        rows += r1 - r0
        seqs += 1
        if time.perf_counter() - t0 >= target_s:
            break
    el = time.perf_counter() - t0
    return {"value": round(done_bytes / el / 1e9, 4), "unit": "GB/s", "cores": 1,
            "kind": "oracle",
            "sample": f"{seqs} of {wl.B} sequences ({rows} new tokens, all {wl.Hq} query "
                      f"heads, {done_bytes / 1e6:.0f} MB of KV), single-threaded fp64 C, "
                      f"{el:.1f} s",
            "cpu_model": _cpu_model(), "host_threads_available": os.cpu_count()}


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
