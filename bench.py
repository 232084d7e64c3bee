#!/usr/bin/env python3
"""Benchmark of the batched multi-adapter LoRA layer on one MI355X.

One step = one pass of the whole hot path over one batch: lora_plan (segment
plan), then lora_apply = shrink (LoRA down projection of every planned pair)
+ base MFMA GEMM + expand (up projection added to the fp32 accumulators, one
rounding).  Default workload: Llama-7B q_proj decode, bf16, d_in = d_out =
4096, 64 tokens, 64 adapters of rank 16, each token on a uniformly drawn
adapter (synthetic, seeded).

Measurement
  * value: tokens per second over exactly --steps steps, wall clock between
    two torch.cuda.synchronize() calls, launches queued eagerly on one stream
    (faster on this stack than replaying a captured HIP graph of the same
    step, whose time is reported as step_us_graph_replay).  Each step is one
    call of lora_forward (plan + shrink + GEMM + epilogue: for decode shapes two
    launches, GEMM + per-slot shrink, then epilogue + plan; for stream-K
    shapes the plan is built inside the GEMM launch) on one of R rotated
    copies of the weights
    and adapter pool, R chosen so that R copies exceed 1 GiB: every step reads
    its W and pages from HBM, not from the 256 MiB Infinity Cache.
    value_apply_only: the same without the plan (built once per batch and
    shared by every layer of a model).
  * per-kernel durations: HIP events on the launch stream around blocks of
    back-to-back launches of one stage on the rotated copies, queued behind a
    busy prefix (so the events time the kernels, not host launch gaps).
  * roofline: the dominant kernel (the base GEMM).  Below the MFMA/HBM ridge
    (~312 flop/byte) it is priced against 8 TB/s HBM with its algorithmic
    bytes (W + X), above it against 2.5 PFLOP/s bf16 MFMA with its
    algorithmic flops (2 T d_in d_out, plus the expand when it runs inside the
    GEMM).  traffic: HBM bytes per launch from rocprofv3 FETCH_SIZE and
    WRITE_SIZE counters, scaled by the same counters on a copy of known size,
    read from the committed summary profiles/traffic.json when the GEMM
    source still matches the hash recorded there (else null).
  * LoRA path: t_apply - t_base where t_base is the same step on an empty
    plan; LoRA bytes = used A and B pages + X rows + U (written and read).
  * cpu_baseline: the CPU oracle (fp64 numpy) on the same workload, on the
    host's cores, for a bounded number of seconds.

  --copy-probe runs a 256 MiB device-to-device copy five times first, so that
  a rocprofv3 --pmc run of this script also holds the calibration kernel.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
FP32_PEAK_TFLOPS = 157.3
RIDGE_FLOP_PER_BYTE = MFMA_BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)
METRIC = "tokens/sec per multi-LoRA layer at 1 GPU; LoRA-path HBM GB/s as % of peak"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--workload", type=int, default=2, help="workload recipe 1..5")
    ap.add_argument("--event-steps", type=int, default=200)
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--rotation", type=int, default=0, help="copies of W/pool (0: >= 1 GiB)")
    ap.add_argument("--no-graph", action="store_true",
                    help="skip the HIP-graph replay timing (the value is timed with eager launches)")
    ap.add_argument("--copy-probe", action="store_true")
    ap.add_argument("--pmc-summary", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="turn two rocprofv3 --pmc counter CSVs of a --copy-probe run into "
                         "profiles/traffic.json entries, then exit")
    return ap.parse_args()


class Copy:
    """One rotated copy of the layer's HBM-resident tensors."""

    def __init__(self, L, B, torch, clone: bool):
        self.X = L.X.clone() if clone else L.X
        self.W_t = L.W_t.clone() if clone else L.W_t
        a = L.a_pages.clone() if clone else L.a_pages
        b = L.b_pages.clone() if clone else L.b_pages
        self.pool = B.Pool(L.dtype, L.w.d_in, L.w.d_out, a, b, L.rank, L.page_start,
                           L.pool.tensors[4], L.scale)
        self.plan = torch.empty_like(L.plan)
        self.ws = torch.empty_like(L.ws)
        self.Y = torch.empty_like(L.Y)


def main():
    args = parse()
    if args.pmc_summary:
        pmc_summary(args.workload, *args.pmc_summary)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE={world}); "
              "the layer shards over tokens with no exchange between GPUs", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from lora_adapter_amd import binding as B
    from lora_adapter_amd import device as D
    from lora_adapter_amd import workloads as wl

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    B.lib()
    torch.cuda.set_device(0)
    if args.copy_probe:
        src = torch.empty(256 << 20, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    w = wl.config(args.workload)
    L = D.DeviceLayer(w)
    T, K = w.T, w.K
    ids, gates, mask = L.ids, L.gates, L.keep_mask
    empty_ids = torch.full_like(ids, -1)

    # rotation copies: >= 1 GiB of W + pool + X
    per_copy = (L.W_t.numel() * L.W_t.element_size() + L.a_pages.numel() * L.a_pages.element_size()
                + L.b_pages.numel() * L.b_pages.element_size() + L.X.numel() * L.X.element_size())
    R = args.rotation or max(2, int(np.ceil((1 << 30) / per_copy)))
    copies = [Copy(L, B, torch, clone=(i > 0)) for i in range(R)]
    stream = torch.cuda.current_stream()

    def step(c, use_ids=ids, plan=True):
        if plan:
            B.lora_forward(use_ids, gates, T, K, c.X, c.W_t, c.Y, mask, L.keep_scale, c.pool, c.plan,
                           c.ws)
            return
        B.lora_shrink_gemm(c.X, c.W_t, c.Y, T, K, gates, mask, L.keep_scale, c.pool, c.plan, c.ws)
        B.lora_expand_epilogue(c.X, c.W_t, c.Y, T, K, c.pool, c.plan, c.ws)

    # ---------------------------------------------------------------- graphs
    def make_graphs(use_ids, plan, graph):
        if not graph:
            return None
        gs = []
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for c in copies:       # warm the allocator / code objects outside capture
                step(c, use_ids)   # (and leave a valid plan in every copy)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        for c in copies:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                step(c, use_ids, plan)
            gs.append(g)
        torch.cuda.synchronize()
        return gs

    def timed(use_ids, steps, warmup, plan=True, graph=False):
        gs = make_graphs(use_ids, plan, graph)
        run = ((lambda i: gs[i % R].replay()) if gs
               else (lambda i: step(copies[i % R], use_ids, plan)))
        for i in range(warmup):
            run(i)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            run(i)
        torch.cuda.synchronize()
        return time.perf_counter() - t0

    elapsed = timed(ids, args.steps, args.warmup)
    for c in copies:       # apply-only steps reuse a plan built once per batch by lora_plan
        B.lora_plan(ids, gates, T, K, c.pool, c.plan)
    elapsed_apply = timed(ids, args.steps, args.warmup, plan=False)
    elapsed_base = timed(empty_ids, args.steps, args.warmup)
    elapsed_graph = None if args.no_graph else timed(ids, args.steps, args.warmup, graph=True)
    # results of the last apply on copy 0 must not be stale: re-run eagerly
    step(copies[0], ids)
    torch.cuda.synchronize()
    hdr = copies[0].plan[L.layout[0] // 4:L.layout[0] // 4 + 16].cpu().numpy()

    # ---------------------------------------------------------------- per-kernel events
    big = torch.randn(8192, 8192, device="cuda", dtype=torch.bfloat16)

    stages = {
        "plan": lambda c, u: B.lora_plan(u, gates, T, K, c.pool, c.plan),
        "fwd_gemm": lambda c, u: B.lora_forward_gemm(u, gates, T, K, c.X, c.W_t, c.Y, mask,
                                                     L.keep_scale, c.pool, c.plan, c.ws),
        "fwd_finish": lambda c, u: B.lora_forward_finish(u, gates, T, K, c.X, c.W_t, c.Y, mask,
                                                         L.keep_scale, c.pool, c.plan, c.ws),
        "shrink_gemm": lambda c, u: B.lora_shrink_gemm(c.X, c.W_t, c.Y, T, K, gates, mask,
                                                       L.keep_scale, c.pool, c.plan, c.ws),
        "shrink": lambda c, u: B.lora_shrink(c.X, mask, L.keep_scale, T, K, gates, c.pool, c.plan, c.ws),
        "gemm": lambda c, u: B.lora_base_gemm(c.X, c.W_t, c.Y, T, K, c.pool, c.plan, c.ws),
        "epilogue": lambda c, u: B.lora_expand_epilogue(c.X, c.W_t, c.Y, T, K, c.pool, c.plan, c.ws),
    }

    def stage_times(use_ids, n):
        """Per stage: blocks of `reps` back-to-back launches on the rotating
        copies, bracketed by two HIP events on the launch stream and queued
        behind a busy prefix so the events time the kernels, not the host."""
        reps = min(R, 32) if R >= 8 else 16
        rounds = max(3, n // reps)
        out = {}
        for name, fn in stages.items():
            for c in copies:              # every copy holds a valid plan (built by lora_plan) and U
                B.lora_plan(use_ids, gates, T, K, c.pool, c.plan)
                B.lora_shrink(c.X, mask, L.keep_scale, T, K, gates, c.pool, c.plan, c.ws)
            torch.cuda.synchronize()
            ts = []
            for rd in range(rounds):
                for _ in range(2):
                    torch.mm(big, big)
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                for i in range(reps):
                    fn(copies[(rd * reps + i) % R], use_ids)
                e1.record(stream)
                torch.cuda.synchronize()
                ts.append(e0.elapsed_time(e1) * 1e3 / reps)
            out[name] = ts
        for c in copies:
            step(c, use_ids)
        torch.cuda.synchronize()
        return ({k: float(np.median(v)) for k, v in out.items()},
                {k: float(np.mean(v)) for k, v in out.items()})

    st_med, st_mean = stage_times(ids, args.event_steps)
    sb_med, sb_mean = stage_times(empty_ids, args.event_steps)

    def event_time(fn, reps, rounds=5):
        """Median over rounds of (events around `reps` back-to-back calls) / reps."""
        ts = []
        for _ in range(rounds):
            for _ in range(2):
                torch.mm(big, big)
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for i in range(reps):
                fn(i)
            e1.record(stream)
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1) * 1e3 / reps)
        return float(np.median(ts))

    e_bytes = 2 if L.dtype == B.LORA_BF16 else 4
    extra = {}
    if w.merge_ids is not None:
        # signed merge of the workload's adapters into W, then the unmerge,
        # alternating on the rotated copies (each copy returns near W)
        m_ids = D.to_device(np.asarray(w.merge_ids, np.int32), "cuda")
        plus = D.to_device(np.ones(len(w.merge_ids), np.float32), "cuda")
        minus = D.to_device(-np.ones(len(w.merge_ids), np.float32), "cuda")
        mcopies = [c.W_t for c in copies]

        def merge_call(i):
            B.lora_merge_delta(mcopies[(i // 2) % R], L.pool, m_ids, plus if i % 2 == 0 else minus,
                               len(w.merge_ids))
        t_m = event_time(merge_call, 2 * min(R, 8))
        rsum = int(sum(int(w.rank[a]) for a in w.merge_ids))
        m_bytes = 2 * w.d_in * w.d_out * e_bytes + rsum * (w.d_in + w.d_out) * e_bytes
        extra["merge"] = {"adapters": len(w.merge_ids), "us": t_m, "bytes": m_bytes,
                          "GB_s": m_bytes / t_m / 1e3, "frac_hbm": m_bytes / t_m / 1e3 / HBM_PEAK_GBS,
                          "flops": 2.0 * w.d_in * w.d_out * rsum}
    if w.dY is not None:
        # LoRA grads dA, dB after the forward of copy 0 (its U in the workspace)
        dA, dB, gws = L.grad_buffers()
        c0 = copies[0]
        step(c0, ids)
        torch.cuda.synchronize()

        def grad_call(i):
            B.lora_grad(c0.X, mask, L.keep_scale, L.dY, T, K, gates, c0.pool, c0.plan, c0.ws,
                        dA, dB, L.max_rank, gws)
        t_g = event_time(grad_call, 8)
        hdr0 = c0.plan[L.layout[0] // 4:L.layout[0] // 4 + 16].cpu().numpy()
        Ru, Rp = int(hdr0[B.PH_RUSED]), int(hdr0[B.PH_RPAIRS])
        g_bytes = (T * w.d_out * e_bytes + T * w.d_in * (e_bytes + (1 if mask is not None else 0))
                   + Ru * (w.d_in + w.d_out) * (e_bytes + 4) + 8 * Rp)
        extra["grads"] = {"us": t_g, "bytes": g_bytes, "GB_s": g_bytes / t_g / 1e3,
                          "frac_hbm": g_bytes / t_g / 1e3 / HBM_PEAK_GBS,
                          "flops": 2.0 * Rp * (2 * w.d_out + w.d_in)}

    # ---------------------------------------------------------------- figures
    e = 2 if L.dtype == B.LORA_BF16 else 4
    P, S, R_pairs, R_used = (int(hdr[B.PH_PAIRS]), int(hdr[B.PH_SEGS]), int(hdr[B.PH_RPAIRS]),
                             int(hdr[B.PH_RUSED]))
    w_bytes = w.d_in * w.d_out * e
    x_bytes = T * w.d_in * e
    y_bytes = T * w.d_out * e
    t_step = elapsed / args.steps
    t_base_step = elapsed_base / args.steps
    # LoRA path time = step - step with an empty plan; when that difference
    # is within run-to-run noise (the LoRA work hidden beside the base GEMM in
    # the same launches) no rate is reported for it
    t_lora = t_step - t_base_step
    lora_hidden = t_lora <= 0.02 * t_step
    lora_bytes = R_used * (w.d_in + w.d_out) * e + P * w.d_in * e + 8 * R_pairs
    if mask is not None:
        lora_bytes += P * w.d_in
    lora_flops = 2.0 * R_pairs * (w.d_in + w.d_out)
    base_flops = 2.0 * T * w.d_in * w.d_out
    value = T * args.steps / elapsed
    roofline = gemm_roofline(B, L, w, T, st_med, base_flops, P, R_pairs, R_used, e)

    out = {
        "metric": METRIC,
        "value": value,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": t_step * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if L.dtype == B.LORA_BF16 else "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "T": T, "K": K, "d_in": w.d_in, "d_out": w.d_out,
                   "adapters": w.n_adapters, "ranks": sorted(set(w.rank.tolist()))[:8],
                   "active_pairs": P, "segments": S, "R_used": R_used, "R_pairs": R_pairs,
                   "rotation_copies": R, "launch": "eager"},
        "roofline": roofline,
        "value_apply_only": T * args.steps / elapsed_apply,
        **extra,
        "stages_us_median": st_med,
        "stages_us_mean": st_mean,
        "stages_us_mean_empty_plan": sb_mean,
        "step_us": t_step * 1e6,
        "step_us_graph_replay": None if elapsed_graph is None else elapsed_graph / args.steps * 1e6,
        "step_us_empty_plan": t_base_step * 1e6,
        "lora_path": ({"t_us": t_lora * 1e6, "bytes": lora_bytes, "GB_s": None, "frac_hbm": None,
                       "flops": lora_flops,
                       "note": "step with LoRA within 2 % of the step with an empty plan: "
                               "the LoRA work is hidden beside the base GEMM, no rate"}
                      if lora_hidden else
                      {"t_us": t_lora * 1e6, "bytes": lora_bytes, "GB_s": lora_bytes / t_lora / 1e9,
                       "frac_hbm": lora_bytes / t_lora / 1e9 / HBM_PEAK_GBS, "flops": lora_flops}),
        "layer": {"bytes": w_bytes + x_bytes + y_bytes + lora_bytes,
                  "GB_s": (w_bytes + x_bytes + y_bytes + lora_bytes) / t_step / 1e9,
                  "TFLOP_s": (base_flops + lora_flops) / t_step / 1e12,
                  "frac_mfma": (base_flops + lora_flops) / t_step / 1e12 / MFMA_BF16_PEAK_TFLOPS},
    }

    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
    print(json.dumps(out), flush=True)


def gemm_kernel_name(T, d_in, d_out, dtype_code, B, fused):
    """The launch that runs the base GEMM inside lora_forward (the library's
    shape rules: decode GEMM for T <= 128, with the per-slot shrink in the
    same launch; fused-epilogue 256 x 256 tiles when they fill the GPU; else
    256 x 128 stream-K tiles over 255 workgroups when there are at least 4
    units each, with the plan built in the same launch)."""
    if dtype_code != B.LORA_BF16:
        return "gemm_f32_kernel (plan)"
    if T <= 128:
        return "decode_gemm_slot_kernel"
    if fused:
        return "gemm_tile_kernel (fused expand)"
    units = ((T + 255) // 256) * ((d_out + 127) // 128) * (d_in // 64)
    return "gemm_tile_plan_kernel" if units >= 4 * 255 else "gemm_tile_kernel"


def gemm_roofline(B, L, w, T, st_med, base_flops, P, R_pairs, R_used, e):
    """Roofline entry of the kernel that runs the base GEMM in the step, from
    its measured duration.  When that launch also runs the per-slot shrink
    (decode) its algorithmic bytes add the used A pages (each once), U and
    the slot descriptors; when it builds the plan (stream-K), the plan's
    inputs (ids, gates, the pool's rank and page tables)."""
    fused = T > 128 and ((T + 255) // 256) * ((w.d_out + 255) // 256) >= 256
    name = gemm_kernel_name(T, w.d_in, w.d_out, L.dtype, B, fused)
    alg_bytes = (w.d_in * w.d_out + T * w.d_in) * e
    flops = base_flops + (2.0 * R_pairs * w.d_out if fused else 0.0)
    if name == "decode_gemm_slot_kernel":
        t_us = st_med["fwd_gemm"]
        alg_bytes += R_used * w.d_in * e + 4 * R_pairs + 16 * T * w.K
        alg_bytes += T * w.d_in if L.keep_mask is not None else 0
        flops += 2.0 * R_pairs * w.d_in
    elif name in ("gemm_tile_plan_kernel", "gemm_f32_kernel (plan)"):
        t_us = st_med["fwd_gemm"]
        alg_bytes += 8 * T * w.K + 8 * w.n_adapters + 4 * R_used
    else:
        t_us = st_med["gemm"]
    intensity = base_flops / ((w.d_in * w.d_out + T * w.d_in + T * w.d_out) * e)
    t = t_us * 1e-6
    if L.dtype != B.LORA_BF16:
        r = {"bound": "alu", "achieved": flops / t / 1e12, "peak": FP32_PEAK_TFLOPS,
             "unit": "TFLOP/s", "alg_flops_per_launch": flops}
    elif intensity > RIDGE_FLOP_PER_BYTE:
        r = {"bound": "mfma", "achieved": flops / t / 1e12, "peak": MFMA_BF16_PEAK_TFLOPS,
             "unit": "TFLOP/s", "alg_flops_per_launch": flops}
    else:
        r = {"bound": "hbm", "achieved": alg_bytes / t / 1e9, "peak": HBM_PEAK_GBS,
             "unit": "GB/s", "alg_bytes_per_launch": alg_bytes}
    r["frac"] = r["achieved"] / r["peak"]
    r["traffic"] = measured_traffic(name, w.name)
    r["kernel"] = name
    r["avg_launch_us"] = t_us
    return r


def kernel_source_hash():
    import hashlib
    h = hashlib.sha256()
    for f in ("gemm.hip", "shrink_units.h", "lora_internal.h", "plan_build.h"):
        with open(os.path.join(ROOT, "lora_adapter_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel, workload):
    """HBM bytes per launch from the committed counter summary, or None when
    there is none for this kernel and workload or the source has changed."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as fh:
            table = json.load(fh)
    except (OSError, ValueError):
        return None
    ent = table.get(kernel.split(" ")[0] + "|" + workload)
    if not ent or ent.get("source_sha256_16") != kernel_source_hash():
        return None
    return ent.get("hbm_bytes_per_launch")


COPY_PROBE_BYTES = 256 << 20


def pmc_summary(workload_id, fetch_csv, write_csv):
    """HBM bytes per launch of the base GEMM from FETCH_SIZE / WRITE_SIZE
    (KiB per dispatch), each scaled by the copy probe's reading of the same
    counter against the bytes that copy must move."""
    import csv
    import numpy as np
    from lora_adapter_amd import workloads as wl

    def per_kernel(path, counter):
        vals = {}
        with open(path) as fh:
            for r in csv.DictReader(fh):
                if r["Counter_Name"] != counter:
                    continue
                vals.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]) * 1024.0)
        return vals

    w = wl.config(workload_id)
    T = w.T
    fused = T > 128 and ((T + 255) // 256) * ((w.d_out + 255) // 256) >= 256
    kname = gemm_kernel_name(T, w.d_in, w.d_out, 1 if w.dtype == "bf16" else 0,
                             type("B", (), {"LORA_BF16": 1}), fused).split(" ")[0]

    def name_of(k):
        for n in ("decode_gemm_slot_kernel", "gemm_tile_plan_kernel", "decode_gemm_shrink_kernel",
                  "gemm_decode_kernel", "gemm_tile_kernel", "gemm_f32_kernel"):
            if n in k:
                return n
        return None

    out = {}
    for counter, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        vals = per_kernel(path, counter)
        copy = [v for k, vs in vals.items() if "copyBuffer" in k for v in vs
                if v > COPY_PROBE_BYTES / 2]
        gemm = [v for k, vs in vals.items() if name_of(k) == kname for v in vs]
        if not copy or not gemm:
            raise SystemExit(f"{path}: no copy probe or GEMM dispatches for {counter}")
        scale = COPY_PROBE_BYTES / float(np.median(copy))
        out[counter] = {"raw_bytes_median": float(np.median(gemm)), "copy_scale": scale,
                        "bytes": float(np.median(gemm)) * scale, "dispatches": len(gemm)}
    name = kname
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as fh:
            table = json.load(fh)
    except (OSError, ValueError):
        table = {}
    table[name + "|" + w.name] = {
        "hbm_bytes_per_launch": out["FETCH_SIZE"]["bytes"] + out["WRITE_SIZE"]["bytes"],
        "fetch": out["FETCH_SIZE"], "write": out["WRITE_SIZE"],
        "source_sha256_16": kernel_source_hash(),
    }
    with open(path, "w") as fh:
        json.dump(table, fh, indent=1, sort_keys=True)
    print(json.dumps(table[name + "|" + w.name]))


def cpu_baseline(w, seconds):
    """The CPU oracle, untuned, on the same workload: plan + apply per step."""
    import numpy as np
    from oracle import lora_oracle as O
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count() or 1
    threads = cores
    try:
        from threadpoolctl import threadpool_info
        info = threadpool_info()
        if info:
            threads = max(int(i.get("num_threads", 1)) for i in info)
    except Exception:
        pass
    n = 0
    t0 = time.perf_counter()
    while True:
        O.plan_workload(w)
        O.apply_workload(w)
        n += 1
        el = time.perf_counter() - t0
        if el >= seconds or n >= 1000:
            break
    return {"value": w.T * n / el, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{n} full steps (plan + apply, fp64 numpy) of the same workload in {el:.1f} s"}


if __name__ == "__main__":
    main()
