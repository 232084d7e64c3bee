#!/usr/bin/env python3
"""Benchmark of the batched multi-adapter LoRA layer on one MI355X.

One step = one pass of the whole hot path over one batch of the workload:
  * lora_forward: the segment plan, the shrink (LoRA down projection of every
    planned pair), the base MFMA GEMM and the expand (up projection added to
    the fp32 accumulators before the one rounding);
  * and, when the workload trains (it carries dY), lora_grad: dA and dB of
    every used adapter.
Default workload: the fine-tune/prefill shape, bf16, X 8192 x 4096, W 4096 ->
11008, 4 adapters of rank 16 on Dirichlet(1) contiguous segments, keep mask
Bernoulli(0.9), forward plus dA, dB for a random dY (synthetic, seeded).  The
other workloads (q_proj decode, heterogeneous ranks, compressed fleet with
top-2 routing and a merge/unmerge) are measured after it, more briefly, and
reported under "workloads".

Measurement
  * value: tokens per second over exactly --steps steps, wall clock between
    two torch.cuda.synchronize() calls, launches queued eagerly on one stream,
    each step on one of R rotated copies of W, X (and dY, mask) and the adapter
    pool, R chosen so that the copies exceed 1 GiB: every step reads from HBM,
    not from the 256 MiB Infinity Cache.  value_forward: the same without the
    gradients; value_apply_only: the forward on a plan built once per batch
    (shared by every layer of a model); value_plan_shared: the full step
    (forward + gradients) on such a plan, i.e. the cost per projection once
    the batch's one lora_plan is paid (value itself includes it).
  * per-launch durations: HIP events on the launch stream around blocks of
    back-to-back launches of one stage on the rotated copies, queued behind a
    busy prefix (so the events time the kernels, not host launch gaps).
  * roofline: the launch that runs the base GEMM.  Above the MFMA/HBM ridge
    (~312 flop/byte) it is priced against 2.5 PFLOP/s bf16 MFMA with its
    algorithmic flops (2 T d_in d_out, plus the expand when it runs inside the
    GEMM), below it against 8 TB/s with its algorithmic bytes.  traffic: HBM
    bytes per launch from rocprofv3 FETCH_SIZE and WRITE_SIZE, scaled by the
    same counters on a copy of known size, read from profiles/traffic.json
    when the kernel sources still match the hash recorded there (else null).
  * LoRA path: the apply's launches (shrink + GEMM, then the epilogue) timed
    with the batch's plan and with an empty plan; the LoRA path's time is the
    sum of the per-launch differences, its bytes the used A and B pages, the X
    rows (and mask) it reads and U (written and read).  The wall-clock step
    difference is reported beside it.
  * cpu_baseline: the CPU oracle (fp64 numpy, untuned) on a bounded sample of
    the same workload, on the host's cores.
  * hipblaslt_gemm_us (each workload): torch.mm (hipBLASLt) of X by W on the
    same rotated copies, timed like the launches: the plain GEMM without the
    LoRA term, context only.

  --copy-probe runs a 256 MiB device-to-device copy five times first, so that
  a rocprofv3 --pmc run of this script also holds the calibration kernel.
"""
from __future__ import annotations

import argparse
import json
import os
import platform
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
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", type=int, default=4, help="workload recipe 1..5 (the headline)")
    ap.add_argument("--others", default="2,3,5",
                    help="workloads measured after the headline, comma separated ('' for none)")
    ap.add_argument("--other-steps", type=int, default=200)
    ap.add_argument("--event-steps", type=int, default=100)
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--rotation", type=int, default=0, help="copies of W/pool (0: >= 1 GiB)")
    ap.add_argument("--graph", action="store_true",
                    help="also time a captured HIP graph of the step (the value is eager)")
    ap.add_argument("--skip-empty-plan", action="store_true",
                    help="no runs on an empty plan (for kernel traces whose averages should "
                         "hold only launches with the batch's plan; no LoRA-path figures)")
    ap.add_argument("--residency", type=int, default=1,
                    help="1: also time the heterogeneous-rank workload with its pool held to "
                         "--residency-frac of the fleet (pages copied in from pinned host memory)")
    ap.add_argument("--residency-frac", type=float, default=0.6)
    ap.add_argument("--no-tsqr", action="store_true", help="skip the fleet QR/compression timing")
    ap.add_argument("--no-blas-ref", action="store_true",
                    help="skip the context timing of torch.mm (hipBLASLt) on each workload's GEMM")
    ap.add_argument("--copy-probe", action="store_true")
    ap.add_argument("--pmc-summary", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="turn two rocprofv3 --pmc counter CSVs of a --copy-probe run into "
                         "profiles/traffic.json entries for --workload, then exit")
    return ap.parse_args()


# ---------------------------------------------------------------- launch rules

def gemm_kind(T, d_in, d_out, bf16):
    """The library's base GEMM choice (host rules in choose_gemm): 'f32',
    'decode' (T <= 128), 'fused' (256 x 256 tiles with the expand in the
    epilogue, when they fill the GPU), 'streamk' (256 x 128 stream-K tiles
    with the plan built in the launch) or 'split'."""
    if not bf16:
        return "f32"
    if T <= 128:
        return "decode"
    if ((T + 255) // 256) * ((d_out + 255) // 256) >= 256:
        return "fused"
    units = ((T + 255) // 256) * ((d_out + 127) // 128) * (d_in // 64)
    return "streamk" if units >= 4 * 255 else "split"


GEMM_KERNEL = {"f32": "gemm_f32_kernel", "decode": "decode_gemm_slot_kernel",
               "fused": "gemm_tile_kernel", "streamk": "gemm_tile_plan_kernel",
               "split": "gemm_tile_kernel"}


class Copy:
    """One rotated copy of the layer's HBM-resident tensors."""

    def __init__(self, L, B, torch, clone: bool):
        cl = (lambda t: None if t is None else t.clone()) if clone else (lambda t: t)
        self.X = cl(L.X)
        self.W_t = cl(L.W_t)
        self.dY = cl(L.dY)
        self.mask = cl(L.keep_mask)
        a = cl(L.a_pages)
        b = cl(L.b_pages)
        self.pool = B.Pool(L.dtype, L.w.d_in, L.w.d_out, a, b, L.rank, L.page_start,
                           L.pool.tensors[4], L.scale)
        self.plan = torch.empty_like(L.plan)
        self.ws = torch.empty_like(L.ws)
        self.Y = torch.empty_like(L.Y)


class Bench:
    """Timing harness for one workload resident on the GPU."""

    def __init__(self, w, args, torch, np, B, D, grads=True, rotation=0):
        self.w, self.args, self.torch, self.np, self.B, self.D = w, args, torch, np, B, D
        L = D.DeviceLayer(w)
        self.L = L
        self.T, self.K = w.T, w.K
        self.ids, self.gates = L.ids, L.gates
        self.empty_ids = torch.full_like(L.ids, -1)
        per_copy = sum(t.numel() * t.element_size() for t in
                       (L.W_t, L.a_pages, L.b_pages, L.X, L.dY, L.keep_mask) if t is not None)
        self.R = rotation or max(2, int(np.ceil((1 << 30) / per_copy)))
        self.copies = [Copy(L, B, torch, clone=(i > 0)) for i in range(self.R)]
        self.stream = torch.cuda.current_stream()
        self.grads = grads and w.dY is not None
        if self.grads:
            self.dA, self.dB, self.gws = L.grad_buffers()
        self.big = torch.randn(8192, 8192, device="cuda", dtype=torch.bfloat16)

    # -- the step and its parts ------------------------------------------------
    def forward(self, c, ids):
        B, L = self.B, self.L
        B.lora_forward(ids, self.gates, self.T, self.K, c.X, c.W_t, c.Y, c.mask, L.keep_scale,
                       c.pool, c.plan, c.ws)

    def apply(self, c):
        B, L = self.B, self.L
        B.lora_apply(c.X, c.W_t, c.Y, self.T, self.K, self.gates, c.mask, L.keep_scale, c.pool,
                     c.plan, c.ws)

    def grad(self, c):
        B, L = self.B, self.L
        B.lora_grad(c.X, c.mask, L.keep_scale, c.dY, self.T, self.K, self.gates, c.pool, c.plan,
                    c.ws, self.dA, self.dB, L.max_rank, self.gws)

    def step(self, c, ids=None):
        self.forward(c, self.ids if ids is None else ids)
        if self.grads:
            self.grad(c)

    def plan_all(self, ids):
        for c in self.copies:
            self.B.lora_plan(ids, self.gates, self.T, self.K, c.pool, c.plan)

    def timed(self, fn, steps, warmup):
        """Seconds for `steps` calls fn(copy), after `warmup` calls, between
        two synchronizes."""
        R, torch = self.R, self.torch
        for i in range(warmup):
            fn(self.copies[i % R])
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            fn(self.copies[i % R])
        torch.cuda.synchronize()
        return time.perf_counter() - t0

    def timed_graph(self, steps, warmup):
        """The step captured in one HIP graph per copy, replayed."""
        torch = self.torch
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for c in self.copies:
                self.step(c)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        gs = []
        for c in self.copies:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                self.step(c)
            gs.append(g)
        torch.cuda.synchronize()
        for i in range(warmup):
            gs[i % self.R].replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            gs[i % self.R].replay()
        torch.cuda.synchronize()
        return time.perf_counter() - t0

    def event_us(self, fn, reps, rounds):
        """Median over rounds of (HIP events around `reps` back-to-back calls
        fn(i) on the launch stream) / reps, each round queued behind two
        large GEMMs so that the events time the kernels, not the host."""
        torch, np = self.torch, self.np
        ts = []
        for _ in range(rounds):
            for _ in range(2):
                torch.mm(self.big, self.big)
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(self.stream)
            for i in range(reps):
                fn(i)
            e1.record(self.stream)
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1) * 1e3 / reps)
        return float(np.median(ts))

    def stage_us(self, ids, n):
        """Per-launch HIP-event times of each stage of the path, every copy
        holding a valid plan (lora_plan) and U (lora_shrink) of `ids`."""
        B, L, T, K, g = self.B, self.L, self.T, self.K, self.gates
        stages = {
            "plan": lambda c: B.lora_plan(ids, g, T, K, c.pool, c.plan),
            "fwd_gemm": lambda c: B.lora_forward_gemm(ids, g, T, K, c.X, c.W_t, c.Y, c.mask,
                                                      L.keep_scale, c.pool, c.plan, c.ws),
            "fwd_finish": lambda c: B.lora_forward_finish(ids, g, T, K, c.X, c.W_t, c.Y, c.mask,
                                                          L.keep_scale, c.pool, c.plan, c.ws),
            "shrink_gemm": lambda c: B.lora_shrink_gemm(c.X, c.W_t, c.Y, T, K, g, c.mask,
                                                        L.keep_scale, c.pool, c.plan, c.ws),
            "shrink": lambda c: B.lora_shrink(c.X, c.mask, L.keep_scale, T, K, g, c.pool, c.plan,
                                              c.ws),
            "gemm": lambda c: B.lora_base_gemm(c.X, c.W_t, c.Y, T, K, c.pool, c.plan, c.ws),
            "epilogue": lambda c: B.lora_expand_epilogue(c.X, c.W_t, c.Y, T, K, c.pool, c.plan,
                                                         c.ws),
        }
        if self.grads:
            stages["grad"] = lambda c: self.grad(c)
        reps = min(self.R, 32) if self.R >= 8 else 8
        rounds = max(3, n // reps)
        out = {}
        for name, fn in stages.items():
            self.plan_all(ids)
            for c in self.copies:
                B.lora_shrink(c.X, c.mask, L.keep_scale, T, K, g, c.pool, c.plan, c.ws)
            self.torch.cuda.synchronize()
            out[name] = self.event_us(lambda i: fn(self.copies[i % self.R]), reps, rounds)
        for c in self.copies:
            self.step(c, ids)
        self.torch.cuda.synchronize()
        return out

    def header(self, c):
        return self.B.lora_plan_header(c.plan)


def lora_bytes(w, P, R_pairs, R_used, e, masked):
    """Algorithmic bytes of the LoRA path (shrink + expand): each used A page
    and B page once, the X rows of the active pairs (and their mask bytes),
    U written and read."""
    b = R_used * (w.d_in + w.d_out) * e + P * w.d_in * e + 8 * R_pairs
    return b + (P * w.d_in if masked else 0)


def measure(w, args, torch, np, B, D, steps, warmup, full):
    """Step time, per-launch times, LoRA path and (full) the roofline of one
    workload."""
    bn = Bench(w, args, torch, np, B, D, rotation=args.rotation)
    T, K = w.T, w.K
    e = 2 if bn.L.dtype == B.LORA_BF16 else 4
    kind = gemm_kind(T, w.d_in, w.d_out, bn.L.dtype == B.LORA_BF16)

    el_step = bn.timed(lambda c: bn.step(c), steps, warmup)
    el_fwd = bn.timed(lambda c: bn.forward(c, bn.ids), steps, warmup)
    skip0 = args.skip_empty_plan
    el_base = None if skip0 else bn.timed(lambda c: bn.forward(c, bn.empty_ids), steps, warmup)
    bn.plan_all(bn.ids)
    el_apply = bn.timed(lambda c: bn.apply(c), steps, warmup)

    def shared(c):
        # the batch's plan already built (lora_plan once per batch, shared by
        # every LoRA projection that routes the same tokens): apply + grads
        bn.apply(c)
        if bn.grads:
            bn.grad(c)
    el_shared = bn.timed(shared, steps, warmup)
    el_graph = bn.timed_graph(steps, warmup) if args.graph else None
    bn.step(bn.copies[0])
    torch.cuda.synchronize()
    hdr = bn.header(bn.copies[0])
    P, S, R_pairs, R_used = (hdr[B.PH_PAIRS], hdr[B.PH_SEGS], hdr[B.PH_RPAIRS], hdr[B.PH_RUSED])

    st = bn.stage_us(bn.ids, args.event_steps if full else 32)
    st0 = None if skip0 else bn.stage_us(bn.empty_ids, args.event_steps if full else 32)
    # context only: the vendor library's plain GEMM (no LoRA term) on the same
    # rotated operands, timed the same way
    blas_us = None
    if bn.L.dtype == B.LORA_BF16 and not args.no_blas_ref:
        n_ev = args.event_steps if full else 32
        reps = min(bn.R, 32) if bn.R >= 8 else 8
        blas_us = bn.event_us(lambda i: torch.mm(bn.copies[i % bn.R].X, bn.copies[i % bn.R].W_t.t(),
                                                 out=bn.copies[i % bn.R].Y),
                              reps, max(3, n_ev // reps))
    lb = lora_bytes(w, P, R_pairs, R_used, e, w.keep_mask is not None)
    lf = 2.0 * R_pairs * (w.d_in + w.d_out)
    # LoRA path from the apply's launches (the plan built once per batch):
    # shrink + GEMM (one launch on decode shapes, two otherwise), then the
    # epilogue (a no-op when the expand runs in the GEMM's epilogue)
    t_lora = None if skip0 else sum(st[k] - st0[k] for k in ("shrink_gemm", "epilogue"))
    ok = t_lora is not None and t_lora > 0.05
    t_step, t_fwd = el_step / steps, el_fwd / steps
    t_base = None if skip0 else el_base / steps
    out = {
        "workload": w.name, "T": T, "K": K, "d_in": w.d_in, "d_out": w.d_out,
        "adapters": w.n_adapters, "active_pairs": P, "segments": S, "R_used": R_used,
        "R_pairs": R_pairs, "rotation_copies": bn.R, "gemm": kind,
        "step_us": t_step * 1e6,
        "step": "forward + grads" if bn.grads else "forward",
        "tokens_per_s": T / t_step,
        "forward_us": t_fwd * 1e6, "forward_tokens_per_s": T / t_fwd,
        "apply_only_us": el_apply / steps * 1e6, "apply_only_tokens_per_s": T * steps / el_apply,
        "step_plan_shared_us": el_shared / steps * 1e6,
        "step_plan_shared_tokens_per_s": T * steps / el_shared,
        "forward_empty_plan_us": None if skip0 else t_base * 1e6,
        "step_us_graph_replay": None if el_graph is None else el_graph / steps * 1e6,
        "stages_us": st, "stages_us_empty_plan": st0,
        "hipblaslt_gemm_us": blas_us,
        "lora_path": {
            "t_us": t_lora if ok else None,
            "bytes": lb, "flops": lf,
            "GB_s": lb / (t_lora * 1e-6) / 1e9 if ok else None,
            "frac_hbm": lb / (t_lora * 1e-6) / 1e9 / HBM_PEAK_GBS if ok else None,
            "t_us_wall_difference": None if skip0 else (t_fwd - t_base) * 1e6,
            "method": "sum over the apply launches of (time with the plan - time with an empty "
                      "plan), HIP events",
        },
    }
    base_flops = 2.0 * T * w.d_in * w.d_out
    if full:
        out["_roofline"] = gemm_roofline(w, bn.L, B, kind, st, base_flops, P, R_pairs, R_used, e)
        out["_lf"] = lf
    if w.merge_ids is not None:
        m_ids = D.to_device(np.asarray(w.merge_ids, np.int32), "cuda")
        plus = D.to_device(np.ones(len(w.merge_ids), np.float32), "cuda")
        minus = D.to_device(-np.ones(len(w.merge_ids), np.float32), "cuda")

        def merge_call(i):
            B.lora_merge_delta(bn.copies[(i // 2) % bn.R].W_t, bn.L.pool, m_ids,
                               plus if i % 2 == 0 else minus, len(w.merge_ids))
        t_m = bn.event_us(merge_call, 2 * min(bn.R, 8), 5)
        rsum = int(sum(int(w.rank[a]) for a in w.merge_ids))
        mb = 2 * w.d_in * w.d_out * e + rsum * (w.d_in + w.d_out) * e
        out["merge"] = {"adapters": len(w.merge_ids), "us": t_m, "bytes": mb, "GB_s": mb / t_m / 1e3,
                        "frac_hbm": mb / t_m / 1e3 / HBM_PEAK_GBS,
                        "flops": 2.0 * w.d_in * w.d_out * rsum}
        # the same merge on every rotated copy as one layer each: one launch
        # for all of them (lora_merge_delta_layers) against one launch per layer
        Ws = [c.W_t for c in bn.copies]
        pools = [c.pool for c in bn.copies]

        def merge_layers_call(i):
            B.lora_merge_delta_layers(Ws, pools, m_ids, plus if i % 2 == 0 else minus,
                                      len(w.merge_ids))

        def merge_each_call(i):
            for W, p in zip(Ws, pools):
                B.lora_merge_delta(W, p, m_ids, plus if i % 2 == 0 else minus, len(w.merge_ids))
        t_ml = bn.event_us(merge_layers_call, 8, 5)
        t_me = bn.event_us(merge_each_call, 8, 5)
        out["merge_layers"] = {"layers": bn.R, "us": t_ml, "us_one_launch_per_layer": t_me,
                               "GB_s": bn.R * mb / t_ml / 1e3,
                               "frac_hbm": bn.R * mb / t_ml / 1e3 / HBM_PEAK_GBS}
    if bn.grads:
        # input gradient dX of the same batch (after lora_grad, which leaves G)
        Wn = bn.L.weight_transposed()
        dX, xws = bn.L.grad_x_buffers()
        c0 = bn.copies[0]
        bn.step(c0)

        def gx_call(i):
            B.lora_grad_x(c0.dY, Wn, c0.mask, T, K, c0.pool, c0.plan, bn.gws, bn.L.max_rank, dX,
                          xws)
        t_x = bn.event_us(gx_call, 8, 5)
        xf = 2.0 * T * w.d_in * w.d_out + 2.0 * R_pairs * w.d_in
        out["grad_x"] = {"us": t_x, "TFLOP_s": xf / t_x / 1e6,
                         "frac_mfma": xf / t_x / 1e6 / MFMA_BF16_PEAK_TFLOPS,
                         "tokens_per_s": T / (t_x * 1e-6)}
        del Wn, dX, xws
        t_g = st["grad"]
        gb = (T * w.d_out * e + T * w.d_in * (e + (1 if w.keep_mask is not None else 0))
              + R_used * (w.d_in + w.d_out) * (e + 4) + 8 * R_pairs)
        out["grads"] = {"us": t_g, "bytes": gb, "GB_s": gb / t_g / 1e3,
                        "frac_hbm": gb / t_g / 1e3 / HBM_PEAK_GBS,
                        "flops": 2.0 * R_pairs * (2 * w.d_out + w.d_in)}
    if args.residency and w.n_adapters >= 256 and not bn.grads:
        out["residency"] = residency_run(w, bn, args, torch, np, B, D)
    del bn
    torch.cuda.empty_cache()
    return out


def residency_run(w, bn, args, torch, np, B, D):
    """The pool held to --residency-frac of the fleet's rank rows, filled from
    a pinned host store: batch b + 1's copies (a gather kernel reading the
    device-mapped store, or one copy per page run where the store cannot be
    mapped, on a side stream) overlap batch b's forward; against the same
    batches on the fully resident pool."""
    from lora_adapter_amd import workloads as wl
    rows = np.concatenate([w.page_ids[w.page_start[a]:w.page_start[a + 1]]
                           for a in range(w.n_adapters)]).astype(np.int64)
    store_row = w.page_start[:-1].astype(np.int64)
    sa = D.to_device(w.a_pages[rows], "cpu").pin_memory()
    sb = D.to_device(w.b_pages[rows], "cpu").pin_memory()
    n_pages = int(args.residency_frac * int(w.rank.sum()))
    ap = torch.empty((n_pages, w.d_in), dtype=torch.bfloat16, device="cuda")
    bp = torch.empty((n_pages, w.d_out), dtype=torch.bfloat16, device="cuda")
    res = B.Residency(B.LORA_BF16, w.d_in, w.d_out, w.rank, store_row, sa, sb, ap, bp, bn.L.scale)
    side = torch.cuda.Stream()
    rng = np.random.default_rng(1234)
    nb = 40
    batches = [wl.zipf_ids(rng, w.T, w.n_adapters).reshape(w.T, 1) for _ in range(nb)]
    dev_ids = [D.to_device(b, "cuda") for b in batches]
    c = bn.copies[0]
    L = bn.L

    def loop(managed):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(nb):
            pool = res.prepare(batches[i], side) if managed else c.pool
            B.lora_forward(dev_ids[i], L.gates, w.T, w.K, c.X, c.W_t, c.Y, None, 1.0, pool, c.plan,
                           c.ws)
            if managed:
                res.finish()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) / nb

    loop(True)                       # warm: fill the pool once
    s0 = res.stats()
    t_managed = loop(True)
    s1 = res.stats()
    t_resident = loop(False)
    res.close()
    moved = (s1["bytes"] - s0["bytes"]) / nb
    return {"pool_fraction": args.residency_frac, "pool_pages": n_pages,
            "fleet_rank_rows": int(w.rank.sum()), "batches": nb,
            "step_us_managed": t_managed * 1e6, "step_us_resident": t_resident * 1e6,
            "copied_bytes_per_batch": moved,
            "evictions_per_batch": (s1["evictions"] - s0["evictions"]) / nb,
            "h2d_GB_s_lower_bound": moved / t_managed / 1e9,
            "note": "each batch's missing adapters copied from the pinned host store on a "
                    "side stream while the previous batch computes; wall time per batch over "
                    "40 Zipf batches"}


def gemm_roofline(w, L, B, kind, st, base_flops, P, R_pairs, R_used, e):
    """Roofline entry of the launch that runs the base GEMM, from its
    HIP-event duration.  On decode shapes that launch also runs the per-slot
    shrink (its bytes add the used A pages, each once, U and the slot
    descriptors) and builds the plan; on stream-K shapes it builds the plan
    (its bytes add the plan's inputs); fused, it runs the expand (its flops
    add 2 R_pairs d_out)."""
    name = GEMM_KERNEL[kind]
    alg_bytes = (w.d_in * w.d_out + w.T * w.d_in) * e
    flops = base_flops
    if kind == "fused":
        flops += 2.0 * R_pairs * w.d_out
        t_us = st["gemm"]
    elif kind == "decode":
        t_us = st["fwd_gemm"]
        alg_bytes += R_used * w.d_in * e + 4 * R_pairs + 16 * w.T * w.K
        alg_bytes += w.T * w.d_in if L.keep_mask is not None else 0
        flops += 2.0 * R_pairs * w.d_in
    elif kind in ("streamk", "f32"):
        t_us = st["fwd_gemm"]
        alg_bytes += 8 * w.T * w.K + 8 * w.n_adapters + 4 * R_used
    else:
        t_us = st["gemm"]
    intensity = base_flops / ((w.d_in * w.d_out + w.T * w.d_in + w.T * w.d_out) * e)
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


def tsqr_bench(torch, np, B):
    """Factor construction for a fleet of 1024 rank-16 adapters of a 4096 x
    4096 projection (bf16 pages, seeded synthetic): the batched QR of every A
    (lora_tsqr, with Q), and the whole recompression to retained ranks
    (lora_compress: QRs of A and B^T, core SVDs, new factors); torch's batched
    QR (the ROCm library routine) on the same A matrices in float32 beside it,
    as context."""
    M, n, d = 1024, 16, 4096
    g = torch.Generator(device="cuda").manual_seed(77)
    a = (torch.randn((M * n, d), generator=g, device="cuda") / 8).to(torch.bfloat16)
    b = (torch.randn((M * n, d), generator=g, device="cuda") * 0.14).to(torch.bfloat16)
    cols = torch.arange(M * n, dtype=torch.int32, device="cuda")
    Qt = torch.empty((M, n, d), dtype=torch.float32, device="cuda")
    R = torch.empty((M, n, n), dtype=torch.float32, device="cuda")
    ws = torch.empty(B.lora_tsqr_workspace_bytes(M, d, n), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()

    def ev(fn, reps=5):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / reps
    t_tsqr = ev(lambda: B.lora_tsqr(a, B.LORA_BF16, cols, M, d, n, Qt, R, ws))
    A32 = a.float().view(M, n, d).transpose(1, 2).contiguous()
    try:
        t_lib = ev(lambda: torch.linalg.qr(A32, mode="reduced"), reps=3)
    except Exception:
        t_lib = None
    rank = torch.full((M,), n, dtype=torch.int32, device="cuda")
    ps = torch.arange(0, M * n + 1, n, dtype=torch.int32, device="cuda")
    scale = torch.ones(M, dtype=torch.float32, device="cuda")
    pool = B.Pool(B.LORA_BF16, d, d, a, b, rank, ps, cols, scale)
    oa, ob = torch.empty_like(a), torch.empty_like(b)
    ork = torch.empty(M, dtype=torch.int32, device="cuda")
    osg = torch.empty((M, n), dtype=torch.float32, device="cuda")
    cws = torch.empty(B.lora_compress_workspace_bytes(M, d, d, n), dtype=torch.uint8, device="cuda")
    ad = torch.arange(M, dtype=torch.int32, device="cuda")
    t_cmp = ev(lambda: B.lora_compress(pool, ad, M, n, 1, 1.0, 0.9, 1, oa, ob, ork, osg, cws), reps=3)
    in_bytes = M * n * d * 2
    out = {"modules": M, "rank": n, "rows": d, "tsqr_us": t_tsqr,
           "tsqr_input_GB_s": in_bytes / t_tsqr / 1e3,
           "torch_linalg_qr_fp32_us": t_lib,
           "compress_us": t_cmp, "compress_mean_retained_rank": float(ork.float().mean()),
           "note": "lora_tsqr forms Q and R from bf16 pages; torch.linalg.qr is given the same "
                   "matrices as float32 (M, 4096, 16), context only"}
    del a, b, Qt, R, ws, A32, oa, ob, cws
    torch.cuda.empty_cache()
    return out


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
    print(f"bench: workload {w.name}", file=sys.stderr, flush=True)
    head = measure(w, args, torch, np, B, D, args.steps, args.warmup, full=True)
    roofline = head.pop("_roofline")
    head.pop("_lf")
    e = 2 if w.dtype == "bf16" else 4
    t_step = head["step_us"] * 1e-6
    base_flops = 2.0 * w.T * w.d_in * w.d_out
    layer_bytes = (w.d_in * w.d_out + w.T * (w.d_in + w.d_out)) * e + head["lora_path"]["bytes"]

    others = {}
    for tok in [s for s in args.others.split(",") if s.strip()]:
        i = int(tok)
        if i == args.workload:
            continue
        wo = wl.config(i)
        print(f"bench: workload {wo.name}", file=sys.stderr, flush=True)
        r = measure(wo, args, torch, np, B, D, args.other_steps, max(5, args.warmup // 2),
                    full=True)
        r["roofline"] = r.pop("_roofline")
        r.pop("_lf")
        others[wo.name] = r
        del wo

    fleet = None if args.no_tsqr else tsqr_bench(torch, np, B)

    out = {
        "metric": METRIC,
        "value": head["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": t_step * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "T": w.T, "K": w.K, "d_in": w.d_in, "d_out": w.d_out,
                   "adapters": w.n_adapters, "ranks": sorted(set(w.rank.tolist()))[:8],
                   "step": head["step"], "launch": "eager",
                   "rotation_copies": head["rotation_copies"]},
        "roofline": roofline,
        "value_forward": head["forward_tokens_per_s"],
        "value_apply_only": head["apply_only_tokens_per_s"],
        "value_plan_shared": head["step_plan_shared_tokens_per_s"],
        "lora_path": head["lora_path"],
        "layer": {"bytes": layer_bytes, "GB_s": layer_bytes / t_step / 1e9,
                  "TFLOP_s": (base_flops + head["lora_path"]["flops"]) / t_step / 1e12},
        "headline": head,
        "workloads": others,
        "fleet_compression": fleet,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
    print(json.dumps(out), flush=True)


# ---------------------------------------------------------------- counters

def kernel_source_hash():
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "lora_adapter_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        if f.endswith((".hip", ".h")):
            with open(os.path.join(csrc, f), "rb") as fh:
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
    # the instantiation of this kernel with the most dispatches in the run,
    # among entries taken from the current sources
    h = kernel_source_hash()
    cands = [v for k, v in table.items()
             if k.endswith("|" + workload) and (k.startswith(kernel + "<") or k.startswith(kernel + "|"))
             and v.get("source_sha256_16") == h]
    if not cands:
        return None
    ent = max(cands, key=lambda v: v["fetch"]["dispatches"])
    return ent.get("hbm_bytes_per_launch")


COPY_PROBE_BYTES = 256 << 20
KERNELS = ("decode_gemm_slot_kernel", "gemm_tile_plan_kernel", "decode_gemm_shrink_kernel",
           "gemm_decode_kernel", "gemm_tile_kernel", "gemm_f32_kernel", "shrink_both_kernel",
           "shrink_units_kernel", "shrink_tile_kernel", "epilogue_kernel", "plan_kernel",
           "merge_mfma_kernel", "seg_outer_mfma_kernel", "seg_outer_reduce_kernel",
           "seg_g_reduce_kernel", "transpose_kernel", "merge_layers_mfma_kernel")


def pmc_summary(workload_id, fetch_csv, write_csv):
    """HBM bytes per launch of every library kernel in two rocprofv3 --pmc
    runs (FETCH_SIZE, then WRITE_SIZE, KiB per dispatch), each scaled by the
    copy probe's reading of the same counter against the bytes that copy must
    move."""
    import csv
    import numpy as np
    from lora_adapter_amd import workloads as wl

    def name_of(k):
        """The kernel's name with its template arguments (one entry per
        instantiation), for the library's kernels."""
        import re
        for n in KERNELS:
            m = re.search(r"(?:::|^)(" + n + r"(?:<[^()]*>)?)\(", k)
            if m:
                return m.group(1)
        return None

    def per_kernel(path, counter):
        vals = {}
        with open(path) as fh:
            for r in csv.DictReader(fh):
                if r["Counter_Name"] != counter:
                    continue
                vals.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]) * 1024.0)
        return vals

    w = wl.config(workload_id)
    res = {}
    for counter, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        vals = per_kernel(path, counter)
        copy = [v for k, vs in vals.items() if "copyBuffer" in k for v in vs
                if v > COPY_PROBE_BYTES / 2]
        if not copy:
            raise SystemExit(f"{path}: no copy probe dispatches for {counter}")
        scale = COPY_PROBE_BYTES / float(np.median(copy))
        for k, vs in vals.items():
            n = name_of(k)
            if n is None:
                continue
            res.setdefault(n, {})[counter] = {"raw_bytes_median": float(np.median(vs)),
                                              "copy_scale": scale,
                                              "bytes": float(np.median(vs)) * scale,
                                              "dispatches": len(vs)}
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as fh:
            table = json.load(fh)
    except (OSError, ValueError):
        table = {}
    for n, d in res.items():
        if "FETCH_SIZE" not in d or "WRITE_SIZE" not in d:
            continue
        table[n + "|" + w.name] = {
            "hbm_bytes_per_launch": d["FETCH_SIZE"]["bytes"] + d["WRITE_SIZE"]["bytes"],
            "fetch": d["FETCH_SIZE"], "write": d["WRITE_SIZE"],
            "source_sha256_16": kernel_source_hash(),
        }
        print(n, json.dumps(table[n + "|" + w.name]))
    with open(path, "w") as fh:
        json.dump(table, fh, indent=1, sort_keys=True)


# ---------------------------------------------------------------- CPU oracle

def host_info():
    info = {"cpu_model": platform.processor() or "unknown", "numpy": None, "blas": None}
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    info["cpu_model"] = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    import numpy as np
    info["numpy"] = np.__version__
    try:
        from threadpoolctl import threadpool_info
        blas = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        if blas:
            info["blas"] = f"{blas[0].get('internal_api')} {blas[0].get('version')}"
            info["blas_threads"] = int(blas[0].get("num_threads", 1))
    except Exception:
        pass
    return info


def cpu_baseline(w, seconds):
    """The CPU oracle, untuned, on a bounded sample of the same workload: the
    plan, the forward and (when the workload trains) the gradients of a set
    of token rows spread over the batch, repeated for about `seconds`."""
    import numpy as np
    from lora_adapter_amd import workloads as wl
    from oracle import lora_oracle as O
    info = host_info()
    try:
        affinity = len(os.sched_getaffinity(0))
    except AttributeError:
        affinity = os.cpu_count() or 1
    n_rows = min(w.T, 256)
    rows = np.linspace(0, w.T - 1, n_rows).round().astype(np.int64)
    sw = wl.subset(w, rows) if n_rows < w.T else w
    n = 0
    t0 = time.perf_counter()
    while True:
        O.plan_workload(sw)
        O.apply_workload(sw)
        if sw.dY is not None:
            O.grad_workload(sw)
        n += 1
        el = time.perf_counter() - t0
        if el >= seconds or n >= 1000:
            break
    what = "plan + forward + grads" if sw.dY is not None else "plan + forward"
    return {"value": n_rows * n / el, "unit": "tokens/s",
            "cores": info.get("blas_threads", affinity), "kind": "oracle",
            "sample": f"{n} runs of the oracle's {what} (fp64 numpy) on {n_rows} token rows "
                      f"spread evenly over the batch of {w.T}, {el:.1f} s",
            "affinity_cpus": affinity, **info}


if __name__ == "__main__":
    main()
