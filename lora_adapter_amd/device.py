"""Device-side holder for one layer's tensors, plan and workspaces.

Uploads a workload (see workloads.py) into torch GPU tensors, owns the plan
and workspace buffers the C ABI needs, and calls the binding.  PyTorch is
used only to allocate device memory and to provide the stream.
"""
from __future__ import annotations

from typing import Optional

import numpy as np
import torch

from . import binding as B
from .workloads import Workload, bf16_bits_to_f32


def to_device(arr: Optional[np.ndarray], device: str):
    if arr is None:
        return None
    a = np.ascontiguousarray(arr)
    if a.dtype == np.uint16:                      # bf16 bits: torch has no uint16 math; bytes only
        return torch.from_numpy(a.view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(a).to(device)


def to_host(t: torch.Tensor) -> np.ndarray:
    """Device tensor -> numpy (bf16 returned as its uint16 bit pattern)."""
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def as_f64(a: np.ndarray) -> np.ndarray:
    return (bf16_bits_to_f32(a) if a.dtype == np.uint16 else a).astype(np.float64)


class DeviceLayer:
    """One projection layer of a workload, resident in HBM."""

    def __init__(self, w: Workload, device: str = "cuda", max_rank: Optional[int] = None):
        self.w = w
        self.device = device
        self.dtype = B.LORA_BF16 if w.dtype == "bf16" else B.LORA_F32
        self.T, self.K = w.T, w.K
        self.max_rank = max(1, int(w.rank.max()) if max_rank is None else max_rank)
        dv = lambda a: to_device(a, device)
        self.X = dv(w.X)
        self.W_t = dv(w.W_t)
        self.a_pages = dv(w.a_pages)
        self.b_pages = dv(w.b_pages)
        self.rank = dv(w.rank)
        self.page_start = dv(w.page_start)
        self.page_ids = dv(w.page_ids) if w.page_ids.size else torch.zeros(1, dtype=torch.int32, device=device)
        self.scale = dv(w.scale)
        self.ids = dv(w.ids)
        self.gates = dv(w.gates)
        self.keep_mask = dv(w.keep_mask)
        self.keep_scale = float(w.keep_scale)
        self.dY = dv(w.dY)
        self.pool = B.Pool(self.dtype, w.d_in, w.d_out, self.a_pages, self.b_pages, self.rank,
                           self.page_start, self.page_ids[:w.page_ids.size] if w.page_ids.size
                           else self.page_ids[:0], self.scale)
        ydt = torch.bfloat16 if self.dtype == B.LORA_BF16 else torch.float32
        self.Y = torch.empty((w.T, w.d_out), dtype=ydt, device=device)
        nplan = B.lora_plan_bytes(w.T, w.K, w.n_adapters)
        self.plan = torch.empty((nplan + 3) // 4, dtype=torch.int32, device=device)
        nws = B.lora_apply_workspace_bytes(w.T, w.K, w.d_in, w.d_out, self.max_rank, self.dtype)
        self.ws = torch.empty(nws, dtype=torch.uint8, device=device)
        self.layout = B.lora_plan_layout(w.T, w.K, w.n_adapters)

    # -- the C entry points ------------------------------------------------
    def run_plan(self, stream=None):
        B.lora_plan(self.ids, self.gates, self.T, self.K, self.pool, self.plan, stream)

    def run_apply(self, stream=None, Y=None, W_t=None):
        B.lora_apply(self.X, self.W_t if W_t is None else W_t, self.Y if Y is None else Y,
                     self.T, self.K, self.gates, self.keep_mask, self.keep_scale,
                     self.pool, self.plan, self.ws, stream)

    def run_shrink(self, stream=None):
        B.lora_shrink(self.X, self.keep_mask, self.keep_scale, self.T, self.K, self.gates,
                      self.pool, self.plan, self.ws, stream)

    def run_base_expand(self, stream=None, Y=None):
        B.lora_base_expand(self.X, self.W_t, self.Y if Y is None else Y, self.T, self.K,
                           self.pool, self.plan, self.ws, stream)

    def run_merge(self, W_t, merge_ids, coeffs, stream=None):
        mi = merge_ids if torch.is_tensor(merge_ids) else to_device(np.asarray(merge_ids, np.int32), self.device)
        co = coeffs if torch.is_tensor(coeffs) else to_device(np.asarray(coeffs, np.float32), self.device)
        B.lora_merge_delta(W_t, self.pool, mi, co, int(mi.numel()), stream)
        return mi, co

    def grad_buffers(self):
        w = self.w
        dA = torch.full((w.n_pages, w.d_in), float("nan"), dtype=torch.float32, device=self.device)
        dB = torch.full((w.n_pages, w.d_out), float("nan"), dtype=torch.float32, device=self.device)
        n = B.lora_grad_workspace_bytes(w.T, w.K, w.n_adapters, w.d_in, w.d_out, self.max_rank, self.dtype)
        gws = torch.empty(n, dtype=torch.uint8, device=self.device)
        return dA, dB, gws

    def run_grad(self, dA, dB, gws, stream=None):
        B.lora_grad(self.X, self.keep_mask, self.keep_scale, self.dY, self.T, self.K,
                    self.gates, self.pool, self.plan, self.ws, dA, dB, self.max_rank, gws, stream)

    def weight_transposed(self, stream=None):
        """W [d_in][d_out] (the frozen weight in its mathematical orientation)
        from W_t, for the input gradient."""
        w = self.w
        Wn = torch.empty((w.d_in, w.d_out), dtype=self.W_t.dtype, device=self.device)
        B.lora_transpose(self.W_t, Wn, w.d_out, w.d_in, self.dtype, stream)
        return Wn

    def grad_x_buffers(self):
        w = self.w
        dX = torch.empty((w.T, w.d_in), dtype=self.Y.dtype, device=self.device)
        n = B.lora_grad_x_workspace_bytes(w.T, w.d_in, w.d_out, self.dtype)
        return dX, torch.empty(n, dtype=torch.uint8, device=self.device)

    def run_grad_x(self, Wn, gws, dX, xws, stream=None):
        B.lora_grad_x(self.dY, Wn, self.keep_mask, self.T, self.K, self.pool, self.plan, gws,
                      self.max_rank, dX, xws, stream)

    # -- reading results ---------------------------------------------------
    def read_plan(self) -> dict:
        P = self.plan.cpu().numpy()
        TK = self.T * self.K
        o = [x // 4 for x in self.layout]
        h = P[o[0]:o[0] + 16]
        nP, nS = int(h[B.PH_PAIRS]), int(h[B.PH_SEGS])
        return {"header": h.copy(), "pair_tk": P[o[1]:o[1] + nP].copy(),
                "seg_adapter": P[o[2]:o[2] + nS].copy(), "seg_off": P[o[3]:o[3] + nS + 1].copy(),
                "seg_row_off": P[o[4]:o[4] + nS + 1].copy(),
                "bucket_seg_off": P[o[5]:o[5] + 10].copy(), "u_off": P[o[6]:o[6] + nP + 1].copy(),
                "slot_pos": P[o[7]:o[7] + TK].copy(), "pair_adapter": P[o[8]:o[8] + nP].copy()}

    def U(self) -> np.ndarray:
        """The packed float32 U written by the shrink stage."""
        n = int(self.read_plan()["header"][B.PH_RPAIRS])
        o = B.lora_apply_u_offset(self.T, self.K, self.w.d_in, self.w.d_out, self.dtype)
        return self.ws[o:o + 4 * n].view(torch.float32).cpu().numpy()

    def Y_host(self) -> np.ndarray:
        return to_host(self.Y)
