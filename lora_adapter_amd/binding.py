"""Thin ctypes binding of liblora (the C ABI in include/lora.h).

Argument marshalling only: every step of the layer runs in the HIP library.
Tensors are torch tensors on the GPU (PyTorch serves as the device allocator
and stream provider); their data pointers are handed to the C entry points
with the current torch stream.  If liblora.so is missing, loading fails loudly:
there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

PKG = os.path.dirname(os.path.abspath(__file__))
# LORA_ADAPTER_LIB names another build of the same library (the host-sanitized
# one that the CPU tests load under the address sanitizer runtime)
LIB_PATH = os.environ.get("LORA_ADAPTER_LIB") or os.path.join(PKG, "liblora.so")

LORA_OK, LORA_ERR_INVALID_ARG, LORA_ERR_UNSUPPORTED, LORA_ERR_CAPACITY, LORA_ERR_DEVICE = range(5)
LORA_F32, LORA_BF16 = 0, 1
LORA_MAX_RANK = 1024
LORA_MAX_K = 8
DEVERR_BAD_ID, DEVERR_BAD_RANK, DEVERR_BAD_POOL, DEVERR_CAPACITY = 1, 2, 4, 8
PH_PAIRS, PH_SEGS, PH_ERR, PH_RPAIRS, PH_RUSED, PH_T, PH_K, PH_N = range(8)

EXPORTS = (
    "lora_abi_version", "lora_status_string", "lora_plan_bytes", "lora_plan_layout", "lora_plan",
    "lora_plan_header",
    "lora_apply_workspace_bytes", "lora_apply_u_offset", "lora_shrink", "lora_base_expand",
    "lora_base_gemm", "lora_expand_epilogue", "lora_shrink_gemm", "lora_apply",
    "lora_forward_gemm", "lora_forward_finish", "lora_forward", "lora_forward_noalloc_bytes",
    "lora_forward_noalloc", "lora_merge_delta", "lora_grad_workspace_bytes", "lora_grad",
    "lora_grad_x_workspace_bytes", "lora_grad_x", "lora_transpose", "lora_merge_delta_layers",
    "lora_page_table_create", "lora_page_table_destroy", "lora_page_table_admit",
    "lora_page_table_tables", "lora_residency_table_ints", "lora_residency_create",
    "lora_residency_destroy", "lora_residency_prepare", "lora_residency_finish",
    "lora_residency_stats", "lora_residency_page_table", "lora_tsqr_workspace_bytes", "lora_tsqr",
    "lora_compress_workspace_bytes", "lora_compress",
)


class LoraError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} failed: status {status} ({status_string(status)})")
        self.status = status


class PoolDesc(ctypes.Structure):
    _fields_ = [
        ("dtype", ctypes.c_int32), ("d_in", ctypes.c_int32), ("d_out", ctypes.c_int32),
        ("n_adapters", ctypes.c_int32), ("n_pages", ctypes.c_int64), ("n_page_ids", ctypes.c_int64),
        ("a_pages", ctypes.c_void_p), ("b_pages", ctypes.c_void_p), ("rank", ctypes.c_void_p),
        ("page_start", ctypes.c_void_p), ("page_ids", ctypes.c_void_p), ("scale", ctypes.c_void_p),
    ]


class LayerDesc(ctypes.Structure):
    _fields_ = [("W_t", ctypes.c_void_p), ("pool", PoolDesc)]


class PageCopy(ctypes.Structure):
    _fields_ = [("adapter", ctypes.c_int32), ("row", ctypes.c_int32), ("page", ctypes.c_int32),
                ("count", ctypes.c_int32)]


class ResidencyConfig(ctypes.Structure):
    _fields_ = [("dtype", ctypes.c_int32), ("d_in", ctypes.c_int32), ("d_out", ctypes.c_int32),
                ("n_adapters", ctypes.c_int32), ("n_pages", ctypes.c_int64),
                ("rank", ctypes.c_void_p), ("store_row", ctypes.c_void_p),
                ("store_a", ctypes.c_void_p), ("store_b", ctypes.c_void_p),
                ("a_pages", ctypes.c_void_p), ("b_pages", ctypes.c_void_p),
                ("scale", ctypes.c_void_p), ("tables", ctypes.c_void_p),
                ("staging", ctypes.c_void_p)]


_lib = None
_I32, _I64, _SZ, _VP, _F32 = ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_float
_PD = ctypes.POINTER(PoolDesc)

_PROTOS = {
    "lora_abi_version": (_I32, []),
    "lora_status_string": (ctypes.c_char_p, [_I32]),
    "lora_plan_bytes": (_SZ, [_I32, _I32, _I32]),
    "lora_plan_layout": (_I32, [_I32, _I32, _I32, ctypes.POINTER(_I64)]),
    "lora_plan": (_I32, [_VP, _VP, _I32, _I32, _PD, _VP, _SZ, _VP]),
    "lora_plan_header": (_I32, [_VP, ctypes.POINTER(_I32), _VP]),
    "lora_apply_workspace_bytes": (_SZ, [_I32, _I32, _I32, _I32, _I32, _I32]),
    "lora_apply_u_offset": (_SZ, [_I32, _I32, _I32, _I32, _I32]),
    "lora_shrink": (_I32, [_VP, _VP, _F32, _I32, _I32, _VP, _PD, _VP, _VP, _SZ, _VP]),
    "lora_base_expand": (_I32, [_VP, _VP, _VP, _I32, _I32, _PD, _VP, _VP, _SZ, _VP]),
    "lora_base_gemm": (_I32, [_VP, _VP, _VP, _I32, _I32, _PD, _VP, _VP, _SZ, _VP]),
    "lora_expand_epilogue": (_I32, [_VP, _VP, _VP, _I32, _I32, _PD, _VP, _VP, _SZ, _VP]),
    "lora_shrink_gemm": (_I32, [_VP, _VP, _VP, _I32, _I32, _VP, _VP, _F32, _PD, _VP, _VP, _SZ, _VP]),
    "lora_apply": (_I32, [_VP, _VP, _VP, _I32, _I32, _VP, _VP, _F32, _PD, _VP, _VP, _SZ, _VP]),
    "lora_forward_gemm": (_I32, [_VP, _VP, _I32, _I32, _VP, _VP, _VP, _VP, _F32, _PD, _VP, _SZ,
                                 _VP, _SZ, _VP]),
    "lora_forward_finish": (_I32, [_VP, _VP, _I32, _I32, _VP, _VP, _VP, _VP, _F32, _PD, _VP, _SZ,
                                   _VP, _SZ, _VP]),
    "lora_forward": (_I32, [_VP, _VP, _I32, _I32, _VP, _VP, _VP, _VP, _F32, _PD, _VP, _SZ, _VP,
                            _SZ, _VP]),
    "lora_forward_noalloc_bytes": (_SZ, [_I32, _I32, _I32, _I32, _I32, _I32, _I32]),
    "lora_forward_noalloc": (_I32, [_VP, _VP, _I32, _I32, _VP, _VP, _VP, _VP, _F32, _PD, _I32,
                                    _VP]),
    "lora_merge_delta": (_I32, [_VP, _PD, _VP, _VP, _I32, _VP]),
    "lora_grad_workspace_bytes": (_SZ, [_I32, _I32, _I32, _I32, _I32, _I32, _I32]),
    "lora_grad": (_I32, [_VP, _VP, _F32, _VP, _I32, _I32, _VP, _PD, _VP, _VP, _SZ, _VP, _VP,
                         _I32, _VP, _SZ, _VP]),
    "lora_grad_x_workspace_bytes": (_SZ, [_I32, _I32, _I32, _I32]),
    "lora_grad_x": (_I32, [_VP, _VP, _VP, _I32, _I32, _PD, _VP, _VP, _SZ, _I32, _VP, _VP, _SZ,
                           _VP]),
    "lora_transpose": (_I32, [_VP, _VP, _I32, _I32, _I32, _VP]),
    "lora_merge_delta_layers": (_I32, [ctypes.POINTER(LayerDesc), _I32, _VP, _VP, _I32, _VP]),
    "lora_page_table_create": (_I32, [_VP, _I32, _I64, ctypes.POINTER(_VP)]),
    "lora_page_table_destroy": (None, [_VP]),
    "lora_page_table_admit": (_I32, [_VP, _VP, _I64, ctypes.POINTER(PageCopy), _I64,
                                     ctypes.POINTER(_I64), ctypes.POINTER(_I32), _I64,
                                     ctypes.POINTER(_I64)]),
    "lora_page_table_tables": (_I32, [_VP, ctypes.POINTER(_I32), ctypes.POINTER(_I32),
                                      ctypes.POINTER(_I32), ctypes.POINTER(_I64)]),
    "lora_residency_table_ints": (_SZ, [_I32, _I64]),
    "lora_residency_create": (_I32, [ctypes.POINTER(ResidencyConfig), ctypes.POINTER(_VP)]),
    "lora_residency_destroy": (None, [_VP]),
    "lora_residency_prepare": (_I32, [_VP, _VP, _I64, _VP, _VP, _PD]),
    "lora_residency_finish": (_I32, [_VP, _VP]),
    "lora_residency_stats": (_I32, [_VP, ctypes.POINTER(_I64)]),
    "lora_residency_page_table": (_VP, [_VP]),
    "lora_tsqr_workspace_bytes": (_SZ, [_I32, _I32, _I32]),
    "lora_tsqr": (_I32, [_VP, _I32, _VP, _I32, _I32, _I32, _VP, _VP, _VP, _SZ, _VP]),
    "lora_compress_workspace_bytes": (_SZ, [_I32, _I32, _I32, _I32]),
    "lora_compress": (_I32, [_PD, _VP, _I32, _I32, _I32, _F32, _F32, _I32, _VP, _VP, _VP, _VP, _VP,
                             _SZ, _VP]),
}


def lib() -> ctypes.CDLL:
    """Load liblora.so (built in-tree); raise if it is not there."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m lora_adapter_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _PROTOS.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().lora_status_string(int(status)).decode()


def _check(fn: str, status: int):
    if status != LORA_OK:
        raise LoraError(fn, status)


def _ptr(t) -> Optional[int]:
    return None if t is None else int(t.data_ptr())


def _stream(stream) -> Optional[int]:
    if stream is not None:
        return int(getattr(stream, "cuda_stream", stream))
    import torch
    return int(torch.cuda.current_stream().cuda_stream)


# ---------------------------------------------------------------- pool

class Pool:
    """Device tensors of one adapter pool and the matching C descriptor."""

    def __init__(self, dtype: int, d_in: int, d_out: int, a_pages, b_pages, rank, page_start,
                 page_ids, scale):
        self.tensors = (a_pages, b_pages, rank, page_start, page_ids, scale)
        self.dtype, self.d_in, self.d_out = dtype, d_in, d_out
        self.n_adapters = int(rank.numel())
        self.desc = PoolDesc(dtype, d_in, d_out, self.n_adapters, int(a_pages.shape[0]),
                             int(page_ids.numel()), _ptr(a_pages), _ptr(b_pages), _ptr(rank),
                             _ptr(page_start), _ptr(page_ids) if page_ids.numel() else None,
                             _ptr(scale))

    @property
    def ref(self):
        return ctypes.byref(self.desc)


# ---------------------------------------------------------------- entry points

def lora_abi_version() -> int:
    return int(lib().lora_abi_version())


def lora_plan_bytes(T: int, K: int, n_adapters: int) -> int:
    return int(lib().lora_plan_bytes(T, K, n_adapters))


def lora_plan_layout(T: int, K: int, n_adapters: int):
    out = (_I64 * 9)()
    _check("lora_plan_layout", lib().lora_plan_layout(T, K, n_adapters, out))
    return [int(v) for v in out]


def lora_plan(ids, gates, T: int, K: int, pool: Pool, plan, stream=None):
    _check("lora_plan", lib().lora_plan(_ptr(ids), _ptr(gates), T, K, pool.ref, _ptr(plan),
                                        plan.numel() * plan.element_size(), _stream(stream)))


def lora_plan_header(plan, stream=None):
    """The plan's 16 header words (waits for the work queued on the stream)."""
    out = (_I32 * 16)()
    _check("lora_plan_header", lib().lora_plan_header(_ptr(plan), out, _stream(stream)))
    return [int(v) for v in out]


def lora_apply_workspace_bytes(T: int, K: int, d_in: int, d_out: int, max_rank: int, dtype: int) -> int:
    return int(lib().lora_apply_workspace_bytes(T, K, d_in, d_out, max_rank, dtype))


def lora_apply_u_offset(T: int, K: int, d_in: int, d_out: int, dtype: int) -> int:
    return int(lib().lora_apply_u_offset(T, K, d_in, d_out, dtype))


def lora_shrink(X, keep_mask, keep_scale: float, T: int, K: int, gates, pool: Pool, plan, ws,
                stream=None):
    _check("lora_shrink", lib().lora_shrink(_ptr(X), _ptr(keep_mask), float(keep_scale), T, K,
                                            _ptr(gates), pool.ref, _ptr(plan), _ptr(ws),
                                            ws.numel() * ws.element_size(), _stream(stream)))


def lora_base_expand(X, W_t, Y, T: int, K: int, pool: Pool, plan, ws, stream=None):
    _check("lora_base_expand", lib().lora_base_expand(_ptr(X), _ptr(W_t), _ptr(Y), T, K,
                                                      pool.ref, _ptr(plan), _ptr(ws),
                                                      ws.numel() * ws.element_size(), _stream(stream)))


def lora_base_gemm(X, W_t, Y, T: int, K: int, pool: Pool, plan, ws, stream=None):
    _check("lora_base_gemm", lib().lora_base_gemm(_ptr(X), _ptr(W_t), _ptr(Y), T, K,
                                                  pool.ref, _ptr(plan), _ptr(ws),
                                                  ws.numel() * ws.element_size(), _stream(stream)))


def lora_expand_epilogue(X, W_t, Y, T: int, K: int, pool: Pool, plan, ws, stream=None):
    _check("lora_expand_epilogue", lib().lora_expand_epilogue(
        _ptr(X), _ptr(W_t), _ptr(Y), T, K, pool.ref, _ptr(plan), _ptr(ws),
        ws.numel() * ws.element_size(), _stream(stream)))


def lora_shrink_gemm(X, W_t, Y, T: int, K: int, gates, keep_mask, keep_scale: float, pool: Pool,
                     plan, ws, stream=None):
    _check("lora_shrink_gemm",
           lib().lora_shrink_gemm(_ptr(X), _ptr(W_t), _ptr(Y), T, K, _ptr(gates), _ptr(keep_mask),
                                  float(keep_scale), pool.ref, _ptr(plan), _ptr(ws),
                                  ws.numel() * ws.element_size(), _stream(stream)))


def lora_apply(X, W_t, Y, T: int, K: int, gates, keep_mask, keep_scale: float, pool: Pool,
               plan, ws, stream=None):
    _check("lora_apply", lib().lora_apply(_ptr(X), _ptr(W_t), _ptr(Y), T, K, _ptr(gates),
                                          _ptr(keep_mask), float(keep_scale), pool.ref, _ptr(plan),
                                          _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)))


def _forward_call(name, ids, gates, T, K, X, W_t, Y, keep_mask, keep_scale, pool, plan, ws, stream):
    _check(name, getattr(lib(), name)(
        _ptr(ids), _ptr(gates), T, K, _ptr(X), _ptr(W_t), _ptr(Y), _ptr(keep_mask),
        float(keep_scale), pool.ref, _ptr(plan), plan.numel() * plan.element_size(), _ptr(ws),
        ws.numel() * ws.element_size(), _stream(stream)))


def lora_forward_gemm(ids, gates, T: int, K: int, X, W_t, Y, keep_mask, keep_scale: float,
                      pool: Pool, plan, ws, stream=None):
    _forward_call("lora_forward_gemm", ids, gates, T, K, X, W_t, Y, keep_mask, keep_scale, pool,
                  plan, ws, stream)


def lora_forward_finish(ids, gates, T: int, K: int, X, W_t, Y, keep_mask, keep_scale: float,
                        pool: Pool, plan, ws, stream=None):
    _forward_call("lora_forward_finish", ids, gates, T, K, X, W_t, Y, keep_mask, keep_scale, pool,
                  plan, ws, stream)


def lora_forward(ids, gates, T: int, K: int, X, W_t, Y, keep_mask, keep_scale: float, pool: Pool,
                 plan, ws, stream=None):
    _forward_call("lora_forward", ids, gates, T, K, X, W_t, Y, keep_mask, keep_scale, pool, plan,
                  ws, stream)


def lora_forward_noalloc_bytes(T: int, K: int, n_adapters: int, d_in: int, d_out: int,
                               max_rank: int, dtype: int) -> int:
    return int(lib().lora_forward_noalloc_bytes(T, K, n_adapters, d_in, d_out, max_rank, dtype))


def lora_forward_noalloc(ids, gates, T: int, K: int, X, W_t, Y, keep_mask, keep_scale: float,
                         pool: Pool, max_rank: int, stream=None):
    _check("lora_forward_noalloc", lib().lora_forward_noalloc(
        _ptr(ids), _ptr(gates), T, K, _ptr(X), _ptr(W_t), _ptr(Y), _ptr(keep_mask),
        float(keep_scale), pool.ref, int(max_rank), _stream(stream)))


def lora_merge_delta(W_t, pool: Pool, merge_ids, coeffs, m: int, stream=None):
    _check("lora_merge_delta", lib().lora_merge_delta(_ptr(W_t), pool.ref, _ptr(merge_ids),
                                                      _ptr(coeffs), m, _stream(stream)))


def lora_grad_workspace_bytes(T: int, K: int, n_adapters: int, d_in: int, d_out: int, max_rank: int,
                              dtype: int) -> int:
    return int(lib().lora_grad_workspace_bytes(T, K, n_adapters, d_in, d_out, max_rank, dtype))


def lora_grad(X, keep_mask, keep_scale: float, dY, T: int, K: int, gates, pool: Pool, plan,
              apply_ws, dA_pages, dB_pages, max_rank: int, ws, stream=None):
    _check("lora_grad", lib().lora_grad(_ptr(X), _ptr(keep_mask), float(keep_scale), _ptr(dY), T, K,
                                        _ptr(gates), pool.ref, _ptr(plan), _ptr(apply_ws),
                                        apply_ws.numel() * apply_ws.element_size(), _ptr(dA_pages),
                                        _ptr(dB_pages), max_rank, _ptr(ws),
                                        ws.numel() * ws.element_size(), _stream(stream)))


def lora_grad_x_workspace_bytes(T: int, d_in: int, d_out: int, dtype: int) -> int:
    return int(lib().lora_grad_x_workspace_bytes(T, d_in, d_out, dtype))


def lora_grad_x(dY, W, keep_mask, T: int, K: int, pool: Pool, plan, grad_ws, max_rank: int, dX,
                ws, stream=None):
    _check("lora_grad_x", lib().lora_grad_x(
        _ptr(dY), _ptr(W), _ptr(keep_mask), T, K, pool.ref, _ptr(plan), _ptr(grad_ws),
        grad_ws.numel() * grad_ws.element_size(), int(max_rank), _ptr(dX), _ptr(ws),
        ws.numel() * ws.element_size(), _stream(stream)))


def lora_transpose(src, dst, rows: int, cols: int, dtype: int, stream=None):
    _check("lora_transpose", lib().lora_transpose(_ptr(src), _ptr(dst), rows, cols, dtype,
                                                  _stream(stream)))


def lora_merge_delta_layers(Ws, pools, merge_ids, coeffs, m: int, stream=None):
    """The same signed merge on every (W_t, pool) pair (one launch per up to
    16 layers of the MFMA form)."""
    n = len(Ws)
    arr = (LayerDesc * max(n, 1))()
    for i, (W, p) in enumerate(zip(Ws, pools)):
        arr[i].W_t = _ptr(W)
        arr[i].pool = p.desc
    _check("lora_merge_delta_layers", lib().lora_merge_delta_layers(
        arr, n, _ptr(merge_ids), _ptr(coeffs), m, _stream(stream)))


# ---------------------------------------------------------------- pool residency

def _host_i32(a):
    import numpy as np
    return np.ascontiguousarray(np.asarray(a, dtype=np.int32))


class PageTable:
    """The residency policy alone (host object, no GPU)."""

    def __init__(self, rank, n_pages: int, handle=None):
        self._rank = _host_i32(rank)
        self.N, self.n_pages = int(self._rank.size), int(n_pages)
        self._own = handle is None
        if handle is None:
            h = _VP()
            _check("lora_page_table_create", lib().lora_page_table_create(
                self._rank.ctypes.data, self.N, self.n_pages, ctypes.byref(h)))
            handle = h.value
        self.h = handle

    def admit(self, ids):
        """{"copies": [(adapter, row, page, count)], "evicted": [...]} or
        {"error": "capacity"}."""
        ids = _host_i32(ids).reshape(-1)
        cp = (PageCopy * max(self.n_pages, 1))()
        ev = (_I32 * max(self.N, 1))()
        nc, ne = _I64(), _I64()
        st = lib().lora_page_table_admit(self.h, ids.ctypes.data if ids.size else None, ids.size,
                                         cp, self.n_pages, ctypes.byref(nc), ev, self.N,
                                         ctypes.byref(ne))
        if st == LORA_ERR_CAPACITY:
            return {"error": "capacity"}
        _check("lora_page_table_admit", st)
        return {"copies": [(c.adapter, c.row, c.page, c.count) for c in cp[:nc.value]],
                "evicted": [int(v) for v in ev[:ne.value]]}

    def tables(self):
        import numpy as np
        rk = np.zeros(self.N, np.int32)
        ps = np.zeros(self.N + 1, np.int32)
        pid = np.zeros(max(self.n_pages, 1), np.int32)
        n = _I64()
        _check("lora_page_table_tables", lib().lora_page_table_tables(
            self.h, rk.ctypes.data_as(ctypes.POINTER(_I32)), ps.ctypes.data_as(ctypes.POINTER(_I32)),
            pid.ctypes.data_as(ctypes.POINTER(_I32)), ctypes.byref(n)))
        return rk, ps, pid[:n.value].copy()

    def close(self):
        if self._own and self.h:
            lib().lora_page_table_destroy(self.h)
        self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class Residency:
    """The GPU pool of one projection, filled from a pinned host store on a
    copy stream (lora_residency_*).  `store_a`/`store_b` are pinned CPU torch
    tensors [rows][d]; `a_pages`/`b_pages` device tensors [n_pages][d]."""

    def __init__(self, dtype, d_in, d_out, rank, store_row, store_a, store_b, a_pages, b_pages,
                 scale):
        import numpy as np
        import torch
        self._rank = _host_i32(rank)
        self._row = np.ascontiguousarray(np.asarray(store_row, dtype=np.int64))
        self.N, self.n_pages = int(self._rank.size), int(a_pages.shape[0])
        nt = int(lib().lora_residency_table_ints(self.N, self.n_pages))
        self.tables = torch.zeros(nt, dtype=torch.int32, device=a_pages.device)
        self.staging = torch.zeros(nt, dtype=torch.int32).pin_memory()
        self._keep = (store_a, store_b, a_pages, b_pages, scale)
        self.cfg = ResidencyConfig(dtype, d_in, d_out, self.N, self.n_pages, self._rank.ctypes.data,
                                   self._row.ctypes.data, _ptr(store_a), _ptr(store_b),
                                   _ptr(a_pages), _ptr(b_pages), _ptr(scale), _ptr(self.tables),
                                   _ptr(self.staging))
        h = _VP()
        _check("lora_residency_create", lib().lora_residency_create(ctypes.byref(self.cfg),
                                                                    ctypes.byref(h)))
        self.h = h.value
        self.dtype, self.d_in, self.d_out = dtype, d_in, d_out

    def prepare(self, ids, copy_stream, compute_stream=None):
        """Returns a Pool (descriptor of the batch's tables) for the batch."""
        ids = _host_i32(ids).reshape(-1)
        desc = PoolDesc()
        st = lib().lora_residency_prepare(self.h, ids.ctypes.data if ids.size else None, ids.size,
                                          _stream(copy_stream), _stream(compute_stream),
                                          ctypes.byref(desc))
        _check("lora_residency_prepare", st)
        p = Pool.__new__(Pool)
        p.tensors = self._keep + (self.tables,)
        p.dtype, p.d_in, p.d_out, p.n_adapters = self.dtype, self.d_in, self.d_out, self.N
        p.desc = desc
        return p

    def finish(self, compute_stream=None):
        _check("lora_residency_finish", lib().lora_residency_finish(self.h, _stream(compute_stream)))

    def stats(self):
        out = (_I64 * 4)()
        _check("lora_residency_stats", lib().lora_residency_stats(self.h, out))
        return {"batches": out[0], "rows_copied": out[1], "evictions": out[2], "bytes": out[3]}

    def page_table(self):
        return PageTable(self._rank, self.n_pages, handle=lib().lora_residency_page_table(self.h))

    def close(self):
        if self.h:
            lib().lora_residency_destroy(self.h)
        self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


# ---------------------------------------------------------------- tall-skinny QR

def lora_tsqr_workspace_bytes(M: int, m: int, n: int) -> int:
    return int(lib().lora_tsqr_workspace_bytes(M, m, n))


def lora_tsqr(src, dtype: int, cols, M: int, m: int, n: int, Qt, R, ws, stream=None):
    _check("lora_tsqr", lib().lora_tsqr(_ptr(src), dtype, _ptr(cols), M, m, n, _ptr(Qt), _ptr(R),
                                        _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)))


def lora_compress_workspace_bytes(M: int, d_in: int, d_out: int, n: int) -> int:
    return int(lib().lora_compress_workspace_bytes(M, d_in, d_out, n))


def lora_compress(pool: Pool, adapters, M: int, n: int, policy: int, ratio: float, energy: float,
                  floor_rank: int, out_a, out_b, out_rank, out_sigma, ws, stream=None):
    _check("lora_compress", lib().lora_compress(
        pool.ref, _ptr(adapters), M, n, policy, float(ratio), float(energy), floor_rank,
        _ptr(out_a), _ptr(out_b), _ptr(out_rank), _ptr(out_sigma), _ptr(ws),
        ws.numel() * ws.element_size(), _stream(stream)))
