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
LIB_PATH = os.path.join(PKG, "liblora.so")

LORA_OK, LORA_ERR_INVALID_ARG, LORA_ERR_UNSUPPORTED, LORA_ERR_CAPACITY, LORA_ERR_DEVICE = range(5)
LORA_F32, LORA_BF16 = 0, 1
LORA_MAX_RANK = 1024
LORA_MAX_K = 8
DEVERR_BAD_ID, DEVERR_BAD_RANK, DEVERR_BAD_POOL, DEVERR_CAPACITY = 1, 2, 4, 8
PH_PAIRS, PH_SEGS, PH_ERR, PH_RPAIRS, PH_RUSED, PH_T, PH_K, PH_N = range(8)

EXPORTS = (
    "lora_abi_version", "lora_status_string", "lora_plan_bytes", "lora_plan_layout", "lora_plan",
    "lora_apply_workspace_bytes", "lora_apply_u_offset", "lora_shrink", "lora_base_expand",
    "lora_base_gemm", "lora_expand_epilogue", "lora_shrink_gemm", "lora_apply",
    "lora_forward_gemm", "lora_forward_finish", "lora_forward", "lora_merge_delta", "lora_grad_workspace_bytes", "lora_grad",
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


_lib = None
_I32, _I64, _SZ, _VP, _F32 = ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_float
_PD = ctypes.POINTER(PoolDesc)

_PROTOS = {
    "lora_abi_version": (_I32, []),
    "lora_status_string": (ctypes.c_char_p, [_I32]),
    "lora_plan_bytes": (_SZ, [_I32, _I32, _I32]),
    "lora_plan_layout": (_I32, [_I32, _I32, _I32, ctypes.POINTER(_I64)]),
    "lora_plan": (_I32, [_VP, _VP, _I32, _I32, _PD, _VP, _SZ, _VP]),
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
    "lora_merge_delta": (_I32, [_VP, _PD, _VP, _VP, _I32, _VP]),
    "lora_grad_workspace_bytes": (_SZ, [_I32, _I32, _I32, _I32, _I32, _I32, _I32]),
    "lora_grad": (_I32, [_VP, _VP, _F32, _VP, _I32, _I32, _VP, _PD, _VP, _VP, _SZ, _VP, _VP,
                         _I32, _VP, _SZ, _VP]),
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
        return int(stream)
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
