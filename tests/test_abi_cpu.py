"""C ABI checks that need no GPU: the library loads, exports every function
include/lora.h declares, and host-visible argument errors come back before any
HIP call (only null pointers and bad sizes are used here, so no kernel runs)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lora.h")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(lora_[a-z_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def B():
    from lora_adapter_amd import binding
    if not os.path.exists(binding.LIB_PATH):
        from lora_adapter_amd import build
        build.build()
    return binding


def test_header_declares_the_binding_exports(B):
    assert _declared() == sorted(B.EXPORTS)


def test_library_exports_every_declared_symbol(B):
    L = B.lib()
    for name in _declared():
        assert hasattr(L, name), name


def test_abi_version_and_status_strings(B):
    assert B.lora_abi_version() == 1
    assert B.status_string(0) == "ok"
    assert "invalid" in B.status_string(1)
    assert B.status_string(99) == "unknown status"


def test_plan_sizes_and_layout(B):
    assert B.lora_plan_bytes(64, 1, 64) > 0
    assert B.lora_plan_bytes(-1, 1, 4) == 0
    assert B.lora_plan_bytes(4, 0, 4) == 0
    assert B.lora_plan_bytes(4, 9, 4) == 0
    assert B.lora_plan_bytes(4, 1, 0) == 0
    off = B.lora_plan_layout(10, 2, 5)
    assert off == sorted(off) and all(o % 64 == 0 for o in off)
    assert B.lora_plan_bytes(10, 2, 5) >= off[-1] + 4 * 10 * 2
    with pytest.raises(B.LoraError):
        B.lora_plan_layout(1 << 20, 2, 5)          # more than 2^20 slots


def test_workspace_sizes(B):
    n = B.lora_apply_workspace_bytes(64, 1, 4096, 4096, 16, B.LORA_BF16)
    assert n >= 64 * 16 * 4
    assert B.lora_apply_u_offset(64, 1, 4096, 4096, B.LORA_BF16) < n
    assert B.lora_apply_workspace_bytes(64, 1, 4000, 4096, 16, B.LORA_BF16) == 0   # d_in % 64
    assert B.lora_apply_workspace_bytes(64, 1, 4096, 4096, 2000, B.LORA_BF16) == 0  # rank cap
    assert B.lora_apply_workspace_bytes(64, 1, 4096, 4096, 16, 7) == 0
    assert B.lora_grad_workspace_bytes(8192, 1, 4, 4096, 11008, 16, B.LORA_BF16) > 0
    assert B.lora_grad_workspace_bytes(8192, 1, 4, 4096, 11008, 0, B.LORA_BF16) == 0


def _desc(B, **kw):
    d = dict(dtype=B.LORA_BF16, d_in=128, d_out=128, n_adapters=2, n_pages=4, n_page_ids=4,
             a_pages=8, b_pages=8, rank=8, page_start=8, page_ids=8, scale=8)
    d.update(kw)
    return B.PoolDesc(*[d[f] for f, _ in B.PoolDesc._fields_])


def test_argument_errors_return_before_any_hip_call(B):
    L = B.lib()
    pd = _desc(B)
    ref = ctypes.byref(pd)
    INV, UNS, CAP = B.LORA_ERR_INVALID_ARG, B.LORA_ERR_UNSUPPORTED, B.LORA_ERR_CAPACITY
    # plan: bad T, K, null pool, null plan, null ids, too-small plan buffer
    assert L.lora_plan(8, 8, -1, 1, ref, 8, 1 << 20, None) == INV
    assert L.lora_plan(8, 8, 4, 0, ref, 8, 1 << 20, None) == INV
    assert L.lora_plan(8, 8, 4, 9, ref, 8, 1 << 20, None) == INV
    assert L.lora_plan(8, 8, 4, 1, None, 8, 1 << 20, None) == INV
    assert L.lora_plan(8, 8, 4, 1, ref, None, 1 << 20, None) == INV
    assert L.lora_plan(None, 8, 4, 1, ref, 8, 1 << 20, None) == INV
    assert L.lora_plan(8, 8, 4, 1, ref, 8, 16, None) == CAP
    bad_dtype = _desc(B, dtype=5)
    assert L.lora_plan(8, 8, 4, 1, ctypes.byref(bad_dtype), 8, 1 << 20, None) == INV
    no_rank = _desc(B, rank=None)
    assert L.lora_plan(8, 8, 4, 1, ctypes.byref(no_rank), 8, 1 << 20, None) == INV
    # apply family: dims not multiples of 64, null tensors, aliasing, tiny workspace
    odd = _desc(B, d_in=100)
    assert L.lora_apply(8, 8, 16, 4, 1, 8, None, 1.0, ctypes.byref(odd), 8, 8, 1 << 20, None) == UNS
    assert L.lora_apply(None, 8, 16, 4, 1, 8, None, 1.0, ref, 8, 8, 1 << 20, None) == INV
    assert L.lora_base_expand(8, 16, 8, 4, 1, ref, 8, 24, 1 << 20, None) == INV   # Y aliases X
    assert L.lora_base_expand(8, 16, 24, 4, 1, ref, 8, None, 1 << 20, None) == INV
    assert L.lora_base_gemm(8, 16, 24, 4, 1, ref, None, 24, 1 << 20, None) == INV
    assert L.lora_expand_epilogue(8, 16, 24, 4, 1, ref, 8, 24, 0, None) == CAP
    assert L.lora_shrink(8, None, 1.0, 4, 1, 8, ref, 8, 8, 0, None) == CAP
    # empty batch is valid and launches nothing
    assert L.lora_apply(None, None, None, 0, 1, None, None, 1.0, ref, 8, None, 0, None) == 0
    # merge: negative count, null W; m == 0 is a no-op
    assert L.lora_merge_delta(8, ref, 8, 8, -1, None) == INV
    assert L.lora_merge_delta(None, ref, 8, 8, 1, None) == INV
    assert L.lora_merge_delta(8, ref, None, None, 0, None) == 0
    # plan header reader: null plan or output
    out = (ctypes.c_int32 * 16)()
    assert L.lora_plan_header(None, out, None) == INV
    assert L.lora_plan_header(8, None, None) == INV
    # forward without allocation: bad max_rank, a batch beyond the library's
    # array (both rejected before any HIP call)
    assert L.lora_forward_noalloc(8, 8, 4, 1, 8, 8, 24, None, 1.0, ref, 2000, None) == INV
    assert L.lora_forward_noalloc(8, 8, 8192, 8, 8, 8, 24, None, 1.0, ref, 1024, None) == CAP
    assert L.lora_forward_noalloc(8, 8, 4, 1, 8, 8, 24, None, 1.0, None, 16, None) == INV
    assert B.lora_forward_noalloc_bytes(64, 1, 64, 4096, 4096, 16, B.LORA_BF16) <= 64 << 20
    # grad: bad max_rank, too-small workspace
    assert L.lora_grad(8, None, 1.0, 8, 4, 1, 8, ref, 8, 8, 1 << 20, 8, 8, 0, 8, 1 << 30, None) == INV
    assert L.lora_grad(8, None, 1.0, 8, 4, 1, 8, ref, 8, 8, 1 << 20, 8, 8, 16, 8, 16, None) == CAP


def test_binding_fails_loudly_without_the_library(monkeypatch, tmp_path):
    from lora_adapter_amd import binding
    monkeypatch.setattr(binding, "_lib", None)
    monkeypatch.setattr(binding, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="missing"):
        binding.lib()
