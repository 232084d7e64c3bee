"""lora_forward_noalloc (plan and workspace in the library's own device array)
against lora_forward with caller-owned buffers, called through the C ABI: two
calls in a row on one GPU, the second with a smaller batch, each equal to
lora_forward bit for bit and within the bf16 bar of the CPU oracle."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from lora_adapter_amd import binding as B
from lora_adapter_amd import device as D
from lora_adapter_amd import workloads as wl
from oracle import lora_oracle as O

pytestmark = pytest.mark.gpu


def _rel(a, b):
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


def _forward_both(w):
    L = D.DeviceLayer(w)
    B.lora_forward(L.ids, L.gates, L.T, L.K, L.X, L.W_t, L.Y, L.keep_mask, L.keep_scale, L.pool,
                   L.plan, L.ws)
    torch.cuda.synchronize()
    ref = L.Y_host().copy()
    Y2 = torch.full_like(L.Y, float("nan"))
    B.lora_forward_noalloc(L.ids, L.gates, L.T, L.K, L.X, L.W_t, Y2, L.keep_mask, L.keep_scale,
                           L.pool, L.max_rank)
    torch.cuda.synchronize()
    return ref, D.to_host(Y2)


def test_noalloc_forward_twice_second_smaller():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.lib()
    # a split-K prefill-sized batch (top-2 routing), then a smaller decode batch
    big = wl.config(5, T=300, d_in=1024, d_out=1536, n_adapters=64, seed=501)
    small = wl.config(5, T=37, d_in=1024, d_out=1536, n_adapters=64, seed=502)
    for w in (big, small):
        need = B.lora_forward_noalloc_bytes(w.T, w.K, w.n_adapters, w.d_in, w.d_out, w.max_rank,
                                            B.LORA_BF16)
        print(f"noalloc case T={w.T} K={w.K} d={w.d_in}x{w.d_out} bytes={need}", flush=True)
        assert 0 < need <= 64 << 20
        ref, got = _forward_both(w)
        assert np.array_equal(got, ref), "noalloc forward differs from lora_forward"
        e = _rel(D.as_f64(got), O.apply_workload(w))
        assert e <= 1e-2, e


def test_noalloc_rejects_batches_beyond_the_array():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    w = wl.small(2)
    L = D.DeviceLayer(w)
    with pytest.raises(B.LoraError) as ei:
        # 8192 slots of rank up to 1024 need 32 MiB of U plus partials: too much
        B.lora_forward_noalloc(L.ids, L.gates, 8192, 8, L.X, L.W_t, L.Y, None, 1.0, L.pool, 1024)
    assert ei.value.status == B.LORA_ERR_CAPACITY
