"""Seeded property sweep over the layer's input space, with canary guards
around every buffer the library writes.

A second, smaller sweep draws prefill-size batches (T in [512, 4096]) so
that the MFMA paths run: the 32-pair shrink tiles with the segments' tails
on the units schedule, the tile GEMMs and the MFMA gradient form.

Each case draws a batch at random: T in [0, 300], K in {1, 2}, d_in and d_out
multiples of 64 up to 1024, 1..40 adapters of ranks 0..130 (odd ones
included), empty slots (id -1), zero gates, an optional keep mask, fp32 or
bf16.  Plan, apply and forward run through the C ABI; the plan must equal the
oracle's bit for bit, Y must meet the float bar, and the gradients are checked
on every third case (120 cases).  Every output, the plan and the workspace sit inside a
larger allocation whose head and tail are filled with a byte pattern that must
survive the call: a write past either end of a buffer fails the case even
when it lands in memory the process owns.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from lora_adapter_amd import binding as B
from lora_adapter_amd import device as D
from lora_adapter_amd import workloads as wl
from oracle import lora_oracle as O

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-5, "bf16": 1e-2}
GUARD = 4096            # bytes of canary before and after each buffer
PATTERN = 0xA5


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.lib()   # fails loudly if the HIP library is missing


class Guarded:
    """A tensor of `shape` and `dtype` inside a byte buffer with canaries."""

    def __init__(self, shape, dtype, fill=None):
        n = int(np.prod(shape)) * torch.tensor([], dtype=dtype).element_size()
        self.n = n
        self.raw = torch.full((GUARD + n + GUARD,), PATTERN, dtype=torch.uint8, device="cuda")
        self.t = self.raw[GUARD:GUARD + n].view(dtype).view(shape)
        if fill is not None:
            self.t.fill_(fill)

    def intact(self) -> bool:
        head = self.raw[:GUARD]
        tail = self.raw[GUARD + self.n:]
        return bool((head == PATTERN).all()) and bool((tail == PATTERN).all())


def rel_err(gpu, ref):
    return float(np.max(np.abs(gpu - ref)) / max(np.max(np.abs(ref)), 1e-300))


def draw_case(seed: int) -> wl.Workload:
    rng = np.random.default_rng(1000 + seed)
    dtype = "bf16" if rng.random() < 0.6 else "f32"
    T = int(rng.choice([0, 1, 2, 63, 64, 65, 127, 200, 255, 256, 257, 300])) if seed % 3 == 0 \
        else int(rng.integers(0, 301))
    K = int(rng.integers(1, 3))
    d_in = 64 * int(rng.integers(1, 17))
    d_out = 64 * int(rng.integers(1, 17))
    N = int(rng.integers(1, 41))
    rank = rng.integers(0, 131, size=N).astype(np.int32)
    odd = rng.random(N) < 0.25          # odd ranks at the 16-row block and bucket edges
    rank[odd] = rng.choice(np.array([1, 3, 5, 17, 33, 65, 129], np.int32), size=int(odd.sum()))
    ids = rng.integers(-1, N, size=(T, K)).astype(np.int32)
    gates = rng.standard_normal((T, K)).astype(np.float32)
    gates[rng.random((T, K)) < 0.1] = 0.0
    keep_p = 0.9 if rng.random() < 0.5 else None
    return wl.build(f"sweep-{seed}", 1000 + seed, dtype, T, K, d_in, d_out, rank, ids, gates,
                    x_var=1.0, w_var=1.0 / d_in, a_var=1.0 / d_in, b_var=0.02,
                    scale=rng.uniform(0.25, 4.0, N).astype(np.float32), keep_p=keep_p,
                    with_dY=seed % 3 == 1)


class GuardedLayer(D.DeviceLayer):
    """A DeviceLayer whose Y, plan and workspace are canary-guarded."""

    def __init__(self, w):
        super().__init__(w)
        self.gY = Guarded(tuple(self.Y.shape), self.Y.dtype)
        self.gplan = Guarded(tuple(self.plan.shape), self.plan.dtype)
        self.gws = Guarded(tuple(self.ws.shape), self.ws.dtype)
        self.Y, self.plan, self.ws = self.gY.t, self.gplan.t, self.gws.t

    def intact(self):
        return {"Y": self.gY.intact(), "plan": self.gplan.intact(), "ws": self.gws.intact()}


def check_plan_apply(w, L):
    got = L.read_plan()
    ref = O.plan_workload(w)
    np.testing.assert_array_equal(got["header"][:8], ref["header"][:8])
    for k in ("pair_tk", "seg_adapter", "seg_off", "seg_row_off", "bucket_seg_off", "u_off",
              "slot_pos", "pair_adapter"):
        np.testing.assert_array_equal(got[k], ref[k], err_msg=k)
    if w.T > 0:
        err = rel_err(D.as_f64(L.Y_host()), O.apply_workload(w))
        assert err <= TOL[w.dtype], (w.name, err)


CASES = list(range(120))


@pytest.mark.parametrize("seed", CASES)
def test_sweep_plan_apply_forward(seed):
    w = draw_case(seed)
    print(f"case {w.name}: {w.dtype} T={w.T} K={w.K} d={w.d_in}x{w.d_out} N={w.n_adapters} "
          f"max_rank={w.max_rank} mask={w.keep_mask is not None}", flush=True)
    L = GuardedLayer(w)
    L.run_plan()
    L.run_apply()
    torch.cuda.synchronize()
    assert all(L.intact().values()), L.intact()
    check_plan_apply(w, L)

    # the one-call forward on fresh (guarded) buffers
    F = GuardedLayer(w)
    B.lora_forward(F.ids, F.gates, F.T, F.K, F.X, F.W_t, F.Y, F.keep_mask, F.keep_scale, F.pool,
                   F.plan, F.ws)
    torch.cuda.synchronize()
    assert all(F.intact().values()), F.intact()
    check_plan_apply(w, F)

    if w.dY is not None and w.T > 0:
        dA = Guarded((w.n_pages, w.d_in), torch.float32, fill=float("nan"))
        dB = Guarded((w.n_pages, w.d_out), torch.float32, fill=float("nan"))
        n = B.lora_grad_workspace_bytes(w.T, w.K, w.n_adapters, w.d_in, w.d_out, L.max_rank, L.dtype)
        gws = Guarded((n,), torch.uint8)
        L.run_grad(dA.t, dB.t, gws.t)
        torch.cuda.synchronize()
        assert dA.intact() and dB.intact() and gws.intact()
        g = O.grad_workload(w)
        rA, rB = O.grad_pages(g, w.rank, w.page_start, w.page_ids, w.n_pages, w.d_in, w.d_out)
        gA = dA.t.cpu().numpy().astype(np.float64)
        gB = dB.t.cpu().numpy().astype(np.float64)
        used = ~np.isnan(rA[:, 0])
        assert np.all(np.isnan(gA[~used])) and np.all(np.isnan(gB[~used]))
        if used.any() and np.max(np.abs(rA[used])) > 0:
            assert rel_err(gA[used], rA[used]) <= TOL[w.dtype]
            assert rel_err(gB[used], rB[used]) <= TOL[w.dtype]


def draw_large(seed: int) -> wl.Workload:
    """A prefill-size bf16 batch: Zipf-weighted adapters so that some
    segments are long (MFMA shrink tiles, with tails of any length) and many
    are short; d_in a multiple of 128 and d_out of 256 (the MFMA shrink and
    gradient forms), K of 1 or 2, empty slots, an optional keep mask."""
    rng = np.random.default_rng(5000 + seed)
    T = int(rng.integers(512, 4097))
    K = int(rng.integers(1, 3))
    d_in = 128 * int(rng.integers(1, 9))
    d_out = 256 * int(rng.integers(1, 5))
    N = int(rng.integers(1, 40))
    rank = rng.integers(1, 65, size=N).astype(np.int32)
    ids = wl.zipf_ids(rng, T * K, N, s=1.2).reshape(T, K)
    ids[rng.random((T, K)) < 0.05] = -1
    gates = rng.standard_normal((T, K)).astype(np.float32)
    keep_p = 0.9 if seed % 2 == 0 else None
    return wl.build(f"sweep-large-{seed}", 5000 + seed, "bf16", T, K, d_in, d_out, rank, ids, gates,
                    x_var=1.0, w_var=1.0 / d_in, a_var=1.0 / d_in, b_var=0.02,
                    scale=rng.uniform(0.25, 4.0, N).astype(np.float32), keep_p=keep_p,
                    with_dY=True)


@pytest.mark.parametrize("seed", list(range(10)))
def test_sweep_large_batches(seed):
    w = draw_large(seed)
    print(f"case {w.name}: T={w.T} K={w.K} d={w.d_in}x{w.d_out} N={w.n_adapters} "
          f"mask={w.keep_mask is not None}", flush=True)
    L = GuardedLayer(w)
    L.run_plan()
    L.run_apply()
    torch.cuda.synchronize()
    assert all(L.intact().values()), L.intact()
    check_plan_apply(w, L)
    F = GuardedLayer(w)
    B.lora_forward(F.ids, F.gates, F.T, F.K, F.X, F.W_t, F.Y, F.keep_mask, F.keep_scale, F.pool,
                   F.plan, F.ws)
    torch.cuda.synchronize()
    assert all(F.intact().values()), F.intact()
    assert np.array_equal(D.to_host(F.Y), D.to_host(L.Y))      # same kernels, same bits
    dA = Guarded((w.n_pages, w.d_in), torch.float32, fill=float("nan"))
    dB = Guarded((w.n_pages, w.d_out), torch.float32, fill=float("nan"))
    n = B.lora_grad_workspace_bytes(w.T, w.K, w.n_adapters, w.d_in, w.d_out, L.max_rank, L.dtype)
    gws = Guarded((n,), torch.uint8)
    L.run_grad(dA.t, dB.t, gws.t)
    torch.cuda.synchronize()
    assert dA.intact() and dB.intact() and gws.intact()
    g = O.grad_workload(w)
    rA, rB = O.grad_pages(g, w.rank, w.page_start, w.page_ids, w.n_pages, w.d_in, w.d_out)
    gA = dA.t.cpu().numpy().astype(np.float64)
    gB = dB.t.cpu().numpy().astype(np.float64)
    used = ~np.isnan(rA[:, 0])
    assert np.all(np.isnan(gA[~used])) and np.all(np.isnan(gB[~used]))
    assert rel_err(gA[used], rA[used]) <= TOL["bf16"]
    assert rel_err(gB[used], rB[used]) <= TOL["bf16"]


@pytest.mark.parametrize("cfg", [1, 4, 5])
def test_guards_merge_and_input_gradient(cfg):
    """Canaries around W during a signed merge, and around dX and its
    workspace during the input gradient."""
    w = wl.small(cfg)
    L = GuardedLayer(w)
    L.run_plan()
    L.run_apply()
    gW = Guarded(tuple(L.W_t.shape), L.W_t.dtype)
    gW.t.copy_(L.W_t)
    ids = np.arange(min(3, w.n_adapters), dtype=np.int32)
    coeffs = np.linspace(1.0, -0.5, ids.size).astype(np.float32)
    L.run_merge(gW.t, ids, coeffs)
    torch.cuda.synchronize()
    assert gW.intact()
    ref = O.merge_workload(w, ids=ids, coeffs=coeffs)
    assert rel_err(D.as_f64(D.to_host(gW.t)), ref) <= TOL[w.dtype]
    if w.dY is None:
        return
    dA, dB, gws = L.grad_buffers()
    L.run_grad(dA, dB, gws)
    Wn = L.weight_transposed()
    dX = Guarded((w.T, w.d_in), L.Y.dtype)
    n = B.lora_grad_x_workspace_bytes(w.T, w.d_in, w.d_out, L.dtype)
    xws = Guarded((n,), torch.uint8)
    L.run_grad_x(Wn, gws, dX.t, xws.t)
    torch.cuda.synchronize()
    assert dX.intact() and xws.intact()
    err = rel_err(D.as_f64(D.to_host(dX.t)), O.grad_x_workload(w))
    assert err <= TOL[w.dtype], err
