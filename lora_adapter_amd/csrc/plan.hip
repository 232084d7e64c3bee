// Plan kernel: groups a batch's active (token, slot) pairs by adapter.
//
// Segmented gather needs the rows of one adapter together (AdaFuse notes,
// section 关键设计 item 3); rank-specialised execution needs segments grouped
// by rank (LoRAForge page, section LoRAForge的核心设计 and its note on
// rank-specialised kernels).  The output is a stable counting sort by the key
// (rank bucket, adapter, token, slot) plus the offsets every later kernel
// uses.  All integer, so it is bit-exact and deterministic.
//
// One workgroup of 1024 threads does the whole plan (a batch has at most
// 2^20 slots; decode batches have tens to hundreds):
//   1. count active slots per adapter (wave-aggregated atomics);
//   2. check the page table of every used adapter, dropping bad ones;
//   3. nine bucket-ordered block scans over the adapters give each adapter
//      its first pair position, segment index, U offset and row offset;
//   4. place pairs in slot order, wave after wave, so that equal adapters keep
//      their (token, slot) order: each wave resolves its lanes' order with
//      ballots and takes positions from a per-adapter cursor.
#include "lora_internal.h"

namespace lora {
namespace {

struct PlanArgs {
  const int32_t *ids;
  const float *gates;
  int T, K, N;
  const int32_t *rank, *page_start, *page_ids;
  int64_t n_pages, n_page_ids;
  int32_t *plan;
};

__device__ __forceinline__ int rank_bucket(int r) {
  if (r <= 1) return 0;
  if (r > 128) return 8;
  return 32 - __clz(r - 1);
}

// Adapter of slot i if the slot is a candidate (valid id, rank in range and
// > 0, gate non-zero), else -1.  Sets error bits for invalid ids and ranks.
__device__ __forceinline__ int classify(const PlanArgs &a, int64_t i, int &err) {
  const int id = a.ids[i];
  if (id == -1) return -1;
  if (id < -1 || id >= a.N) {
    err |= LORA_DEVERR_BAD_ID;
    return -1;
  }
  const int r = a.rank[id];
  if (r < 0 || r > LORA_MAX_RANK) {
    err |= LORA_DEVERR_BAD_RANK;
    return -1;
  }
  return (r > 0 && a.gates[i] != 0.0f) ? id : -1;
}

// Counters may live in global memory (large pools): read them with
// agent-scope loads so a line cached in L1 before an atomic is never reused.
__device__ __forceinline__ int ld_ctr(const int *p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_ctr(int *p, int v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

struct Scan4 {
  int v[4];
};

// Exclusive block scan of four ints over 1024 threads; returns the totals.
__device__ Scan4 block_exclusive_scan4(Scan4 x, Scan4 &total, int *lds_tot /* [16*4] */) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  Scan4 inc = x;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int y = __shfl_up(inc.v[q], d, 64);
      if (lane >= d) inc.v[q] += y;
    }
  }
  if (lane == 63) {
#pragma unroll
    for (int q = 0; q < 4; ++q) lds_tot[wave * 4 + q] = inc.v[q];
  }
  __syncthreads();
  Scan4 before{{0, 0, 0, 0}};
  Scan4 tot{{0, 0, 0, 0}};
  for (int w = 0; w < kPlanThreads / 64; ++w) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int t = lds_tot[w * 4 + q];
      if (w < wave) before.v[q] += t;
      tot.v[q] += t;
    }
  }
  __syncthreads();  // lds_tot is reused by the next call
  Scan4 ex;
#pragma unroll
  for (int q = 0; q < 4; ++q) ex.v[q] = before.v[q] + inc.v[q] - x.v[q];
  total = tot;
  return ex;
}

template <bool kLdsCounters>
__global__ __launch_bounds__(kPlanThreads) void plan_kernel(PlanArgs a) {
  extern __shared__ int lds_dyn[];          // [2*N] when kLdsCounters
  __shared__ int lds_tot[(kPlanThreads / 64) * 4];
  __shared__ int lds_err;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int64_t TK = int64_t(a.T) * a.K;
  const PlanLayout L = plan_layout(TK, a.N);
  int32_t *P = a.plan;
  int *cnt = kLdsCounters ? lds_dyn : P + L.cnt;
  int *cur = kLdsCounters ? lds_dyn + a.N : P + L.cur;
  int32_t *start = P + L.start;
  int32_t *ustart = P + L.ustart;

  // 0. clear counters
  if (tid == 0) lds_err = 0;
  for (int i = tid; i < a.N; i += kPlanThreads) st_ctr(&cnt[i], 0);
  __syncthreads();

  // 1. count candidate slots per adapter
  int err = 0;
  for (int64_t base = 0; base < TK; base += kPlanThreads) {
    const int64_t i = base + tid;
    const int ad = (i < TK) ? classify(a, i, err) : -1;
    uint64_t pending = __ballot(ad >= 0);
    while (pending) {
      const int leader = __ffsll((unsigned long long)pending) - 1;
      const int la = __shfl(ad, leader, 64);
      const uint64_t m = __ballot(ad == la);
      if (lane == leader) atomicAdd(&cnt[la], __popcll(m));
      pending &= ~m;
    }
  }
  if (err) atomicOr(&lds_err, err);
  __syncthreads();

  // 2. page-table check of every used adapter; a bad adapter gets cnt = -1
  for (int ad = tid; ad < a.N; ad += kPlanThreads) {
    if (ld_ctr(&cnt[ad]) <= 0) continue;
    const int64_t r = a.rank[ad];
    const int64_t s0 = a.page_start[ad], s1 = a.page_start[ad + 1];
    bool ok = s0 >= 0 && s1 - s0 == r && s1 <= a.n_page_ids;
    for (int64_t j = 0; ok && j < r; ++j) {
      const int64_t pg = a.page_ids[s0 + j];
      ok = pg >= 0 && pg < a.n_pages;
    }
    if (!ok) {
      st_ctr(&cnt[ad], -1);
      atomicOr(&lds_err, LORA_DEVERR_BAD_POOL);
    }
  }
  __syncthreads();

  // 3. bucket-ordered scans: pairs, segments, U floats, rank rows
  int pair_base = 0, seg_base = 0, u_base = 0, row_base = 0;
  for (int b = 0; b < LORA_N_BUCKETS; ++b) {
    if (tid == 0) P[L.bucket_seg_off + b] = seg_base;
    for (int c0 = 0; c0 < a.N; c0 += kPlanThreads) {
      const int ad = c0 + tid;
      int c = 0, r = 0;
      if (ad < a.N) {
        c = ld_ctr(&cnt[ad]);
        r = a.rank[ad];
        if (c <= 0 || rank_bucket(r) != b) c = 0;
      }
      Scan4 x{{c, c > 0 ? 1 : 0, c * r, c > 0 ? r : 0}};
      Scan4 tot;
      const Scan4 ex = block_exclusive_scan4(x, tot, lds_tot);
      if (c > 0) {
        const int st = pair_base + ex.v[0];
        const int sg = seg_base + ex.v[1];
        start[ad] = st;
        st_ctr(&cur[ad], st);
        ustart[ad] = u_base + ex.v[2];
        P[L.seg_adapter + sg] = ad;
        P[L.seg_off + sg] = st;
        P[L.seg_row_off + sg] = row_base + ex.v[3];
      }
      pair_base += tot.v[0];
      seg_base += tot.v[1];
      u_base += tot.v[2];
      row_base += tot.v[3];
    }
  }
  if (tid == 0) {
    P[L.bucket_seg_off + LORA_N_BUCKETS] = seg_base;
    P[L.seg_off + seg_base] = pair_base;
    P[L.seg_row_off + seg_base] = row_base;
    P[L.u_off + pair_base] = u_base;
  }
  __syncthreads();

  // 4. ordered placement, one wave at a time within each 1024-slot chunk
  const uint64_t lt_mask = (uint64_t(1) << lane) - 1;
  for (int64_t base = 0; base < TK; base += kPlanThreads) {
    const int64_t i = base + tid;
    int dummy = 0;
    int ad = (i < TK) ? classify(a, i, dummy) : -1;
    if (ad >= 0 && ld_ctr(&cnt[ad]) <= 0) ad = -1;
    const uint64_t act = __ballot(ad >= 0);
    int pos = -1;
    for (int w = 0; w < kPlanThreads / 64; ++w) {
      __syncthreads();
      if (wave == w && act != 0) {
        uint64_t pending = act;
        while (pending) {
          const int leader = __ffsll((unsigned long long)pending) - 1;
          const int la = __shfl(ad, leader, 64);
          const uint64_t m = __ballot(ad == la);
          int b0 = 0;
          if (lane == leader) b0 = atomicAdd(&cur[la], __popcll(m));
          b0 = __shfl(b0, leader, 64);
          if (ad == la) pos = b0 + __popcll(m & lt_mask);
          pending &= ~m;
        }
      }
    }
    if (i < TK) {
      P[L.slot_pos + i] = pos;
      if (pos >= 0) {
        P[L.pair_tk + pos] = int32_t(i);
        P[L.pair_adapter + pos] = ad;
        P[L.u_off + pos] = ustart[ad] + (pos - start[ad]) * a.rank[ad];
      }
    }
  }
  __syncthreads();
  if (tid == 0) {
    int32_t *h = P + L.hdr;
    h[LORA_PH_PAIRS] = pair_base;
    h[LORA_PH_SEGS] = seg_base;
    h[LORA_PH_ERR] = lds_err;
    h[LORA_PH_RPAIRS] = u_base;
    h[LORA_PH_RUSED] = row_base;
    h[LORA_PH_T] = a.T;
    h[LORA_PH_K] = a.K;
    h[LORA_PH_N] = a.N;
    for (int q = 8; q < LORA_PLAN_HEADER_INTS; ++q) h[q] = 0;
    for (int q = LORA_N_BUCKETS + 1; q < 16; ++q) P[L.bucket_seg_off + q] = 0;
  }
}

}  // namespace

hipError_t launch_plan(const int32_t *ids, const float *gates, int T, int K, const PoolView &pool,
                       int32_t *plan, hipStream_t s) {
  PlanArgs a{ids, gates, T, K, pool.n_adapters, pool.rank, pool.page_start, pool.page_ids,
             pool.n_pages, pool.n_page_ids, plan};
  if (pool.n_adapters <= kPlanLdsMaxAdapters) {
    const size_t lds = size_t(2) * pool.n_adapters * sizeof(int);
    hipLaunchKernelGGL(plan_kernel<true>, dim3(1), dim3(kPlanThreads), lds, s, a);
  } else {
    hipLaunchKernelGGL(plan_kernel<false>, dim3(1), dim3(kPlanThreads), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace lora
