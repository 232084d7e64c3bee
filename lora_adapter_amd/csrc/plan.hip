// Plan kernel: groups a batch's active (token, slot) pairs by adapter.
//
// Segmented gather needs the rows of one adapter together (AdaFuse notes,
// section 关键设计 item 3); rank-specialised execution needs segments grouped
// by rank (LoRAForge page, section LoRAForge的核心设计 and its note on
// rank-specialised kernels).  The output is a stable counting sort by the key
// (rank bucket, adapter, token, slot) plus the offsets and packed descriptors
// the later kernels use.  All integer: bit-exact and deterministic.
//
// One workgroup of 1024 threads builds the whole plan.  At decode sizes the
// cost is latency, so the kernel is organised around few global round trips:
//   0. every thread loads the rank and page_start of its own block of
//      adapters (contiguous ids) into LDS;
//   1. each slot is classified (ids and gates: one round trip; adapter data
//      from LDS) and counted per adapter;
//   2. page_start consistency of every used adapter;
//   3. one block scan per non-empty rank bucket gives each used adapter its
//      first pair position, segment, U offset and rank-row offset;
//   4. page ids of every used rank row are range-checked in parallel over rows
//      (a bad adapter is dropped and step 3 redone once);
//   5. pairs are placed in slot order: lanes holding the same adapter find
//      each other with one ballot per id bit, the first of them takes
//      positions from the adapter's cursor, and the waves of a 1024-slot
//      chunk take their turns in order, which keeps the sort stable.
// Per-adapter arrays live in LDS when they fit (96 KiB), else in the plan
// buffer's scratch (accessed with agent-scope atomics where counters change).
#include "lora_internal.h"

namespace lora {
namespace {

constexpr int kInfBadRank = 1 << 11;   // rank < 0 or > LORA_MAX_RANK
constexpr int kInfBadStart = 1 << 12;  // page_start inconsistent with rank
constexpr int kInfRankMask = 0x7ff;

struct PlanArgs {
  const int32_t *ids;
  const float *gates;
  int T, K, N;
  const int32_t *rank, *page_start, *page_ids;
  int64_t n_pages, n_page_ids;
  int32_t *plan;
  int slot_cache;    // 1: per-slot adapters cached in LDS
};

__device__ __forceinline__ int rank_bucket(int r) {
  if (r <= 1) return 0;
  if (r > 128) return 8;
  return 32 - __clz(r - 1);
}

__device__ __forceinline__ int ld_ctr(const int *p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_ctr(int *p, int v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

struct Scan4 {
  int v[4];
};

// Exclusive block scan of four ints over the 1024 threads; also the totals.
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

// Lanes of this wave whose adapter equals mine (a >= 0), one ballot per id bit.
__device__ __forceinline__ uint64_t match_lanes(int a, int nbits) {
  uint64_t m = __ballot(a >= 0);
#pragma unroll 1
  for (int b = 0; b < nbits; ++b) {
    const bool bit = (a >> b) & 1;
    const uint64_t bb = __ballot(bit);
    m &= bit ? bb : ~bb;
  }
  return a >= 0 ? m : 0;
}

template <bool kLds>
__global__ __launch_bounds__(kPlanThreads) void plan_kernel(PlanArgs a) {
  extern __shared__ int dyn[];
  __shared__ int lds_tot[(kPlanThreads / 64) * 4];
  __shared__ int s_err, s_bmask, s_bad;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int N = a.N;
  const int64_t TK = int64_t(a.T) * a.K;
  const int Smax = int(TK < N ? TK : N);
  const PlanLayout L = plan_layout(TK, N);
  int32_t *P = a.plan;
  // per-adapter arrays
  int *cnt = kLds ? dyn : P + L.cnt;
  int *cur = kLds ? dyn + N : P + L.cur;
  int *psa = kLds ? dyn + 2 * N : P + L.ps;
  int *inf = kLds ? dyn + 3 * N : P + L.inf;
  // segment arrays (outputs; LDS copies when they fit)
  int *seg_row = kLds ? dyn + 4 * N : P + L.seg_row_off;
  int *seg_ad = kLds ? dyn + 4 * N + Smax + 1 : P + L.seg_adapter;
  int *slot_ad = dyn + (kLds ? 4 * N + 2 * Smax + 1 : 0);
  int32_t *start = P + L.start;
  int32_t *ustart = P + L.ustart;

  const int m = (N + kPlanThreads - 1) / kPlanThreads;  // adapters per thread
  const int a0 = tid * m, a1 = min(N, a0 + m);

  // 0. per-adapter data
  if (tid == 0) { s_err = 0; s_bmask = 0; s_bad = 0; }
  for (int ad = a0; ad < a1; ++ad) {
    const int r = a.rank[ad];
    const int64_t s0 = a.page_start[ad], s1 = a.page_start[ad + 1];
    int v = (r < 0 || r > LORA_MAX_RANK) ? kInfBadRank : r;
    if (s0 < 0 || s1 - s0 != int64_t(r) || s1 > a.n_page_ids) v |= kInfBadStart;
    inf[ad] = v;
    psa[ad] = int(s0);
    st_ctr(&cnt[ad], 0);
  }
  __syncthreads();

  // 1. classify and count
  const int nbits = N > 1 ? 32 - __clz(N - 1) : 1;
  int err = 0;
  for (int64_t base = 0; base < TK; base += kPlanThreads) {
    const int64_t i = base + tid;
    int ad = -1;
    if (i < TK) {
      const int id = a.ids[i];
      const float g = a.gates[i];
      if (id < -1 || id >= N) {
        err |= LORA_DEVERR_BAD_ID;
      } else if (id >= 0) {
        const int v = inf[id];
        if (v & kInfBadRank) err |= LORA_DEVERR_BAD_RANK;
        else if ((v & kInfRankMask) > 0 && g != 0.0f) ad = id;
      }
      if (a.slot_cache) slot_ad[i] = ad;
    }
    const uint64_t mm = match_lanes(ad, nbits);
    if (ad >= 0 && (mm & ((uint64_t(1) << lane) - 1)) == 0) atomicAdd(&cnt[ad], __popcll(mm));
  }
  if (err) atomicOr(&s_err, err);
  __syncthreads();

  // 2. page_start consistency of used adapters; bucket occupancy
  {
    int bm = 0;
    for (int ad = a0; ad < a1; ++ad) {
      const int c = ld_ctr(&cnt[ad]);
      if (c <= 0) continue;
      const int v = inf[ad];
      if (v & kInfBadStart) {
        st_ctr(&cnt[ad], -1);
        atomicOr(&s_err, LORA_DEVERR_BAD_POOL);
      } else {
        bm |= 1 << rank_bucket(v & kInfRankMask);
      }
    }
    if (bm) atomicOr(&s_bmask, bm);
  }
  __syncthreads();

  // 3. scans (redone once if step 4 drops an adapter)
  int pair_base = 0, seg_base = 0, u_base = 0, row_base = 0;
  for (int pass = 0; pass < 2; ++pass) {
    const int bmask = s_bmask;
    pair_base = seg_base = u_base = row_base = 0;
    for (int b = 0; b < LORA_N_BUCKETS; ++b) {
      if (tid == 0) P[L.bucket_seg_off + b] = seg_base;
      if (!(bmask & (1 << b))) continue;
      Scan4 x{{0, 0, 0, 0}};
      for (int ad = a0; ad < a1; ++ad) {
        const int c = ld_ctr(&cnt[ad]);
        const int r = inf[ad] & kInfRankMask;
        if (c > 0 && rank_bucket(r) == b) {
          x.v[0] += c; x.v[1] += 1; x.v[2] += c * r; x.v[3] += r;
        }
      }
      Scan4 tot;
      const Scan4 ex = block_exclusive_scan4(x, tot, lds_tot);
      int st = pair_base + ex.v[0], sg = seg_base + ex.v[1];
      int ub = u_base + ex.v[2], rb = row_base + ex.v[3];
      for (int ad = a0; ad < a1; ++ad) {
        const int c = ld_ctr(&cnt[ad]);
        const int r = inf[ad] & kInfRankMask;
        if (c > 0 && rank_bucket(r) == b) {
          start[ad] = st;
          ustart[ad] = ub;
          st_ctr(&cur[ad], st);
          seg_ad[sg] = ad;
          seg_row[sg] = rb;
          if (kLds) {
            P[L.seg_adapter + sg] = ad;
            P[L.seg_row_off + sg] = rb;
          }
          P[L.seg_off + sg] = st;
          int4 *d = reinterpret_cast<int4 *>(P + L.seg_desc) + 2 * sg;
          d[0] = make_int4(ad, r, psa[ad], st);
          d[1] = make_int4(st + c, ub, rb, 0);
          st += c; sg += 1; ub += c * r; rb += r;
        }
      }
      pair_base += tot.v[0];
      seg_base += tot.v[1];
      u_base += tot.v[2];
      row_base += tot.v[3];
    }
    if (tid == 0) {
      P[L.bucket_seg_off + LORA_N_BUCKETS] = seg_base;
      P[L.seg_off + seg_base] = pair_base;
      seg_row[seg_base] = row_base;
      if (kLds) P[L.seg_row_off + seg_base] = row_base;
      P[L.u_off + pair_base] = u_base;
    }
    __syncthreads();
    if (pass == 1) break;
    // 4. page ids of every used rank row, in parallel over rows
    for (int g = tid; g < row_base; g += kPlanThreads) {
      int lo = 0, hi = seg_base;
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (seg_row[mid] <= g) lo = mid; else hi = mid;
      }
      const int ad = seg_ad[lo];
      const int64_t pg = a.page_ids[int64_t(psa[ad]) + (g - seg_row[lo])];
      if (pg < 0 || pg >= a.n_pages) {
        st_ctr(&cnt[ad], -1);
        s_bad = 1;
      }
    }
    __syncthreads();
    if (s_bad == 0) break;
    if (tid == 0) {
      atomicOr(&s_err, LORA_DEVERR_BAD_POOL);
      s_bmask = 0;
    }
    __syncthreads();
    {   // the occupancy mask may have lost buckets: rebuild it
      int bm = 0;
      for (int ad = a0; ad < a1; ++ad)
        if (ld_ctr(&cnt[ad]) > 0) bm |= 1 << rank_bucket(inf[ad] & kInfRankMask);
      if (bm) atomicOr(&s_bmask, bm);
    }
    __syncthreads();
  }

  // 5. ordered placement, one wave at a time within each 1024-slot chunk
  const uint64_t lt_mask = (uint64_t(1) << lane) - 1;
  int4 *slot_desc = reinterpret_cast<int4 *>(P + L.slot_desc);
  for (int64_t base = 0; base < TK; base += kPlanThreads) {
    const int64_t i = base + tid;
    int ad = -1;
    if (i < TK) {
      if (a.slot_cache) {
        ad = slot_ad[i];
      } else {
        const int id = a.ids[i];
        if (id >= 0 && id < N) {
          const int v = inf[id];
          if (!(v & kInfBadRank) && (v & kInfRankMask) > 0 && a.gates[i] != 0.0f) ad = id;
        }
      }
      if (ad >= 0 && ld_ctr(&cnt[ad]) <= 0) ad = -1;
    }
    const uint64_t mm = match_lanes(ad, nbits);
    const int rank_in_wave = __popcll(mm & lt_mask);
    const int leader = mm ? __ffsll((unsigned long long)mm) - 1 : lane;
    int pos = -1;
    for (int w = 0; w < kPlanThreads / 64; ++w) {
      __syncthreads();
      if (wave == w) {
        int b0 = 0;
        if (ad >= 0 && rank_in_wave == 0) b0 = atomicAdd(&cur[ad], __popcll(mm));
        b0 = __shfl(b0, leader, 64);
        if (ad >= 0) pos = b0 + rank_in_wave;
      }
    }
    if (i < TK) {
      P[L.slot_pos + i] = pos;
      if (pos >= 0) {
        const int r = inf[ad] & kInfRankMask;
        const int uo = ustart[ad] + (pos - start[ad]) * r;
        P[L.pair_tk + pos] = int32_t(i);
        P[L.pair_adapter + pos] = ad;
        P[L.u_off + pos] = uo;
        slot_desc[i] = make_int4(pos, r, uo, psa[ad]);
      } else {
        slot_desc[i] = make_int4(-1, 0, 0, 0);
      }
    }
  }
  __syncthreads();
  if (tid == 0) {
    int32_t *h = P + L.hdr;
    h[LORA_PH_PAIRS] = pair_base;
    h[LORA_PH_SEGS] = seg_base;
    h[LORA_PH_ERR] = s_err;
    h[LORA_PH_RPAIRS] = u_base;
    h[LORA_PH_RUSED] = row_base;
    h[LORA_PH_T] = a.T;
    h[LORA_PH_K] = a.K;
    h[LORA_PH_N] = N;
    for (int q = 8; q < LORA_PLAN_HEADER_INTS; ++q) h[q] = 0;
    for (int q = LORA_N_BUCKETS + 1; q < 16; ++q) P[L.bucket_seg_off + q] = 0;
  }
}

}  // namespace

hipError_t launch_plan(const int32_t *ids, const float *gates, int T, int K, const PoolView &pool,
                       int32_t *plan, hipStream_t s) {
  const int64_t TK = int64_t(T) * K;
  const int64_t N = pool.n_adapters;
  const int64_t Smax = TK < N ? TK : N;
  PlanArgs a{ids, gates, T, K, pool.n_adapters, pool.rank, pool.page_start, pool.page_ids,
             pool.n_pages, pool.n_page_ids, plan, 0};
  const int64_t adapter_ints = 4 * N + 2 * Smax + 1;
  if (adapter_ints <= kPlanLdsInts) {
    a.slot_cache = adapter_ints + TK <= kPlanLdsInts ? 1 : 0;
    const size_t lds = size_t(adapter_ints + (a.slot_cache ? TK : 0)) * sizeof(int);
    hipLaunchKernelGGL(plan_kernel<true>, dim3(1), dim3(kPlanThreads), lds, s, a);
  } else {
    a.slot_cache = TK <= kPlanLdsInts ? 1 : 0;
    const size_t lds = size_t(a.slot_cache ? TK : 0) * sizeof(int);
    hipLaunchKernelGGL(plan_kernel<false>, dim3(1), dim3(kPlanThreads), lds, s, a);
  }
  return hipGetLastError();
}

}  // namespace lora
