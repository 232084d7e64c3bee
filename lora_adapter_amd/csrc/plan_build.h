// The plan: one workgroup groups a batch's active (token, slot) pairs by
// adapter.  A device function, run by the plan kernel and by the split GEMM
// launches that build the plan in their first workgroup beside the base
// product (which does not depend on the routing).
//
// Segmented gather needs the rows of one adapter together (AdaFuse notes,
// section 关键设计 item 3); rank-specialised execution needs segments grouped
// by rank (LoRAForge page, section LoRAForge的核心设计 and its note on
// rank-specialised kernels).  The output is a stable counting sort by the key
// (rank bucket, adapter, token, slot) plus the offsets and packed descriptors
// the later kernels use.  All integer: bit-exact and deterministic.
//
// One workgroup builds the whole plan.  At decode sizes the cost is latency:
// every wave of a workgroup shares one CU's four SIMDs, so each step costs
// its instruction count times the waves per SIMD.  The block is therefore
// sized to the problem (64 threads for a 64-token batch over 64 adapters, up
// to 1024), and the kernel is organised around few global round trips and
// few barriers:
//   0. adapters are dealt to threads round-robin; each thread loads rank and
//      page_start of its adapters (the first slots' ids and gates are already
//      in flight);
//   1. each slot is classified (adapter data from LDS) and counted per adapter;
//   2. page_start consistency of every used adapter; bucket occupancy;
//   3. segment order: one ballot per occupied bucket gives every used adapter
//      its rank among the used adapters of its bucket dealt to its wave; the
//      per-wave counts are scanned (one wave per bucket), which places every
//      adapter in (bucket, adapter) order; one block scan over the segments
//      then gives pair, U and rank-row offsets;
//   4. page ids of every used rank row are range-checked in parallel over rows
//      (a bad adapter is dropped and step 3 redone once);
//   5. pairs are placed in slot order: lanes holding the same adapter find
//      each other with one ballot per id bit, the first of them takes
//      positions from the adapter's cursor, and the waves of each chunk of
//      slots (one slot per thread) take their turns in order, which keeps the
//      sort stable; with a (wave, adapter) count table in LDS, every slot
//      instead adds the counts of the chunk's earlier waves to the cursor,
//      the same positions with three barriers a chunk instead of one a wave;
//      and when a (chunk, wave, adapter) table fits, step 1 fills it, one
//      scan per adapter turns it into start positions, and the placement
//      needs no barrier at all.
// The ids and gates of the first 8 chunks of slots are fetched in one round
// trip at the start (a later chunk's loads would each be one more).
// Per-adapter arrays live in LDS when they fit (96 KiB); then the barriers
// order LDS only, and global stores (outputs only) never stall them.  Larger
// pools keep those arrays in the plan buffer's scratch (agent-scope atomics
// where counters change, full barriers).
#pragma once
#include "lora_internal.h"

namespace lora {
namespace {

constexpr int kInfBadRank = 1 << 11;   // rank < 0 or > LORA_MAX_RANK
constexpr int kInfBadStart = 1 << 12;  // page_start inconsistent with rank
constexpr int kInfRankMask = 0x7ff;
constexpr int kMaxWaves = kPlanThreads / 64;
// Per-bucket entries of the (round, wave) count table: at most N/64 + 16.
// When the per-adapter arrays fit LDS (N <= kPlanLdsInts / 5) this bound is:
constexpr int kLdsCountCols = kPlanLdsInts / 5 / 64 + kMaxWaves + 1;


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

// Workgroup barrier.  With every shared array in LDS it orders LDS only, so
// outstanding global stores do not hold it up.
template <bool kLds>
__device__ __forceinline__ void bar() {
  if constexpr (kLds) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
  } else {
    __syncthreads();
  }
}

// Bitwise OR over the wave of a value below 2^LORA_N_BUCKETS (wave-uniform).
__device__ __forceinline__ int wave_or_buckets(int v) {
  int r = 0;
#pragma unroll
  for (int b = 0; b < LORA_N_BUCKETS; ++b)
    if (__ballot((v >> b) & 1)) r |= 1 << b;
  return r;
}

// Inclusive prefix sum over the 64 lanes of a wave: shifts by 1, 2, 4, 8
// within each row of 16 lanes, then the last lane of row 0 is added to row 1
// and row 3, and the last lane of row 1 to rows 2 and 3 (DPP row broadcasts).
__device__ __forceinline__ int wave_scan_incl(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, false);   // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, false);   // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, false);   // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, false);   // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false);   // row_bcast:15
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false);   // row_bcast:31
  return v;
}

template <int NV>
struct ScanV {
  int v[NV];
};

// Exclusive block scan of NV ints over the workgroup; also the totals.
// Wave totals go through LDS once; every wave then scans the (at most 16)
// totals in its lanes.
template <bool kLds, int NV>
__device__ ScanV<NV> block_exclusive_scan(ScanV<NV> x, ScanV<NV> &total, int *lds_tot /* [16*NV] */) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nwv = blockDim.x >> 6;
  ScanV<NV> inc;
#pragma unroll
  for (int q = 0; q < NV; ++q) inc.v[q] = wave_scan_incl(x.v[q]);
  if (lane == 63) {
#pragma unroll
    for (int q = 0; q < NV; ++q) lds_tot[wave * NV + q] = inc.v[q];
  }
  bar<kLds>();
  int tw[NV];
#pragma unroll
  for (int q = 0; q < NV; ++q) tw[q] = lds_tot[min(lane, nwv - 1) * NV + q];
  ScanV<NV> ex;
#pragma unroll
  for (int q = 0; q < NV; ++q) {
    const int t = lane < nwv ? tw[q] : 0;
    const int ti = wave_scan_incl(t);
    const int before = __builtin_amdgcn_readlane(ti - t, wave);
    total.v[q] = __builtin_amdgcn_readlane(ti, 63);
    ex.v[q] = before + inc.v[q] - x.v[q];
  }
  bar<kLds>();  // lds_tot is reused by the next call
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

// Loads in flight per thread in the adapter and page-id passes.
constexpr int kPreChunks = 8;        // chunks of nt slots whose ids and gates are fetched up front
constexpr int kAdBatch = 4;
constexpr int kRowBatch = 12;
constexpr int kWsBatch = 8;

// The whole plan, built by the calling workgroup (64..1024 threads, any
// block size).  dyn: LDS for the per-adapter arrays (kLds) and the slot cache.
template <bool kLds>
__device__ __forceinline__ void plan_build(const PlanArgs &a, int *dyn) {
  __shared__ int lds_tot[kMaxWaves * 5];
  __shared__ int s_wcnt[kLds ? LORA_N_BUCKETS * kLdsCountCols : 1];
  __shared__ int s_btot[LORA_N_BUCKETS];
  __shared__ int s_err, s_bmask, s_bad;

  const int tid = threadIdx.x;
  const int nt = blockDim.x, nwv = nt >> 6;   // 64..1024 threads, chosen by problem size
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const uint64_t lt_mask = (uint64_t(1) << lane) - 1;
  const int N = a.N;
  const int64_t TK = int64_t(a.T) * a.K;
  const int Smax = int(TK < N ? TK : N);
  const PlanLayout L = plan_layout(TK, N);
  int32_t *P = a.plan;
  // per-adapter arrays; ubias[a] = U offset of the adapter's first pair minus
  // (its first pair position) * rank, so that a pair at position p starts at
  // ubias[a] + p * rank
  int *cnt = kLds ? dyn : P + L.cnt;
  int *cur = kLds ? dyn + N : P + L.cur;
  int *psa = kLds ? dyn + 2 * N : P + L.ps;
  int *inf = kLds ? dyn + 3 * N : P + L.inf;
  int *ubias = kLds ? dyn + 4 * N : P + L.ubias;
  // segment arrays (outputs; LDS copies when they fit)
  int *seg_row = kLds ? dyn + 5 * N : P + L.seg_row_off;
  int *seg_ad = kLds ? dyn + 5 * N + Smax + 1 : P + L.seg_adapter;
  // LDS case only: seg_pgb[s] = page_start of segment s's adapter minus its
  // first rank row; seg_pp[s] = its first pair (copy of the seg_off output)
  int *seg_pgb = dyn + 5 * N + 2 * Smax + 1;
  int *seg_pp = dyn + 5 * N + 3 * Smax + 1;
  // first decode-shrink unit of each segment
  int *seg_uo = kLds ? dyn + 5 * N + 4 * Smax + 2 : P + L.seg_uoff;
  int *slot_ad = dyn + (kLds ? 5 * N + 5 * Smax + 3 : 0);
  // the whole page table, when it fits (its range check then needs no
  // global round trip after the segment order)
  int *slot_g = slot_ad + TK;                 // gate bits of each slot (with the cache)
  int *pcache = slot_ad + (a.slot_cache ? 2 * TK : 0);
  // place_table 1: placement counts per (wave, adapter), zero between
  // chunks; 2: per (chunk, wave, adapter), counted by step 1 and turned into
  // start positions before step 5
  const int nch = int((TK + nt - 1) / nt);
  int *ptab = pcache + (a.page_cache ? a.n_page_ids : 0);
  if (a.place_table)
    for (int e = tid; e < (a.place_table == 2 ? nch : 1) * nwv * N; e += nt) ptab[e] = 0;
  // counts of used adapters per (bucket, round of nt adapters, wave)
  const int Q = (N + nt - 1) / nt;
  const int E = Q * nwv;
  int *wcnt = kLds ? s_wcnt : P + L.wcnt;

  // The first kPreChunks x nt slots are fetched now, in one round trip that
  // overlaps the adapter loads below (each later chunk costs a round trip).
  int id_pre[kPreChunks];
  float g_pre[kPreChunks];
#pragma unroll
  for (int c = 0; c < kPreChunks; ++c) {
    const int64_t i = int64_t(c) * nt + tid;
    id_pre[c] = -1;
    g_pre[c] = 0.0f;
    if (i < TK) {
      id_pre[c] = a.ids[i];
      g_pre[c] = a.gates[i];
    }
  }

  // 0. per-adapter data; adapter ad belongs to thread ad % nt.  The page
  //    table is copied to LDS first (when cached), so that its loads are in
  //    flight with the adapter loads.
  if (tid == 0) { s_err = 0; s_bmask = 0; s_bad = 0; }
  if (a.page_cache) {
    const int npi = int(a.n_page_ids);
    for (int b0 = tid; b0 < npi; b0 += nt * kAdBatch) {
      int v[kAdBatch];
#pragma unroll
      for (int q = 0; q < kAdBatch; ++q) v[q] = a.page_ids[min(b0 + q * nt, npi - 1)];
#pragma unroll
      for (int q = 0; q < kAdBatch; ++q)
        if (b0 + q * nt < npi) pcache[b0 + q * nt] = v[q];
    }
  }
  for (int base = tid; base < N; base += nt * kAdBatch) {
    int r[kAdBatch], s0[kAdBatch], s1[kAdBatch];
#pragma unroll
    for (int q = 0; q < kAdBatch; ++q) {
      const int ad = min(base + q * nt, N - 1);
      r[q] = a.rank[ad];
      s0[q] = a.page_start[ad];
      s1[q] = a.page_start[ad + 1];
    }
#pragma unroll
    for (int q = 0; q < kAdBatch; ++q) {
      const int ad = base + q * nt;
      if (ad >= N) break;
      int v = (r[q] < 0 || r[q] > LORA_MAX_RANK) ? kInfBadRank : r[q];
      if (s0[q] < 0 || int64_t(s1[q]) - s0[q] != int64_t(r[q]) || s1[q] > a.n_page_ids)
        v |= kInfBadStart;
      inf[ad] = v;
      psa[ad] = s0[q];
      st_ctr(&cnt[ad], 0);
    }
  }
  bar<kLds>();

  // 1. classify and count
  const int nbits = N > 1 ? 32 - __clz(N - 1) : 1;
  int err = 0;
  auto classify = [&](int64_t i, int ch, int id, float g) __attribute__((always_inline)) {
    int ad = -1;
    if (i < TK) {
      if (id < -1 || id >= N) {
        err |= LORA_DEVERR_BAD_ID;
      } else if (id >= 0) {
        const int v = inf[id];
        if (v & kInfBadRank) err |= LORA_DEVERR_BAD_RANK;
        else if ((v & kInfRankMask) > 0 && g != 0.0f) ad = id;
      }
      if (a.slot_cache) slot_g[i] = __float_as_int(g);
    }
    const uint64_t mm = match_lanes(ad, nbits);
    // place_table 2 packs the slot's rank among its wave's slots of ad
    // (below 64; ad < 2^25 there, as the table fits in LDS)
    if (a.slot_cache && i < TK)
      slot_ad[i] = a.place_table == 2 && ad >= 0 ? ad * 64 + __popcll(mm & lt_mask) : ad;
    if (ad >= 0 && (mm & lt_mask) == 0) {
      atomicAdd(&cnt[ad], __popcll(mm));
      if (a.place_table == 2) ptab[(ch * nwv + wave) * N + ad] = __popcll(mm);
    }
  };
#pragma unroll
  for (int c = 0; c < kPreChunks; ++c)
    if (int64_t(c) * nt < TK) classify(int64_t(c) * nt + tid, c, id_pre[c], g_pre[c]);
  {
    int ch = kPreChunks;
    for (int64_t base = int64_t(kPreChunks) * nt; base < TK; base += nt, ++ch) {
      const int64_t i = base + tid;
      classify(i, ch, i < TK ? a.ids[i] : -1, i < TK ? a.gates[i] : 0.0f);
    }
  }
  if (err) atomicOr(&s_err, err);
  bar<kLds>();

  // 2. page_start consistency of used adapters (and, with the page table in
  //    LDS, the range of their page ids); bucket occupancy
  {
    int bm = 0;
    for (int ad = tid; ad < N; ad += nt) {
      const int c = ld_ctr(&cnt[ad]);
      if (c <= 0) continue;
      const int v = inf[ad];
      bool ok = !(v & kInfBadStart);
      if (ok && a.page_cache) {
        const int ps = psa[ad], r = v & kInfRankMask;
        int bad = 0;
        for (int j0 = 0; j0 < r; j0 += 8) {      // 8 LDS reads in flight
          int pg[8];
#pragma unroll
          for (int q = 0; q < 8; ++q) pg[q] = pcache[ps + min(j0 + q, r - 1)];
#pragma unroll
          for (int q = 0; q < 8; ++q) bad |= (pg[q] < 0 || pg[q] >= a.n_pages) ? 1 : 0;
        }
        ok = bad == 0;
      }
      if (!ok) {
        st_ctr(&cnt[ad], -1);
        atomicOr(&s_err, LORA_DEVERR_BAD_POOL);
      } else {
        bm |= 1 << rank_bucket(v & kInfRankMask);
      }
    }
    bm = wave_or_buckets(bm);
    if (lane == 0 && bm) atomicOr(&s_bmask, bm);
  }
  bar<kLds>();

  // 3. segment order (redone once if step 4 drops an adapter; step 4 is not
  //    needed when the page table was checked in step 2)
  int S = 0, pair_base = 0, u_base = 0, row_base = 0, n_units = 0, n_big = 0;
  for (int pass = 0; pass < 2; ++pass) {
    const int bmask = s_bmask;
    // (a) used adapters per (bucket, round, wave)
    for (int q = 0; q < Q; ++q) {
      const int ad = q * nt + tid;
      int b = -1;
      if (ad < N && ld_ctr(&cnt[ad]) > 0) b = rank_bucket(inf[ad] & kInfRankMask);
#pragma unroll
      for (int bb = 0; bb < LORA_N_BUCKETS; ++bb) {
        if (!((bmask >> bb) & 1)) continue;
        const uint64_t m = __ballot(b == bb);
        if (lane == 0) st_ctr(&wcnt[bb * E + q * nwv + wave], __popcll(m));
      }
    }
    bar<kLds>();
    // (b) exclusive scan of each occupied bucket's counts; bucket b is
    //     scanned by wave b % nwv (every bucket total is written)
    for (int b = wave; b < LORA_N_BUCKETS; b += nwv) {
      int carry = 0;
      if ((bmask >> b) & 1) {
        for (int e0 = 0; e0 < E; e0 += 64) {
          const int e = e0 + lane;
          const int v = e < E ? ld_ctr(&wcnt[b * E + e]) : 0;
          const int inc = wave_scan_incl(v);
          if (e < E) st_ctr(&wcnt[b * E + e], carry + inc - v);
          carry += __builtin_amdgcn_readlane(inc, 63);
        }
      }
      if (lane == 0) s_btot[b] = carry;
    }
    bar<kLds>();
    // (c) each used adapter's segment index: first segment of its bucket +
    //     used adapters of the bucket in earlier (round, wave) cells + its rank
    //     among the wave's lanes of that bucket
    {
      const int bt = lane < LORA_N_BUCKETS ? s_btot[lane] : 0;
      const int bi = wave_scan_incl(bt);
      // lanes 0..9 of wave 0 (with the arrays in LDS: stored at the end)
      if (!kLds && tid <= LORA_N_BUCKETS) P[L.bucket_seg_off + tid] = bi - bt;
      S = __builtin_amdgcn_readlane(bi, 63);
      for (int q = 0; q < Q; ++q) {
        const int ad = q * nt + tid;
        int b = -1;
        if (ad < N && ld_ctr(&cnt[ad]) > 0) b = rank_bucket(inf[ad] & kInfRankMask);
        int rk = 0;
#pragma unroll
        for (int bb = 0; bb < LORA_N_BUCKETS; ++bb) {
          if (!((bmask >> bb) & 1)) continue;
          const uint64_t m = __ballot(b == bb);
          if (b == bb) rk = __popcll(m & lt_mask);
        }
        const int bs = __shfl(bi - bt, b < 0 ? 0 : b, 64);   // first segment of bucket b
        if (b >= 0) seg_ad[bs + ld_ctr(&wcnt[b * E + q * nwv + wave]) + rk] = ad;
      }
    }
    bar<kLds>();
    // (d) pair, U, rank-row and decode-shrink-unit offsets of the segments
    //     (contiguous blocks per thread), and the list of big segments
    const int ms = (S + nt - 1) / nt;
    const int g0 = min(S, tid * ms), g1 = min(S, g0 + ms);
    ScanV<5> x{{0, 0, 0, 0, 0}};
    for (int sg = g0; sg < g1; ++sg) {
      const int ad = seg_ad[sg];
      const int c = ld_ctr(&cnt[ad]);
      const int r = inf[ad] & kInfRankMask;
      const bool big = a.use_tile && c >= kBigSegPairs;
      x.v[0] += c; x.v[1] += c * r; x.v[2] += r;
      // decode-shrink units: every pair of a small segment, the last c % 16
      // pairs of a big one (its whole 32-pair tiles go to the MFMA shrink)
      x.v[3] += (big ? c % kTileTok : c) * ((r + kShrinkRows - 1) / kShrinkRows);
      x.v[4] += big ? 1 : 0;
    }
    ScanV<5> tot;
    const ScanV<5> ex = block_exclusive_scan<kLds, 5>(x, tot, lds_tot);
    int st = ex.v[0], ub = ex.v[1], rb = ex.v[2], uo = ex.v[3], bi = ex.v[4];
    for (int sg = g0; sg < g1; ++sg) {
      const int ad = seg_ad[sg];
      const int c = ld_ctr(&cnt[ad]);
      const int r = inf[ad] & kInfRankMask;
      const bool big = a.use_tile && c >= kBigSegPairs;
      ubias[ad] = ub - st * r;
      st_ctr(&cur[ad], st);
      seg_row[sg] = rb;
      seg_uo[sg] = uo;
      if (kLds) {
        seg_pgb[sg] = psa[ad] - rb;
        seg_pp[sg] = st;
      } else {
        P[L.seg_off + sg] = st;
        int4 *d = reinterpret_cast<int4 *>(P + L.seg_desc) + 2 * sg;
        d[0] = make_int4(ad, r, psa[ad], st);
        d[1] = make_int4(st + c, ub, rb, uo);
      }
      if (big) P[L.big_list + 1 + bi] = sg;
      st += c; ub += c * r; rb += r; bi += big ? 1 : 0;
      uo += (big ? c % kTileTok : c) * ((r + kShrinkRows - 1) / kShrinkRows);
    }
    pair_base = tot.v[0];
    u_base = tot.v[1];
    row_base = tot.v[2];
    n_units = tot.v[3];
    n_big = tot.v[4];
    if (tid == 0) {
      seg_row[S] = row_base;
      seg_uo[S] = n_units;
      if (kLds) {
        seg_pp[S] = pair_base;
      } else {
        P[L.seg_off + S] = pair_base;
        P[L.u_off + pair_base] = u_base;
        P[L.big_list] = n_big;
      }
    }
    bar<kLds>();
    if (pass == 1 || a.page_cache) break;   // page ids already checked
    // 4. page ids of every used rank row, kRowBatch rows per thread in flight.
    //    Row g belongs to the last segment whose first row is <= g (segment
    //    row offsets strictly increase), found by binary lifting.
    int top = 1;
    while (top * 2 <= S) top *= 2;
    for (int h0 = 0; h0 < row_base; h0 += nt * kRowBatch) {
      const int nq = min(kRowBatch, (row_base - h0 + nt - 1) / nt);   // uniform
      int lo[kRowBatch], gq[kRowBatch], pg[kRowBatch];
#pragma unroll
      for (int q = 0; q < kRowBatch; ++q) {
        gq[q] = min(h0 + q * nt + tid, row_base - 1);
        lo[q] = 0;
      }
      // seg_row[S] = row_base exceeds every row, so clamping to S never moves lo.
      // Every slot of the batch is searched and loaded, past nq too (its row
      // is clamped to the last one, a valid row): a load under a condition
      // leaves the compiler waiting for each load before the next.
      for (int step = top; step > 0; step >>= 1) {
        int rc[kRowBatch];
#pragma unroll
        for (int q = 0; q < kRowBatch; ++q) rc[q] = seg_row[min(lo[q] + step, S)];
#pragma unroll
        for (int q = 0; q < kRowBatch; ++q) lo[q] = rc[q] <= gq[q] ? min(lo[q] + step, S) : lo[q];
      }
      int pix[kRowBatch];
      if constexpr (kLds) {
#pragma unroll
        for (int q = 0; q < kRowBatch; ++q) pix[q] = seg_pgb[lo[q]] + gq[q];
      } else {
#pragma unroll
        for (int q = 0; q < kRowBatch; ++q) pix[q] = psa[seg_ad[lo[q]]] - seg_row[lo[q]] + gq[q];
      }
#pragma unroll
      for (int q = 0; q < kRowBatch; ++q) pg[q] = a.page_ids[pix[q]];
#pragma unroll
      for (int q = 0; q < kRowBatch; ++q) {
        if (q < nq && h0 + q * nt + tid < row_base && (pg[q] < 0 || pg[q] >= a.n_pages)) {
          st_ctr(&cnt[seg_ad[lo[q]]], -1);
          s_bad = 1;
        }
      }
    }
    bar<kLds>();
    if (s_bad == 0) break;
    if (tid == 0) {
      atomicOr(&s_err, LORA_DEVERR_BAD_POOL);
      s_bmask = 0;
    }
    bar<kLds>();
    {   // the occupancy mask may have lost buckets: rebuild it
      int bm = 0;
      for (int ad = tid; ad < N; ad += nt)
        if (ld_ctr(&cnt[ad]) > 0) bm |= 1 << rank_bucket(inf[ad] & kInfRankMask);
      bm = wave_or_buckets(bm);
      if (lane == 0 && bm) atomicOr(&s_bmask, bm);
    }
    bar<kLds>();
  }

  // place_table 2: each used adapter's (chunk, wave) counts, in slot order,
  // become start positions: its first pair plus the exclusive scan.  A pool
  // of a few adapters takes one wave per adapter (a wave-wide scan of its
  // counts); larger pools one lane per adapter walking its counts in order,
  // so that no wave steps through the adapters one LDS round trip at a time
  // (1024 adapters on 4 waves: 256 dependent trips each)
  if (a.place_table == 2) {
    const int EC = nch * nwv;
    if (N > 2 * nwv) {
      for (int ad = tid; ad < N; ad += nt) {
        if (ld_ctr(&cnt[ad]) <= 0) continue;
        int carry = ld_ctr(&cur[ad]);
        for (int e0 = 0; e0 < EC; e0 += 8) {
          int v[8];
#pragma unroll
          for (int q = 0; q < 8; ++q) v[q] = e0 + q < EC ? ptab[(e0 + q) * N + ad] : 0;
#pragma unroll
          for (int q = 0; q < 8; ++q) {
            if (e0 + q < EC) ptab[(e0 + q) * N + ad] = carry;
            carry += v[q];
          }
        }
      }
    } else {
      for (int ad = wave; ad < N; ad += nwv) {
        if (ld_ctr(&cnt[ad]) <= 0) continue;
        int carry = ld_ctr(&cur[ad]);
        for (int e0 = 0; e0 < EC; e0 += 64) {
          const int e = e0 + lane;
          const int v = e < EC ? ptab[e * N + ad] : 0;
          const int inc = wave_scan_incl(v);
          if (e < EC) ptab[e * N + ad] = carry + inc - v;
          carry += __builtin_amdgcn_readlane(inc, 63);
        }
      }
    }
    bar<kLds>();
  }

  // U per slot to the u_off layout needs room for R_pairs floats
  const bool copy_u = a.slot_u != nullptr && int64_t(u_base) <= a.u_cap;
  if (a.slot_u != nullptr && !copy_u && tid == 0) atomicOr(&s_err, LORA_DEVERR_CAPACITY);
  // Every global load so far has landed: waiting here (no store is in flight
  // yet) settles them, so that the loops below, which store, need no flush
  // of the counter that, on this target, also counts stores.
  __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
  // 5. ordered placement: within each nt-slot chunk the waves holding slots
  //    take positions from the adapter cursors in wave order (stable sort)
  int4 *slot_desc = reinterpret_cast<int4 *>(P + L.slot_desc);
  // the slot's outputs: its position, and for a placed pair the pair arrays,
  // its descriptor and (decode) its U moved to the u_off layout
  auto emit = [&](int64_t i, int ad, int pos, float gate) __attribute__((always_inline)) {
    P[L.slot_pos + i] = pos;
    if (pos >= 0) {
      const int r = inf[ad] & kInfRankMask;
      const int uo = ubias[ad] + pos * r;
      P[L.pair_tk + pos] = int32_t(i);
      P[L.pair_adapter + pos] = ad;
      P[L.pair_gate + pos] = __float_as_int(gate);
      P[L.u_off + pos] = uo;
      slot_desc[i] = make_int4(pos, r, uo, psa[ad]);
      if (copy_u) {
        // this slot's U (per-slot layout, 16-byte aligned rows of
        // slot_stride floats) to its u_off place: 8 loads in flight
        const float4 *src = reinterpret_cast<const float4 *>(a.slot_u + i * int64_t(a.slot_stride));
        for (int j0 = 0; j0 < r; j0 += 32) {
          float4 v[8];
#pragma unroll
          for (int q = 0; q < 8; ++q) v[q] = src[min(j0 / 4 + q, (r - 1) / 4)];
#pragma unroll
          for (int q = 0; q < 8; ++q) {
            const float e4[4] = {v[q].x, v[q].y, v[q].z, v[q].w};
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (j0 + 4 * q + e < r) a.u_out[uo + j0 + 4 * q + e] = e4[e];
          }
        }
      }
    } else {
      slot_desc[i] = make_int4(-1, 0, 0, 0);
    }
  };
  if (a.place_table == 2) {
    // no barrier and no ballot: the slot cache holds each slot's adapter and
    // its rank among its wave's slots of that adapter (step 1), the table the
    // start of every (chunk, wave, adapter)
    int ch = 0;
    for (int64_t base = 0; base < TK; base += nt, ++ch) {
      const int64_t i = base + tid;
      if (i >= TK) break;
      const int sa = slot_ad[i];
      const int ad = sa >= 0 ? sa >> 6 : -1;
      int pos = -1;
      if (ad >= 0 && ld_ctr(&cnt[ad]) > 0) pos = ptab[(ch * nwv + wave) * N + ad] + (sa & 63);
      emit(i, pos >= 0 ? ad : -1, pos, __int_as_float(slot_g[i]));
    }
  } else {
    for (int64_t base = 0; base < TK; base += nt) {
      const int64_t i = base + tid;
      int ad = -1;
      float gate = 0.0f;
      if (i < TK) {
        if (a.slot_cache) {
          ad = slot_ad[i];
          gate = __int_as_float(slot_g[i]);
        } else {
          const int id = a.ids[i];
          gate = a.gates[i];
          if (id >= 0 && id < N) {
            const int v = inf[id];
            if (!(v & kInfBadRank) && (v & kInfRankMask) > 0 && gate != 0.0f) ad = id;
          }
        }
        if (ad >= 0 && ld_ctr(&cnt[ad]) <= 0) ad = -1;
      }
      const uint64_t mm = match_lanes(ad, nbits);
      const int rank_in_wave = __popcll(mm & lt_mask);
      const int leader = mm ? __ffsll((unsigned long long)mm) - 1 : lane;
      const int64_t here = TK - base < nt ? TK - base : nt;
      const int nw = int((here + 63) >> 6);
      int pos = -1;
      if (a.place_table == 1) {
        // the same positions as the waves taking turns: the adapter's cursor,
        // plus its slots in the chunk's earlier waves (the count table), plus
        // the slot's rank in its own wave; cursors move after every wave has
        // read them, and each wave clears its own table entries
        const bool lead = ad >= 0 && rank_in_wave == 0;
        bar<kLds>();
        if (lead) ptab[wave * N + ad] = __popcll(mm);
        bar<kLds>();
        if (ad >= 0) {
          int before = 0;
          for (int w = 0; w < wave; ++w) before += ptab[w * N + ad];
          pos = ld_ctr(&cur[ad]) + before + rank_in_wave;
        }
        bar<kLds>();
        if (lead) {
          atomicAdd(&cur[ad], __popcll(mm));
          ptab[wave * N + ad] = 0;
        }
      } else {
        for (int w = 0; w < nw; ++w) {
          bar<kLds>();
          if (wave == w) {
            int b0 = 0;
            if (ad >= 0 && rank_in_wave == 0) b0 = atomicAdd(&cur[ad], __popcll(mm));
            b0 = __shfl(b0, leader, 64);
            if (ad >= 0) pos = b0 + rank_in_wave;
          }
        }
      }
      if (i < TK) emit(i, ad, pos, gate);
    }
  }
  bar<kLds>();

  // 4b. decode-shrink schedule (skipped when no_sched: the decode shrink then
  //     finds each wave's start itself): its units (pairs x groups of kShrinkRows rank
  //     rows, over the segments it handles) split into equal runs, one per
  //     wave; each working wave's first segment and unit, with that
  //     segment's descriptor, so that a shrink wave starts with one load.
  //     Runs are found kWsBatch at a time by binary lifting over the
  //     segments' first units (seg_uo[S] = n_units exceeds every unit).
  {
    const int upw = max(1, (n_units + kShrinkWaves - 1) / kShrinkWaves);
    const int n_active = (n_units + upw - 1) / upw;       // <= kShrinkWaves
    int top = 1;
    while (top * 2 <= S) top *= 2;
    int4 *ws = reinterpret_cast<int4 *>(P + L.wave_start);
    for (int w0 = 0; w0 < (a.no_sched ? 0 : n_active); w0 += nt * kWsBatch) {
      int lo[kWsBatch], uq[kWsBatch];
#pragma unroll
      for (int q = 0; q < kWsBatch; ++q) {
        uq[q] = min(w0 + q * nt + tid, n_active - 1) * upw;
        lo[q] = 0;
      }
      for (int step = top; step > 0; step >>= 1) {
        int rc[kWsBatch];
#pragma unroll
        for (int q = 0; q < kWsBatch; ++q) rc[q] = seg_uo[min(lo[q] + step, S)];
#pragma unroll
        for (int q = 0; q < kWsBatch; ++q) lo[q] = rc[q] <= uq[q] ? min(lo[q] + step, S) : lo[q];
      }
#pragma unroll
      for (int q = 0; q < kWsBatch; ++q) {
        const int w = w0 + q * nt + tid;
        if (w < n_active) {
          const int sg = lo[q];
          const int ad = seg_ad[sg];
          const int pb = kLds ? seg_pp[sg] : P[L.seg_off + sg];
          const int pe = kLds ? seg_pp[sg + 1] : P[L.seg_off + sg + 1];
          ws[2 * w] = make_int4(sg, uq[q] - seg_uo[sg], ad, inf[ad] & kInfRankMask);
          ws[2 * w + 1] = make_int4(psa[ad], pb, pe, 0);
        }
      }
    }
    if (tid == 0) {
      P[L.hdr + kPhUnits] = n_units;
      P[L.hdr + kPhUnitsPerWave] = upw;
      P[L.hdr + kPhBig] = n_big;
      P[L.hdr + kPhSched] = a.no_sched ? 0 : 1;
    }
  }

  // 6. with the arrays in LDS, the segment outputs are stored last: on this
  //    target stores count in the same counter as loads, so earlier stores
  //    would hold up every wait the compiler places for a later load
  if constexpr (kLds) {
    const int ms = (S + nt - 1) / nt;
    const int g0 = min(S, tid * ms), g1 = min(S, g0 + ms);
    for (int sg = g0; sg < g1; ++sg) {
      const int ad = seg_ad[sg];
      const int c = ld_ctr(&cnt[ad]);
      const int r = inf[ad] & kInfRankMask;
      const int st = seg_pp[sg], rb = seg_row[sg], uo = seg_uo[sg];
      const int ub = ubias[ad] + st * r;
      P[L.seg_adapter + sg] = ad;
      P[L.seg_row_off + sg] = rb;
      P[L.seg_uoff + sg] = uo;
      P[L.seg_off + sg] = st;
      int4 *d = reinterpret_cast<int4 *>(P + L.seg_desc) + 2 * sg;
      d[0] = make_int4(ad, r, psa[ad], st);
      d[1] = make_int4(st + c, ub, rb, uo);
    }
    if (tid == 0) {
      P[L.seg_off + S] = pair_base;
      P[L.seg_row_off + S] = row_base;
      P[L.seg_uoff + S] = n_units;
      P[L.u_off + pair_base] = u_base;
      P[L.big_list] = n_big;
    }
    if (wave == 0) {
      const int bt = lane < LORA_N_BUCKETS ? s_btot[lane] : 0;
      const int bi = wave_scan_incl(bt);
      if (lane <= LORA_N_BUCKETS) P[L.bucket_seg_off + lane] = bi - bt;
    }
  }
  if (tid == 0) {
    int32_t *h = P + L.hdr;
    h[LORA_PH_PAIRS] = pair_base;
    h[LORA_PH_SEGS] = S;
    h[LORA_PH_ERR] = s_err;
    h[LORA_PH_RPAIRS] = u_base;
    h[LORA_PH_RUSED] = row_base;
    h[LORA_PH_T] = a.T;
    h[LORA_PH_K] = a.K;
    h[LORA_PH_N] = N;
    for (int q = kPhSched + 1; q < LORA_PLAN_HEADER_INTS; ++q) h[q] = 0;
    for (int q = LORA_N_BUCKETS + 1; q < 16; ++q) P[L.bucket_seg_off + q] = 0;
  }
}

}  // namespace
}  // namespace lora
