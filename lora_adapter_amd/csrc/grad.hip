// LoRA factor gradients, as per-segment outer-product reductions over tokens.
//
// Only A and B train while W stays frozen (LoRAFusion explainer, section
// 解决什么真问题); the pages give no backward formula, so these are the
// derivatives of <dY, Y> for the forward computed by the apply:
//   dB_a[j][n] = sum_{p of a} U[u_off[p]+j] . dY[t_p][n]
//   dA_a[i][j] = sum_{p of a} (X . m)[t_p][i] . G[u_off[p]+j],
//   G[u_off[p]+j] = kappa . g . s_a . (dY[t_p] . B_a[j])
// Both are out_page(a, j)[c] = sum over the segment's pairs of coef[u_off[p]+j]
// . Z[t_p][c].  Pairs are cut into fixed chunks of 256 (in plan order); each
// (chunk, column slice, 16-rank-row block) workgroup accumulates in registers
// and writes one partial per segment it meets, then a second kernel adds a
// segment's partials in chunk order.  No atomics: results are deterministic.
// Prefill-size bf16 batches run the outer products on MFMA with the pairs as
// K (seg_outer_mfma_kernel), and the dB pass also forms the per-tile partials
// of G from the same staged dY rows; other batches use the vector ALU
// (seg_outer_partial_kernel) and the shrink kernel on (dY, B pages) for G.
// Both forms are organised for bandwidth (rows in flight, 16-byte loads).
#include "lora_internal.h"

namespace lora {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef short v4i16_t __attribute__((ext_vector_type(4)));

constexpr int kGradThreads = 256;
constexpr int kGradCPL = 4;                           // columns per lane
constexpr int kGradCols = kGradThreads * kGradCPL;    // columns per workgroup
constexpr int kGradAhead = 8;                         // token rows per batch (two in flight)
static_assert(kGradPairChunk == kGradThreads, "one staged pair per thread");

// 4 consecutive elements held raw until used.
template <typename E> struct Z4;
template <> struct Z4<uint16_t> {
  uint2 w;
  __device__ __forceinline__ void load(const uint16_t *p) { w = *reinterpret_cast<const uint2 *>(p); }
  __device__ __forceinline__ void get(float v[4]) const {
    v[0] = bf_lo(w.x); v[1] = bf_hi(w.x); v[2] = bf_lo(w.y); v[3] = bf_hi(w.y);
  }
};
template <> struct Z4<float> {
  float4 w;
  __device__ __forceinline__ void load(const float *p) { w = *reinterpret_cast<const float4 *>(p); }
  __device__ __forceinline__ void get(float v[4]) const { v[0] = w.x; v[1] = w.y; v[2] = w.z; v[3] = w.w; }
};

__device__ __forceinline__ int seg_of(const int32_t *seg_off, int S, int p) {
  int lo = 0, hi = S;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (seg_off[mid] <= p) lo = mid; else hi = mid;
  }
  return lo;
}

// One workgroup per (column slice of 1024, chunk of 256 pairs, block of 16
// rank rows).  The chunk's token rows and coefficients are staged in LDS by
// one load per thread; each lane then streams its 4 columns of the pairs'
// token rows, kGradAhead rows in flight, and accumulates 16 x 4 sums.
template <typename E, bool kMask>
__global__ __launch_bounds__(kGradThreads) void seg_outer_partial_kernel(SegOuterArgs a) {
  constexpr int RB = kGradRankChunk;
  __shared__ int s_row[kGradPairChunk];
  __shared__ __attribute__((aligned(16))) float s_cf[kGradPairChunk][RB];
  const int P = a.plan.hdr[LORA_PH_PAIRS];
  const int S = a.plan.hdr[LORA_PH_SEGS];
  const int q = blockIdx.y;
  const int pbeg = q * kGradPairChunk;
  if (pbeg >= P) return;
  if (int64_t(a.plan.hdr[LORA_PH_RPAIRS]) > a.coef_cap) {
    if (q == 0 && blockIdx.x == 0 && blockIdx.z == 0 && threadIdx.x == 0)
      atomicOr(a.err_word, LORA_DEVERR_CAPACITY);
    return;
  }
  const int pend = min(P, pbeg + kGradPairChunk);
  const int tid = threadIdx.x;
  const int j0 = blockIdx.z * RB;
  // stage the chunk: token row and coefficients of pair pbeg + tid
  {
    const int pp = pbeg + tid;
    int row = 0;
    float cf[RB];
#pragma unroll
    for (int jj = 0; jj < RB; ++jj) cf[jj] = 0.f;
    if (pp < pend) {
      row = a.plan.pair_tk[pp] / a.K;
      const int r = a.rank[a.plan.pair_adapter[pp]];
      const int nr = min(RB, min(r, a.max_rank) - j0);
      const float *c = a.coef + a.plan.u_off[pp] + j0;
#pragma unroll
      for (int jj = 0; jj < RB; ++jj)
        if (jj < nr) cf[jj] = c[jj];
    }
    s_row[tid] = row;
#pragma unroll
    for (int jj = 0; jj < RB; jj += 4)
      *reinterpret_cast<float4 *>(&s_cf[tid][jj]) = make_float4(cf[jj], cf[jj + 1], cf[jj + 2], cf[jj + 3]);
  }
  __syncthreads();

  const int col_raw = (blockIdx.x * kGradThreads + tid) * kGradCPL;
  const bool col_ok = col_raw < a.d;
  const int col = col_ok ? col_raw : a.d - kGradCPL;     // loads stay in bounds
  const E *Z = static_cast<const E *>(a.Z);
  int s = seg_of(a.plan.seg_off, S, pbeg);
  for (int p = pbeg; p < pend; ++s) {
    const int send = min(pend, a.plan.seg_off[s + 1]);
    const int ad = a.plan.seg_adapter[s];
    const int r = a.rank[ad];
    if (r > a.max_rank) {
      if (tid == 0 && blockIdx.x == 0 && j0 == 0) atomicOr(a.err_word, LORA_DEVERR_CAPACITY);
    } else if (j0 < r) {
      const int nr = min(RB, r - j0);
      float acc[RB][kGradCPL];
#pragma unroll
      for (int jj = 0; jj < RB; ++jj)
#pragma unroll
        for (int c = 0; c < kGradCPL; ++c) acc[jj][c] = 0.f;
      const int l_end = send - pbeg;
      // two batches of kGradAhead token rows, the next one in flight while
      // the current one is added (rows clamped to the segment's last pair; a
      // row past the end, or a masked element, is multiplied by an exact 0)
      Z4<E> za[kGradAhead], zb[kGradAhead];
      uint32_t ma[kGradAhead], mb[kGradAhead];
      auto load_batch = [&](Z4<E> (&z)[kGradAhead], uint32_t (&m)[kGradAhead], int l0) {
#pragma unroll
        for (int u = 0; u < kGradAhead; ++u) {
          const int64_t row = s_row[min(l0 + u, l_end - 1)];
          z[u].load(Z + row * a.d + col);
          if (kMask) m[u] = *reinterpret_cast<const uint32_t *>(a.mask + row * a.d + col);
        }
      };
      auto add_batch = [&](const Z4<E> (&z)[kGradAhead], const uint32_t (&m)[kGradAhead], int l0) {
#pragma unroll
        for (int u = 0; u < kGradAhead; ++u) {
          float zv[kGradCPL];
          z[u].get(zv);
          const float in = l0 + u < l_end ? 1.f : 0.f;
#pragma unroll
          for (int c = 0; c < kGradCPL; ++c) {
            float f = in;
            if (kMask) f *= float((m[u] >> (8 * c)) & 0xffu);   // keep mask is 0/1
            zv[c] *= f;
          }
          const float *cf = s_cf[min(l0 + u, l_end - 1)];
#pragma unroll
          for (int jj = 0; jj < RB; ++jj) {
            const float cj = cf[jj];   // zero past nr
#pragma unroll
            for (int c = 0; c < kGradCPL; ++c) acc[jj][c] = fmaf(cj, zv[c], acc[jj][c]);
          }
        }
      };
      load_batch(za, ma, p - pbeg);
      for (int l0 = p - pbeg; l0 < l_end; l0 += 2 * kGradAhead) {
        load_batch(zb, mb, l0 + kGradAhead);
        add_batch(za, ma, l0);
        if (l0 + kGradAhead >= l_end) break;
        load_batch(za, ma, l0 + 2 * kGradAhead);
        add_batch(zb, mb, l0 + kGradAhead);
      }
      if (col_ok) {
        float *dst = a.part + (int64_t(s + q) * a.max_rank + j0) * a.d + col;
#pragma unroll
        for (int jj = 0; jj < RB; ++jj)
          if (jj < nr)
            *reinterpret_cast<float4 *>(dst + int64_t(jj) * a.d) =
                make_float4(acc[jj][0], acc[jj][1], acc[jj][2], acc[jj][3]);
      }
    }
    p = send;
  }
}

// The same partials with bf16 MFMA (prefill-size batches): out[j][n] =
// sum_p cf[p][j] . Z[t_p][n] is a (16 rank rows) x (columns) product over the
// pairs, v_mfma_f32_16x16x32_bf16 with the pairs as K.  One workgroup per
// (256 columns, chunk of 256 pairs, 16 rank rows); per step of 32 pairs the
// gathered token rows (keep mask applied: exact zeros) are staged in LDS, the
// next step's rows in flight meanwhile.  The fp32 coefficients are split
// exactly into bf16 high and low parts (two MFMAs), which keeps ~16 bits.
// Workgroup barrier for LDS only: the next step's token-row loads and the
// partial stores stay in flight across it (__syncthreads() would wait for
// every outstanding load and store).
__device__ __forceinline__ void lds_bar() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

constexpr int kOuterCols = 256;
constexpr int kOuterK = 32;

// Segment index of pair p, found by the whole workgroup: each round tests
// 256 evenly spaced segment starts, one load per thread, so S <= 256 takes
// one round trip and S <= 65536 two (a binary search took log2 S dependent
// ones).  seg_off[0] = 0 <= p < seg_off[S] holds throughout.
__device__ __forceinline__ int seg_of_wg(const int32_t *seg_off, int S, int p, int *s_cnt) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int lo = 0, hi = S;
  while (hi - lo > 1) {
    const int step = (hi - lo + 255) / 256;
    const int i = lo + tid * step;
    const uint64_t b = __ballot(i < hi && seg_off[i] <= p);
    if (lane == 0) s_cnt[wave] = __popcll(b);
    lds_bar();
    const int c = s_cnt[0] + s_cnt[1] + s_cnt[2] + s_cnt[3];   // >= 1: i = lo passes
    lds_bar();                                                  // s_cnt reused next round
    lo += (c - 1) * step;
    hi = min(hi, lo + step);
  }
  return lo;
}

// First pair after l that starts a segment (bit set in the chunk's start
// mask), or n.
__device__ __forceinline__ int next_start(const uint64_t *bits, int l, int n) {
  for (int w = (l + 1) >> 6; w < 4; ++w) {
    uint64_t b = bits[w];
    const int lo = (l + 1) - 64 * w;
    if (lo > 0) b &= ~0ull << lo;
    if (b) return min(n, 64 * w + __builtin_ctzll(b));
  }
  return n;
}

template <bool kMask, bool kG>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(kMask ? 2 : 3)))
void seg_outer_mfma_kernel(SegOuterArgs a) {
  constexpr int RB = kGradRankChunk;
  // staged row pitch (bf16; 4 banks): the 16 rows of a 16-byte G operand
  // read fall on distinct banks
  constexpr int ZP = kOuterCols + 8;
  __shared__ int s_row[kGradPairChunk];
  __shared__ int s_ad[kGradPairChunk];
  __shared__ int s_rk[kGradPairChunk];
  // the coefficients split once into bf16 high and low parts, rank row
  // major, so that a lane's A operand (8 consecutive pairs of one rank row)
  // is one 16-byte read; the row pitch puts the 16 rank rows of a read on
  // distinct banks
  constexpr int AP = kGradPairChunk + 8;
  __shared__ __attribute__((aligned(16))) uint16_t s_ah[RB][AP];
  __shared__ __attribute__((aligned(16))) uint16_t s_al[RB][AP];
  __shared__ __attribute__((aligned(16))) uint16_t s_z[kOuterK][ZP];
  __shared__ uint64_t s_start[4];          // segment starts of the chunk, one bit per pair
  __shared__ int s_cnt[4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int q = blockIdx.y;
  const int pbeg = q * kGradPairChunk;
  const int64_t TK = int64_t(a.T) * a.K;
  // The prologue keeps its dependent round trips few and overlapped: the
  // header and this thread's pair in one; then the pair's rank, the first
  // segment's B page entry, the first step's token rows and the segment
  // search together; then the coefficients and the B page ids; then the B
  // rows.  Plan entries past the pair count are read (in bounds) but unused.
  const int P = a.plan.hdr[LORA_PH_PAIRS];
  const int S = a.plan.hdr[LORA_PH_SEGS];
  const int64_t rpairs = a.plan.hdr[LORA_PH_RPAIRS];
  const int pp = pbeg + tid;
  const bool inb = pp < TK;
  const int tk = inb ? a.plan.pair_tk[pp] : 0;
  const int adp = inb ? a.plan.pair_adapter[pp] : 0;
  const int uo = inb ? a.plan.u_off[pp] : 0;
  if (pbeg >= P) return;
  if (rpairs > a.coef_cap) {
    if (q == 0 && blockIdx.x == 0 && blockIdx.z == 0 && tid == 0)
      atomicOr(a.err_word, LORA_DEVERR_CAPACITY);
    return;
  }
  const int n = min(P, pbeg + kGradPairChunk) - pbeg;
  const bool valid = tid < n;
  const int j0 = blockIdx.z * RB;
  const int rk = valid ? a.rank[adp] : 0;
  s_row[tid] = valid ? tk / a.K : 0;
  s_ad[tid] = valid ? adp : -1;
  lds_bar();
  {
    const uint64_t b = __ballot(valid && (tid == 0 || s_ad[tid - 1] != adp));
    if (lane == 0) s_start[wave] = b;
  }
  lds_bar();

  const int c0 = blockIdx.x * kOuterCols;
  const uint16_t *Z = static_cast<const uint16_t *>(a.Z);
  // staging: thread tid fills row tid / 8 of the step, columns (tid % 8) * 32 .. +31
  const int zr = tid >> 3, zc = (tid & 7) * 32;
  // two steps of token rows in flight: buffer A holds a segment's even
  // steps, buffer B its odd ones.  Every fetch is issued unconditionally
  // (past the segment's end it re-reads its last row, a cache hit, and the
  // staging zeroes it): a conditional fetch leaves the compiler a merge of
  // old and new register values, which it resolves with copies that wait
  // for the loads just issued, and the prefetch is lost.
  uint4 zA[4], zB[4];
  uint4 mA[2], mB[2];
  auto fetch = [&](uint4 (&zv)[4], uint4 (&mv)[2], int k0, int l_beg, int l_end) {
    const int64_t row = s_row[min(max(k0 + zr, l_beg), l_end - 1)];
    const uint16_t *src = Z + row * a.d + c0 + zc;
#pragma unroll
    for (int e = 0; e < 4; ++e) zv[e] = *reinterpret_cast<const uint4 *>(src + 8 * e);
    if (kMask) {
      const uint8_t *m = a.mask + row * a.d + c0 + zc;
      mv[0] = *reinterpret_cast<const uint4 *>(m);
      mv[1] = *reinterpret_cast<const uint4 *>(m + 16);
    }
  };
  auto stage = [&](const uint4 (&zv)[4], const uint4 (&mv)[2], int k0, int l_beg, int l_end) {
    uint32_t w[16];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      w[4 * e] = zv[e].x; w[4 * e + 1] = zv[e].y; w[4 * e + 2] = zv[e].z; w[4 * e + 3] = zv[e].w;
    }
    // rows outside the segment (a step that crosses one of its ends) are
    // zeroed; the test is uniform over the workgroup
    if (k0 < l_beg || k0 + kOuterK > l_end) {
      const bool in = k0 + zr >= l_beg && k0 + zr < l_end;
#pragma unroll
      for (int i = 0; i < 16; ++i) w[i] = in ? w[i] : 0u;
    }
    if constexpr (kMask) {
      // keep-mask bytes are 0 or 1: the bytes of elements 2i and 2i + 1 go
      // to bits 0 and 16 of x (one byte permute), and x . 0xffff (as
      // (x << 16) - x) is the 16-bit lane mask of the pair
      const uint32_t mb[8] = {mv[0].x, mv[0].y, mv[0].z, mv[0].w, mv[1].x, mv[1].y, mv[1].z, mv[1].w};
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const uint32_t x = __builtin_amdgcn_perm(0u, mb[i >> 1], (i & 1) ? 0x0c030c02u : 0x0c010c00u);
        w[i] &= (x << 16) - x;
      }
    }
    // rows are 8-byte aligned (pitch ZP): memcpy lets the compiler pick
    // the widest aligned LDS stores
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint4 v4 = make_uint4(w[4 * e], w[4 * e + 1], w[4 * e + 2], w[4 * e + 3]);
      __builtin_memcpy(&s_z[zr][zc + 8 * e], &v4, 16);
    }
  };
  // dY.B^T partials (dB pass): the segment's 16 B rows over this column
  // tile, staged in LDS (row pitch GP: the 16 rows of one 16-byte column
  // chunk, read by 16 lanes at once, fall on distinct banks).  Thread tid
  // moves column chunk tid % 32 of rows tid / 32 and tid / 32 + 8.
  constexpr int GP = kOuterCols + 8;
  __shared__ __attribute__((aligned(16))) uint16_t s_gb[kG ? RB : 1][kG ? GP : 8];
  const int jr = lane & 15;
  const int gj = tid >> 5, gc = (tid & 31) * 8;
  int gpid[2] = {0, 0};
  uint4 gv[2];
  auto g_ids = [&](int ps, int nr) {
    if constexpr (kG) {
#pragma unroll
      for (int h = 0; h < 2; ++h)
        if (gj + 8 * h < nr) gpid[h] = a.page_ids[ps + j0 + gj + 8 * h];
    }
  };
  auto g_rows = [&](int nr) {
    if constexpr (kG) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        gv[h] = make_uint4(0u, 0u, 0u, 0u);
        if (gj + 8 * h < nr)
          gv[h] = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(a.b_pages) +
                                                   int64_t(gpid[h]) * a.d + c0 + gc);
      }
    }
  };
  auto g_put = [&]() {
    if constexpr (kG) {
#pragma unroll
      for (int h = 0; h < 2; ++h) __builtin_memcpy(&s_gb[gj + 8 * h][gc], &gv[h], 16);
    }
  };

  // first segment: its adapter's page entry and rank (dB pass) and its
  // first two steps' token rows; then its B page ids and this thread's
  // coefficients; then the search for its index (uniform over the
  // workgroup) and its B rows
  const int ad0 = s_ad[0];
  const int l_end0 = next_start(s_start, 0, n);
  int ps0 = 0, r0 = 0;
  if constexpr (kG) {
    ps0 = a.page_start[ad0];
    r0 = a.rank[ad0];
  }
  fetch(zA, mA, 0, 0, l_end0);
  fetch(zB, mB, kOuterK, 0, l_end0);
  const int nr0 = min(RB, r0 - j0);
  const bool g0 = kG && r0 <= a.max_rank && nr0 > 0;
  if (g0) g_ids(ps0, nr0);
  {
    // the coefficients of this thread's pair (zero past its rank)
    float cf[RB];
#pragma unroll
    for (int jj = 0; jj < RB; ++jj) cf[jj] = 0.f;
    const int nr = min(RB, min(rk, a.max_rank) - j0);
    const float *c = a.coef + uo + j0;
#pragma unroll
    for (int jj = 0; jj < RB; ++jj)
      if (valid && jj < nr) cf[jj] = c[jj];
    s_rk[tid] = rk;
#pragma unroll
    for (int jj = 0; jj < RB; ++jj) {
      const uint16_t h = f2bf(cf[jj]);
      s_ah[jj][tid] = h;
      s_al[jj][tid] = f2bf(cf[jj] - bf2f(h));
    }
  }
  int s = seg_of_wg(a.plan.seg_off, S, pbeg, s_cnt);
  if (g0) {
    g_rows(nr0);
    g_put();
  }
  lds_bar();                                             // s_rk, s_ah, s_al, s_gb

  for (int l_beg = 0; l_beg < n; ++s) {
    const int l_end = l_beg == 0 ? l_end0 : next_start(s_start, l_beg, n);
    const int ad = s_ad[l_beg];
    const int r = s_rk[l_beg];
    if (r > a.max_rank) {
      if (tid == 0 && blockIdx.x == 0 && j0 == 0) atomicOr(a.err_word, LORA_DEVERR_CAPACITY);
    } else if (j0 < r) {
      const int nr = min(RB, r - j0);
      if (l_beg > 0) {
        const int k1 = l_beg & ~(kOuterK - 1);
        fetch(zA, mA, k1, l_beg, l_end);
        fetch(zB, mB, k1 + kOuterK, l_beg, l_end);
        if constexpr (kG) {
          g_ids(a.page_start[ad], nr);
          g_rows(nr);
          lds_bar();                           // the last segment's G steps are done with s_gb
          g_put();                             // published by the first step's barrier
        }
      }
      f32x4_t acc[4];
#pragma unroll
      for (int b = 0; b < 4; ++b) acc[b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      // one step of 32 pairs from buffer (zv, mv), which then takes the
      // rows two steps ahead.  Steps start at multiples of 32 pairs of the
      // chunk (aligned A operand reads); rows outside the segment are staged
      // as exact zeros, so a step that is partly or wholly outside it adds
      // exact zeros and stores no G partial there.  The fetch goes out after
      // the step's G partial stores: those may or may not issue, so the
      // compiler counts none of them, and a fetch issued before them would
      // be waited for at the next step's staging.
      auto step = [&](uint4 (&zv)[4], uint4 (&mv)[2], int k0) {
        // nothing of this step is scheduled above the previous step's fetch
        // (its staging would wait for this buffer's loads before that fetch
        // goes out)
        __builtin_amdgcn_sched_barrier(0);
        lds_bar();                             // the previous step is done with s_z
        stage(zv, mv, k0, l_beg, l_end);
        lds_bar();
        // A operand: rank row j = lane % 16, pairs k0 + 8 * (lane / 16) .. + 7
        // (pairs of other segments meet zeroed rows; past the chunk's end
        // the coefficients are zero)
        // (a step wholly past the chunk's end reads the last step's)
        const int kk = (lane >> 4) * 8;
        const int ka = min(k0, kGradPairChunk - kOuterK) + kk;
        bf16x8_t ahi, alo;
        __builtin_memcpy(&ahi, &s_ah[lane & 15][ka], 16);
        __builtin_memcpy(&alo, &s_al[lane & 15][ka], 16);
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          // B operand: column wave*64 + 16b + lane % 16, the same 8 pairs,
          // by two transposing reads: in each group of 16 lanes, lane L
          // gives the address of row (L / 4) of a 4-row block, columns
          // 4 (L % 4) .. + 3, and receives column L of the 4 rows
          const int cb = wave * 64 + 16 * b + 4 * (lane & 3);
          const int rb = kk + ((lane & 15) >> 2);
          const v4i16_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) v4i16_t *)(&s_z[rb][cb]));
          const v4i16_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) v4i16_t *)(&s_z[rb + 4][cb]));
          bf16x8_t bfrag;
          __builtin_memcpy(&bfrag, &lo, 8);
          __builtin_memcpy(reinterpret_cast<char *>(&bfrag) + 8, &hi, 8);
          acc[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ahi, bfrag, acc[b], 0, 0, 0);
          acc[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(alo, bfrag, acc[b], 0, 0, 0);
        }
        if constexpr (kG) {
          if (wave < 2) {
            // waves 0 and 1: pairs k0 + 16 * wave .. + 15 of the step (rows
            // of s_z) times the B rows, over the tile's 256 columns in 8 K steps
            f32x4_t ga = {0.f, 0.f, 0.f, 0.f};
            const int zrow = 16 * wave + (lane & 15);
#pragma unroll
            for (int ks = 0; ks < 8; ++ks) {
              bf16x8_t fa, fb;
              __builtin_memcpy(&fa, &s_z[zrow][32 * ks + 8 * (lane >> 4)], 16);
              __builtin_memcpy(&fb, &s_gb[jr][32 * ks + 8 * (lane >> 4)], 16);
              ga = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa, fb, ga, 0, 0, 0);
            }
            // lane holds rank column (lane % 16) and pair rows 4 * (lane / 16) + i
            if (jr < nr) {
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                const int l = k0 + 16 * wave + (lane >> 4) * 4 + i;
                if (l >= l_beg && l < l_end)
                  a.gpart[(int64_t(blockIdx.x) * TK + pbeg + l) * a.max_rank + j0 + jr] = ga[i];
              }
            }
          }
        }
        fetch(zv, mv, k0 + 2 * kOuterK, l_beg, l_end);
      };
      for (int k0 = l_beg & ~(kOuterK - 1); k0 < l_end; k0 += 2 * kOuterK) {
        step(zA, mA, k0);
        step(zB, mB, k0 + kOuterK);
      }
      // lane holds column (lane % 16) of each block and rank rows 4 * (lane / 16) + i
      float *dst = a.part + (int64_t(s + q) * a.max_rank + j0) * a.d + c0 + wave * 64 + (lane & 15);
#pragma unroll
      for (int b = 0; b < 4; ++b)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int jj = (lane >> 4) * 4 + i;
          if (jj < nr) dst[int64_t(jj) * a.d + 16 * b] = acc[b][i];
        }
    }
    l_beg = l_end;
  }
}

// Adds each segment's partials in chunk order (up to 8 loads in flight) and
// writes the fp32 gradient page of every rank row: one workgroup per (1024
// columns, segment, rank row); workgroup (bx, by, bz) of a (., gy, .) grid.
__device__ __forceinline__ void seg_outer_reduce_wg(const SegOuterArgs &a, int bx, int by, int bz, int gy) {
  const int S = a.plan.hdr[LORA_PH_SEGS];
  const int col = (bx * kGradThreads + threadIdx.x) * kGradCPL;
  if (col >= a.d) return;
  if (int64_t(a.plan.hdr[LORA_PH_RPAIRS]) > a.coef_cap) return;
  const int j = bz;
  for (int s = by; s < S; s += gy) {
    const int ad = a.plan.seg_adapter[s];
    const int r = a.rank[ad];
    if (r > a.max_rank || j >= r) continue;
    const int q0 = a.plan.seg_off[s] / kGradPairChunk;
    const int q1 = (a.plan.seg_off[s + 1] - 1) / kGradPairChunk;
    float4 sum = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int qb = q0; qb <= q1; qb += 8) {
      float4 v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u)
        v[u] = *reinterpret_cast<const float4 *>(
            a.part + (int64_t(s + min(qb + u, q1)) * a.max_rank + j) * a.d + col);
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        if (qb + u <= q1) {
          sum.x += v[u].x; sum.y += v[u].y; sum.z += v[u].z; sum.w += v[u].w;
        }
      }
    }
    *reinterpret_cast<float4 *>(a.out_pages + int64_t(a.page_ids[a.page_start[ad] + j]) * a.d + col) = sum;
  }
}

__global__ __launch_bounds__(kGradThreads) void seg_outer_reduce_kernel(SegOuterArgs a) {
  seg_outer_reduce_wg(a, blockIdx.x, blockIdx.y, blockIdx.z, gridDim.y);
}

// G[u_off[p] + j] = (gate . scale . extra) . sum over tiles of gpart, one
// thread per (pair, rank row), tiles added in order; workgroup b.
__device__ __forceinline__ void g_reduce_wg(const GReduceArgs &a, int64_t b) {
  const int64_t idx = b * 256 + threadIdx.x;
  const int P = a.plan.hdr[LORA_PH_PAIRS];
  const int64_t p = idx / a.max_rank;
  const int j = int(idx % a.max_rank);
  if (p >= P) return;
  if (int64_t(a.plan.hdr[LORA_PH_RPAIRS]) > a.g_cap) return;
  const int adp = a.plan.pair_adapter[p];
  const int r = a.rank[adp];
  if (j >= r || r > a.max_rank) return;
  // tiles in order, 8 loads in flight
  float sum = 0.f;
  const int64_t stride = a.TK * a.max_rank;
  const float *src = a.gpart + p * a.max_rank + j;
  for (int x0 = 0; x0 < a.n_tiles; x0 += 8) {
    float v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = src[int64_t(min(x0 + u, a.n_tiles - 1)) * stride];
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (x0 + u < a.n_tiles) sum += v[u];
  }
  const float sc = a.scale[adp] * a.extra_scale;
  a.G[a.plan.u_off[p] + j] = a.plan.pair_gate[p] * sc * sum;
}

// The dB pass's two reductions in one launch (they read different partials
// and write different outputs): workgroups 0 .. n_seg - 1 add the dB chunk
// partials ((cols, gy, rank rows) flattened, cols fastest), the rest form G.
static_assert(kGradThreads == 256, "both reductions run 256-thread workgroups");
__global__ __launch_bounds__(256) void seg_g_reduce_kernel(SegOuterArgs a, GReduceArgs g, int cols,
                                                           int gy, int64_t n_seg) {
  const int64_t b = blockIdx.x;
  if (b < n_seg) {
    seg_outer_reduce_wg(a, int(b % cols), int((b / cols) % gy), int(b / (int64_t(cols) * gy)), gy);
  } else {
    g_reduce_wg(g, b - n_seg);
  }
}

}  // namespace

bool grad_mfma_form(int dtype, int64_t TK, int d_out) {
  return dtype == LORA_BF16 && TK >= 2048 && d_out % kOuterCols == 0;
}

int grad_gpart_tiles(int d_out) { return d_out / kOuterCols; }

int64_t grad_pieces(int64_t TK, int64_t N) {
  const int64_t segs = TK < N ? TK : N;
  return segs + (TK + kGradPairChunk - 1) / kGradPairChunk + 1;
}

hipError_t launch_seg_outer(const SegOuterArgs &a, int dtype, int64_t TK, int64_t N, hipStream_t st,
                            const GReduceArgs *g) {
  if (TK == 0) return hipSuccess;
  const unsigned cols = unsigned((a.d + kGradCols - 1) / kGradCols);
  const unsigned chunks = unsigned((TK + kGradPairChunk - 1) / kGradPairChunk);
  const unsigned rchunks = unsigned((a.max_rank + kGradRankChunk - 1) / kGradRankChunk);
  const dim3 g1(cols, chunks, rchunks), block(kGradThreads);
  if (grad_mfma_form(dtype, TK, a.d)) {
    // prefill-size batches: the MFMA form (long segments make it dense)
    const dim3 gm(unsigned(a.d / kOuterCols), chunks, rchunks);
    if (a.mask) hipLaunchKernelGGL((seg_outer_mfma_kernel<true, false>), gm, block, 0, st, a);
    else if (a.gpart) hipLaunchKernelGGL((seg_outer_mfma_kernel<false, true>), gm, block, 0, st, a);
    else hipLaunchKernelGGL((seg_outer_mfma_kernel<false, false>), gm, block, 0, st, a);
  } else if (dtype == LORA_BF16) {
    if (a.mask) hipLaunchKernelGGL((seg_outer_partial_kernel<uint16_t, true>), g1, block, 0, st, a);
    else hipLaunchKernelGGL((seg_outer_partial_kernel<uint16_t, false>), g1, block, 0, st, a);
  } else {
    if (a.mask) hipLaunchKernelGGL((seg_outer_partial_kernel<float, true>), g1, block, 0, st, a);
    else hipLaunchKernelGGL((seg_outer_partial_kernel<float, false>), g1, block, 0, st, a);
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const int64_t segs = TK < N ? TK : N;
  const unsigned gy = unsigned(segs < 65535 ? segs : 65535);
  if (g != nullptr) {
    const int64_t n_seg = int64_t(cols) * gy * a.max_rank;
    const int64_t n_g = (g->TK * g->max_rank + 255) / 256;
    hipLaunchKernelGGL(seg_g_reduce_kernel, dim3(unsigned(n_seg + n_g)), block, 0, st, a, *g,
                       int(cols), int(gy), n_seg);
    return hipGetLastError();
  }
  const dim3 g2(cols, gy, unsigned(a.max_rank));
  hipLaunchKernelGGL(seg_outer_reduce_kernel, g2, block, 0, st, a);
  return hipGetLastError();
}

}  // namespace lora
