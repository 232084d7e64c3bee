// LoRA factor gradients, as per-segment outer-product reductions over tokens.
//
// Only A and B train while W stays frozen (LoRAFusion explainer, section
// 解决什么真问题); the pages give no backward formula, so these are the
// derivatives of <dY, Y> for the forward computed by the apply:
//   dB_a[j][n] = sum_{p of a} U[u_off[p]+j] . dY[t_p][n]
//   dA_a[i][j] = sum_{p of a} (X . m)[t_p][i] . G[u_off[p]+j],
//   G[u_off[p]+j] = kappa . g . s_a . (dY[t_p] . B_a[j])   (the shrink kernel on dY, B)
// Both are out_page(a, j)[c] = sum over the segment's pairs of coef[u_off[p]+j]
// . Z[t_p][c].  Pairs are cut into fixed chunks of 256 (in plan order); each
// (chunk, column slice, 16-rank-row block) workgroup accumulates in registers
// and writes one partial per segment it meets, then a second kernel adds a
// segment's partials in chunk order.  No atomics: results are deterministic.
// The work per (pair, column, rank row) is one fma, so it stays on the vector
// ALU; the kernels are organised for bandwidth (rows in flight, 16-byte loads).
#include "lora_internal.h"

namespace lora {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

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

template <bool kMask>
__global__ __launch_bounds__(256) void seg_outer_mfma_kernel(SegOuterArgs a) {
  constexpr int RB = kGradRankChunk;
  // staged row pitch (bf16): rows 8 apart (the four lane groups of a
  // transposed 16-bit read) then start 16 banks apart
  constexpr int ZP = kOuterCols + 4;
  __shared__ int s_row[kGradPairChunk];
  __shared__ __attribute__((aligned(16))) float s_cf[kGradPairChunk][RB];
  __shared__ __attribute__((aligned(16))) uint16_t s_z[kOuterK][ZP];
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
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int j0 = blockIdx.z * RB;
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

  const int c0 = blockIdx.x * kOuterCols;
  const uint16_t *Z = static_cast<const uint16_t *>(a.Z);
  // staging: thread tid fills row tid / 8 of the step, columns (tid % 8) * 32 .. +31
  const int zr = tid >> 3, zc = (tid & 7) * 32;
  int s = seg_of(a.plan.seg_off, S, pbeg);
  for (int p = pbeg; p < pend; ++s) {
    const int send = min(pend, a.plan.seg_off[s + 1]);
    const int ad = a.plan.seg_adapter[s];
    const int r = a.rank[ad];
    if (r > a.max_rank) {
      if (tid == 0 && blockIdx.x == 0 && j0 == 0) atomicOr(a.err_word, LORA_DEVERR_CAPACITY);
    } else if (j0 < r) {
      const int nr = min(RB, r - j0);
      const int l_beg = p - pbeg, l_end = send - pbeg;
      uint4 zv[4];
      uint4 mv[2];
      auto fetch = [&](int k0) {
        const int64_t row = s_row[min(k0 + zr, l_end - 1)];
        const uint16_t *src = Z + row * a.d + c0 + zc;
#pragma unroll
        for (int e = 0; e < 4; ++e) zv[e] = *reinterpret_cast<const uint4 *>(src + 8 * e);
        if (kMask) {
          const uint8_t *m = a.mask + row * a.d + c0 + zc;
          mv[0] = *reinterpret_cast<const uint4 *>(m);
          mv[1] = *reinterpret_cast<const uint4 *>(m + 16);
        }
      };
      auto stage = [&](int k0) {
        const bool in = k0 + zr < l_end;
        uint32_t w[16];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          w[4 * e] = zv[e].x; w[4 * e + 1] = zv[e].y; w[4 * e + 2] = zv[e].z; w[4 * e + 3] = zv[e].w;
        }
        const uint32_t mb[8] = {mv[0].x, mv[0].y, mv[0].z, mv[0].w, mv[1].x, mv[1].y, mv[1].z, mv[1].w};
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          uint32_t keep = in ? 0xffffffffu : 0u;
          if (kMask) {
            // element 2i is byte (2i) of the mask, element 2i+1 byte (2i+1)
            const uint32_t m4 = mb[i >> 1] >> (16 * (i & 1));
            keep &= ((m4 & 0xffu) ? 0x0000ffffu : 0u) | ((m4 & 0xff00u) ? 0xffff0000u : 0u);
          }
          w[i] &= keep;
        }
        // rows are 8-byte aligned (pitch ZP): memcpy lets the compiler pick
        // the widest aligned LDS stores
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint4 v4 = make_uint4(w[4 * e], w[4 * e + 1], w[4 * e + 2], w[4 * e + 3]);
          __builtin_memcpy(&s_z[zr][zc + 8 * e], &v4, 16);
        }
      };
      f32x4_t acc[4];
#pragma unroll
      for (int b = 0; b < 4; ++b) acc[b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      // dY.B^T partials (dB pass): B operand = rank row j0 + lane % 16 of the
      // segment's adapter, 8 columns at 32 ks + 8 (lane / 16) of this tile
      uint4 gb[8];
      const bool with_g = a.gpart != nullptr;
      if (with_g) {
        const int jr = lane & 15;
        const uint16_t *Bp = static_cast<const uint16_t *>(a.b_pages);
        const uint16_t *brow =
            Bp + int64_t(a.page_ids[a.page_start[ad] + j0 + min(jr, nr - 1)]) * a.d + c0 + 8 * (lane >> 4);
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
          gb[ks] = *reinterpret_cast<const uint4 *>(brow + 32 * ks);
          if (jr >= nr) gb[ks] = make_uint4(0u, 0u, 0u, 0u);
        }
      }
      fetch(l_beg);
      for (int k0 = l_beg; k0 < l_end; k0 += kOuterK) {
        lds_bar();                             // the previous step is done with s_z
        stage(k0);
        lds_bar();
        if (k0 + kOuterK < l_end) fetch(k0 + kOuterK);
        // A operand: rank row j = lane % 16, pairs k0 + 8 * (lane / 16) + e
        const int kk = (lane >> 4) * 8;
        uint32_t hw[4], lw[4];
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          const int la = k0 + kk + e, lb = la + 1;
          const float ua = la < l_end ? s_cf[la][lane & 15] : 0.f;
          const float ub = lb < l_end ? s_cf[lb][lane & 15] : 0.f;
          const uint16_t ha = f2bf(ua), hb = f2bf(ub);
          const uint16_t xa = f2bf(ua - bf2f(ha)), xb = f2bf(ub - bf2f(hb));
          hw[e >> 1] = uint32_t(ha) | (uint32_t(hb) << 16);
          lw[e >> 1] = uint32_t(xa) | (uint32_t(xb) << 16);
        }
        bf16x8_t ahi, alo;
        const uint4 ph = make_uint4(hw[0], hw[1], hw[2], hw[3]);
        const uint4 pl = make_uint4(lw[0], lw[1], lw[2], lw[3]);
        __builtin_memcpy(&ahi, &ph, 16);
        __builtin_memcpy(&alo, &pl, 16);
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          // B operand: column wave*64 + 16b + lane % 16, the same 8 pairs
          const int col = wave * 64 + 16 * b + (lane & 15);
          uint32_t bw[4];
#pragma unroll
          for (int e = 0; e < 8; e += 2)
            bw[e >> 1] = uint32_t(s_z[kk + e][col]) | (uint32_t(s_z[kk + e + 1][col]) << 16);
          bf16x8_t bfrag;
          const uint4 pb = make_uint4(bw[0], bw[1], bw[2], bw[3]);
          __builtin_memcpy(&bfrag, &pb, 16);
          acc[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ahi, bfrag, acc[b], 0, 0, 0);
          acc[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(alo, bfrag, acc[b], 0, 0, 0);
        }
        if (with_g && wave < 2) {
          // waves 0 and 1: pairs k0 + 16 * wave .. + 15 of the step (rows of
          // s_z) times the B rows, over the tile's 256 columns in 8 K steps
          f32x4_t ga = {0.f, 0.f, 0.f, 0.f};
          const int zrow = 16 * wave + (lane & 15);
#pragma unroll
          for (int ks = 0; ks < 8; ++ks) {
            bf16x8_t fa, fb;
            __builtin_memcpy(&fa, &s_z[zrow][32 * ks + 8 * (lane >> 4)], 16);
            __builtin_memcpy(&fb, &gb[ks], 16);
            ga = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa, fb, ga, 0, 0, 0);
          }
          // lane holds rank column (lane % 16) and pair rows 4 * (lane / 16) + i
          const int jj = lane & 15;
          if (jj < nr) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int l = k0 + 16 * wave + (lane >> 4) * 4 + i;
              if (l < l_end)
                a.gpart[(int64_t(blockIdx.x) * a.T * a.K + pbeg + l) * a.max_rank + j0 + jj] = ga[i];
            }
          }
        }
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
    p = send;
  }
}

// Adds each segment's partials in chunk order (up to 8 loads in flight) and
// writes the fp32 gradient page of every rank row: one workgroup per (1024
// columns, segment, rank row).
__global__ __launch_bounds__(kGradThreads) void seg_outer_reduce_kernel(SegOuterArgs a) {
  const int S = a.plan.hdr[LORA_PH_SEGS];
  const int col = (blockIdx.x * kGradThreads + threadIdx.x) * kGradCPL;
  if (col >= a.d) return;
  if (int64_t(a.plan.hdr[LORA_PH_RPAIRS]) > a.coef_cap) return;
  const int j = blockIdx.z;
  for (int s = blockIdx.y; s < S; s += gridDim.y) {
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

// G[u_off[p] + j] = (gate . scale . extra) . sum over tiles of gpart, one
// thread per (pair, rank row), tiles added in order.
__global__ __launch_bounds__(256) void g_reduce_kernel(GReduceArgs a) {
  const int64_t idx = int64_t(blockIdx.x) * 256 + threadIdx.x;
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

}  // namespace

bool grad_mfma_form(int dtype, int64_t TK, int d_out) {
  return dtype == LORA_BF16 && TK >= 2048 && d_out % kOuterCols == 0;
}

int grad_gpart_tiles(int d_out) { return d_out / kOuterCols; }

hipError_t launch_g_reduce(const GReduceArgs &a, hipStream_t st) {
  const int64_t n = a.TK * a.max_rank;
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(g_reduce_kernel, dim3(unsigned((n + 255) / 256)), dim3(256), 0, st, a);
  return hipGetLastError();
}

int64_t grad_pieces(int64_t TK, int64_t N) {
  const int64_t segs = TK < N ? TK : N;
  return segs + (TK + kGradPairChunk - 1) / kGradPairChunk + 1;
}

hipError_t launch_seg_outer(const SegOuterArgs &a, int dtype, int64_t TK, int64_t N, hipStream_t st) {
  if (TK == 0) return hipSuccess;
  const unsigned cols = unsigned((a.d + kGradCols - 1) / kGradCols);
  const unsigned chunks = unsigned((TK + kGradPairChunk - 1) / kGradPairChunk);
  const unsigned rchunks = unsigned((a.max_rank + kGradRankChunk - 1) / kGradRankChunk);
  const dim3 g1(cols, chunks, rchunks), block(kGradThreads);
  if (grad_mfma_form(dtype, TK, a.d)) {
    // prefill-size batches: the MFMA form (long segments make it dense)
    const dim3 gm(unsigned(a.d / kOuterCols), chunks, rchunks);
    if (a.mask) hipLaunchKernelGGL((seg_outer_mfma_kernel<true>), gm, block, 0, st, a);
    else hipLaunchKernelGGL((seg_outer_mfma_kernel<false>), gm, block, 0, st, a);
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
  const dim3 g2(cols, unsigned(segs < 65535 ? segs : 65535), unsigned(a.max_rank));
  hipLaunchKernelGGL(seg_outer_reduce_kernel, g2, block, 0, st, a);
  return hipGetLastError();
}

}  // namespace lora
