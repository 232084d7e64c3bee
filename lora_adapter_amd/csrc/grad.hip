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

constexpr int kGradThreads = 256;
constexpr int kGradCPL = 4;                           // columns per lane
constexpr int kGradCols = kGradThreads * kGradCPL;    // columns per workgroup
constexpr int kGradAhead = 8;                         // token rows in flight per lane
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
      for (int l0 = p - pbeg; l0 < l_end; l0 += kGradAhead) {
        // every row of the group is loaded before any is used (clamped to
        // the last pair, so no load sits behind a branch)
        Z4<E> z[kGradAhead];
        uint32_t mk[kGradAhead];
#pragma unroll
        for (int u = 0; u < kGradAhead; ++u) {
          const int64_t row = s_row[min(l0 + u, l_end - 1)];
          z[u].load(Z + row * a.d + col);
          if (kMask) mk[u] = *reinterpret_cast<const uint32_t *>(a.mask + row * a.d + col);
        }
#pragma unroll
        for (int u = 0; u < kGradAhead; ++u) {
          if (l0 + u >= l_end) break;
          float zv[kGradCPL];
          z[u].get(zv);
          if (kMask) {
#pragma unroll
            for (int c = 0; c < kGradCPL; ++c)
              if (((mk[u] >> (8 * c)) & 0xffu) == 0) zv[c] = 0.f;
          }
          const float *cf = s_cf[l0 + u];
#pragma unroll
          for (int jj = 0; jj < RB; ++jj) {
            const float cj = cf[jj];   // zero past nr
#pragma unroll
            for (int c = 0; c < kGradCPL; ++c) acc[jj][c] = fmaf(cj, zv[c], acc[jj][c]);
          }
        }
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

// Adds each segment's partials in chunk order (up to 8 loads in flight) and
// writes the fp32 gradient page of every rank row.
__global__ __launch_bounds__(kGradThreads) void seg_outer_reduce_kernel(SegOuterArgs a) {
  constexpr int RB = kGradRankChunk;
  const int S = a.plan.hdr[LORA_PH_SEGS];
  const int col = (blockIdx.x * kGradThreads + threadIdx.x) * kGradCPL;
  if (col >= a.d) return;
  if (int64_t(a.plan.hdr[LORA_PH_RPAIRS]) > a.coef_cap) return;
  const int j0 = blockIdx.z * RB;
  for (int s = blockIdx.y; s < S; s += gridDim.y) {
    const int ad = a.plan.seg_adapter[s];
    const int r = a.rank[ad];
    if (r > a.max_rank || j0 >= r) continue;
    const int nr = min(RB, r - j0);
    const int q0 = a.plan.seg_off[s] / kGradPairChunk;
    const int q1 = (a.plan.seg_off[s + 1] - 1) / kGradPairChunk;
    const int32_t *pid = a.page_ids + a.page_start[ad];
    for (int jj = 0; jj < nr; ++jj) {
      float4 sum = make_float4(0.f, 0.f, 0.f, 0.f);
      for (int qb = q0; qb <= q1; qb += 8) {
        float4 v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u)
          v[u] = *reinterpret_cast<const float4 *>(
              a.part + (int64_t(s + min(qb + u, q1)) * a.max_rank + j0 + jj) * a.d + col);
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          if (qb + u <= q1) {
            sum.x += v[u].x; sum.y += v[u].y; sum.z += v[u].z; sum.w += v[u].w;
          }
        }
      }
      *reinterpret_cast<float4 *>(a.out_pages + int64_t(pid[j0 + jj]) * a.d + col) = sum;
    }
  }
}

}  // namespace

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
  if (dtype == LORA_BF16) {
    if (a.mask) hipLaunchKernelGGL((seg_outer_partial_kernel<uint16_t, true>), g1, block, 0, st, a);
    else hipLaunchKernelGGL((seg_outer_partial_kernel<uint16_t, false>), g1, block, 0, st, a);
  } else {
    if (a.mask) hipLaunchKernelGGL((seg_outer_partial_kernel<float, true>), g1, block, 0, st, a);
    else hipLaunchKernelGGL((seg_outer_partial_kernel<float, false>), g1, block, 0, st, a);
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const int64_t segs = TK < N ? TK : N;
  const dim3 g2(cols, unsigned(segs < 65535 ? segs : 65535), rchunks);
  hipLaunchKernelGGL(seg_outer_reduce_kernel, g2, block, 0, st, a);
  return hipGetLastError();
}

}  // namespace lora
