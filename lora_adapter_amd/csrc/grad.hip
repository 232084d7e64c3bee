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
#include "lora_internal.h"

namespace lora {
namespace {

constexpr int kGradThreads = 256;
constexpr int kGradCPL = 2;                           // columns per lane
constexpr int kGradCols = kGradThreads * kGradCPL;    // columns per workgroup

template <typename E> struct Z2;
template <> struct Z2<uint16_t> {
  static __device__ __forceinline__ void load(const uint16_t *p, float v[2]) {
    const uint32_t w = *reinterpret_cast<const uint32_t *>(p);
    v[0] = bf_lo(w); v[1] = bf_hi(w);
  }
};
template <> struct Z2<float> {
  static __device__ __forceinline__ void load(const float *p, float v[2]) {
    const float2 w = *reinterpret_cast<const float2 *>(p);
    v[0] = w.x; v[1] = w.y;
  }
};

__device__ __forceinline__ int seg_of(const int32_t *seg_off, int S, int p) {
  int lo = 0, hi = S;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (seg_off[mid] <= p) lo = mid; else hi = mid;
  }
  return lo;
}

template <typename E, bool kMask>
__global__ __launch_bounds__(kGradThreads) void seg_outer_partial_kernel(SegOuterArgs a) {
  constexpr int RB = kGradRankChunk;
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
  const int col = (blockIdx.x * kGradThreads + threadIdx.x) * kGradCPL;
  const bool col_ok = col < a.d;
  const int j0 = blockIdx.z * RB;
  const E *Z = static_cast<const E *>(a.Z);
  int s = seg_of(a.plan.seg_off, S, pbeg);
  for (int p = pbeg; p < pend; ++s) {
    const int send = min(pend, a.plan.seg_off[s + 1]);
    const int ad = a.plan.seg_adapter[s];
    const int r = a.rank[ad];
    if (r > a.max_rank) {
      if (threadIdx.x == 0 && blockIdx.x == 0 && j0 == 0) atomicOr(a.err_word, LORA_DEVERR_CAPACITY);
    } else if (j0 < r) {
      const int nr = min(RB, r - j0);
      float acc[RB][kGradCPL];
#pragma unroll
      for (int jj = 0; jj < RB; ++jj)
#pragma unroll
        for (int c = 0; c < kGradCPL; ++c) acc[jj][c] = 0.f;
      for (int pp = p; pp < send; ++pp) {
        const int64_t t = a.plan.pair_tk[pp] / a.K;
        float z[kGradCPL] = {0.f, 0.f};
        if (col_ok) {
          Z2<E>::load(Z + t * a.d + col, z);
          if (kMask) {
            const uint16_t mb = *reinterpret_cast<const uint16_t *>(a.mask + t * a.d + col);
            if ((mb & 0xffu) == 0) z[0] = 0.f;
            if ((mb >> 8) == 0) z[1] = 0.f;
          }
        }
        const float *cf = a.coef + a.plan.u_off[pp] + j0;
#pragma unroll
        for (int jj = 0; jj < RB; ++jj) {
          if (jj < nr) {
            const float cj = cf[jj];
#pragma unroll
            for (int c = 0; c < kGradCPL; ++c) acc[jj][c] = fmaf(cj, z[c], acc[jj][c]);
          }
        }
      }
      if (col_ok) {
        float *dst = a.part + (int64_t(s + q) * a.max_rank + j0) * a.d + col;
#pragma unroll
        for (int jj = 0; jj < RB; ++jj)
          if (jj < nr)
            *reinterpret_cast<float2 *>(dst + int64_t(jj) * a.d) = make_float2(acc[jj][0], acc[jj][1]);
      }
    }
    p = send;
  }
}

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
      float2 sum = make_float2(0.f, 0.f);
      for (int q = q0; q <= q1; ++q) {
        const float2 v = *reinterpret_cast<const float2 *>(
            a.part + (int64_t(s + q) * a.max_rank + j0 + jj) * a.d + col);
        sum.x += v.x;
        sum.y += v.y;
      }
      *reinterpret_cast<float2 *>(a.out_pages + int64_t(pid[j0 + jj]) * a.d + col) = sum;
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
