// Signed in-place merge: W_t <- round(W_t + sum_i c_i . s_i . (A_i . B_i)^T).
//
// Merging one adapter into the base weight is S-LoRA's single-adapter path
// (section 批处理); a list with the previous adapters at negative weight and
// the next ones at positive weight is AdaFuse's fused switch (section 关键设计
// item 2: concat of the negated previous down factors with the new ones), done
// here in one launch.  SGMM (item 3) adds in place; so does this kernel.
//
// Each workgroup owns a 64 x 64 tile of W_t (rows n over d_out, columns i
// over d_in) and walks the merge list: 16 rank rows at a time it stages
// c.s.B[j][n-tile] and A[:, j][i-tile] (both page-contiguous) in LDS, and
// every thread accumulates its 4 x 4 outputs as outer products in float32.
// W is read once and written once, with one rounding per element.
#include "lora_internal.h"

namespace lora {
namespace {

constexpr int kMT = 64;       // tile edge
constexpr int kMR = 16;       // rank rows staged per step

template <typename E>
__global__ __launch_bounds__(256) void merge_kernel(MergeArgs m) {
  __shared__ float Bs[kMR][kMT + 4];
  __shared__ float As[kMR][kMT + 4];
  __shared__ int bad;
  const int tid = threadIdx.x;
  const int tx = tid & 15, ty = tid >> 4;
  const int i0 = blockIdx.x * kMT;   // d_in columns
  const int n0 = blockIdx.y * kMT;   // d_out rows
  const E *Ap = static_cast<const E *>(m.a_pages);
  const E *Bp = static_cast<const E *>(m.b_pages);
  float acc[4][4] = {};

  for (int e = 0; e < m.m; ++e) {
    const int ad = m.ids[e];
    if (ad < 0 || ad >= m.n_adapters) continue;
    const int r = m.rank[ad];
    if (r <= 0 || r > LORA_MAX_RANK) continue;
    const int64_t s0 = m.page_start[ad], s1 = m.page_start[ad + 1];
    if (s0 < 0 || s1 - s0 != r || s1 > m.n_page_ids) continue;
    if (tid == 0) bad = 0;
    __syncthreads();
    for (int j = tid; j < r; j += 256) {
      const int64_t pg = m.page_ids[s0 + j];
      if (pg < 0 || pg >= m.n_pages) bad = 1;
    }
    __syncthreads();
    const bool skip = bad != 0;
    __syncthreads();   // everyone has read `bad` before it is reset
    if (skip) continue;
    const float coef = m.coeffs[e] * m.scale[ad];
    for (int j0 = 0; j0 < r; j0 += kMR) {
      const int nr = min(kMR, r - j0);
#pragma unroll
      for (int q = 0; q < kMR * kMT / 256; ++q) {
        const int idx = tid + q * 256;
        const int jj = idx / kMT, cc = idx % kMT;
        float bv = 0.f, av = 0.f;
        if (jj < nr) {
          const int64_t pg = m.page_ids[s0 + j0 + jj];
          bv = coef * Elem<E>::to_f(Bp[pg * m.d_out + n0 + cc]);
          av = Elem<E>::to_f(Ap[pg * m.d_in + i0 + cc]);
        }
        Bs[jj][cc] = bv;
        As[jj][cc] = av;
      }
      __syncthreads();
      for (int jj = 0; jj < nr; ++jj) {
        float b4[4], a4[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) { b4[q] = Bs[jj][ty * 4 + q]; a4[q] = As[jj][tx * 4 + q]; }
#pragma unroll
        for (int y = 0; y < 4; ++y)
#pragma unroll
          for (int x = 0; x < 4; ++x) acc[y][x] = fmaf(b4[y], a4[x], acc[y][x]);
      }
      __syncthreads();
    }
  }
  E *W = static_cast<E *>(m.W);
#pragma unroll
  for (int y = 0; y < 4; ++y) {
    E *row = W + int64_t(n0 + ty * 4 + y) * m.d_in + i0 + tx * 4;
#pragma unroll
    for (int x = 0; x < 4; ++x) row[x] = Elem<E>::from_f(Elem<E>::to_f(row[x]) + acc[y][x]);
  }
}

}  // namespace

hipError_t launch_merge(const MergeArgs &a, int dtype, hipStream_t s) {
  const dim3 grid(a.d_in / kMT, a.d_out / kMT);
  if (dtype == LORA_BF16) hipLaunchKernelGGL(merge_kernel<uint16_t>, grid, dim3(256), 0, s, a);
  else hipLaunchKernelGGL(merge_kernel<float>, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace lora
