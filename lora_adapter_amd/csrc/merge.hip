// Signed in-place merge: W_t <- round(W_t + sum_i c_i . s_i . (A_i . B_i)^T).
//
// Merging one adapter into the base weight is S-LoRA's single-adapter path
// (section 批处理); a list with the previous adapters at negative weight and
// the next ones at positive weight is AdaFuse's fused switch (section 关键设计
// item 2: concat of the negated previous down factors with the new ones), done
// here in one launch.  SGMM (item 3) adds in place; so does this kernel.
//
// Workgroups walk 64 x 64 tiles of W_t (rows n over d_out, columns i over
// d_in).  The 256 threads of a workgroup read the merge list in parallel (one
// adapter per thread: id, coefficient, rank, page table, scale, page ids) and
// drop invalid entries; a block scan lays the valid rank rows out as one list
// of (page, c.s) in LDS, built once when it fits.  The list is then staged 32 rank rows at a time,
// across adapter boundaries: c.s.B[j][n-tile] and A[:, j][i-tile] (both
// page-contiguous) as float32 in LDS, every thread accumulating its 4 x 4
// outputs as outer products in float32.  W is read once and written once,
// with one rounding per element, by 8-byte (bf16) or 16-byte (fp32) accesses.
#include "lora_internal.h"

namespace lora {
namespace {

constexpr int kMT = 64;        // tile edge
constexpr int kMR = 32;        // rank rows staged per step
constexpr int kMAd = 256;      // adapters read per group (one per thread)
constexpr int kMList = 1024;   // rank rows listed per pass

// 4 consecutive elements of W / of a page row.
template <typename E> struct W4;
template <> struct W4<uint16_t> {
  static __device__ __forceinline__ void load(const uint16_t *p, float v[4]) {
    const uint2 w = *reinterpret_cast<const uint2 *>(p);
    v[0] = bf_lo(w.x); v[1] = bf_hi(w.x); v[2] = bf_lo(w.y); v[3] = bf_hi(w.y);
  }
  static __device__ __forceinline__ void store(uint16_t *p, const float v[4]) {
    *reinterpret_cast<uint2 *>(p) = make_uint2(uint32_t(f2bf(v[0])) | (uint32_t(f2bf(v[1])) << 16),
                                               uint32_t(f2bf(v[2])) | (uint32_t(f2bf(v[3])) << 16));
  }
};
template <> struct W4<float> {
  static __device__ __forceinline__ void load(const float *p, float v[4]) {
    const float4 w = *reinterpret_cast<const float4 *>(p);
    v[0] = w.x; v[1] = w.y; v[2] = w.z; v[3] = w.w;
  }
  static __device__ __forceinline__ void store(float *p, const float v[4]) {
    *reinterpret_cast<float4 *>(p) = make_float4(v[0], v[1], v[2], v[3]);
  }
};

// Lists the valid rank rows of merge entries [e0, e0 + kMAd) that fall in
// list window [lb, lb + kMList): page id and c.s in LDS.  Returns the group's
// total row count.  All threads call it (it has barriers).
__device__ __forceinline__ int merge_list(const MergeArgs &m, int e0, int lb, int *s_pid,
                                          float *s_cf, int *s_tot) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int e = e0 + tid;
  int r = 0, ps = 0;
  float cf = 0.f;
  if (e < m.m) {
    const int ad = m.ids[e];
    if (ad >= 0 && ad < m.n_adapters) {
      const int rr = m.rank[ad];
      const int64_t s0 = m.page_start[ad], s1 = m.page_start[ad + 1];
      if (rr > 0 && rr <= LORA_MAX_RANK && s0 >= 0 && s1 - s0 == rr && s1 <= m.n_page_ids) {
        bool ok = true;
        for (int j = 0; j < rr; ++j) {
          const int64_t pg = m.page_ids[s0 + j];
          ok = ok && pg >= 0 && pg < m.n_pages;
        }
        if (ok) {
          r = rr;
          ps = int(s0);
          cf = m.coeffs[e] * m.scale[ad];
        }
      }
    }
  }
  // exclusive prefix of the valid ranks over the group (wave sums through LDS)
  int inc = r;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(inc, d, 64);
    if (lane >= d) inc += y;
  }
  __syncthreads();   // s_tot / the list may still be read by a previous pass
  if (lane == 63) s_tot[wave] = inc;
  __syncthreads();
  int before = 0, total = 0;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const int t = s_tot[w];
    if (w < wave) before += t;
    total += t;
  }
  const int off = before + inc - r;
  const int ja = max(0, lb - off), jb = min(r, lb + kMList - off);
  for (int j = ja; j < jb; ++j) {
    s_pid[off + j - lb] = m.page_ids[ps + j];
    s_cf[off + j - lb] = cf;
  }
  __syncthreads();
  return total;
}

// Adds the listed rows [0, nl) to acc for the tile (i0, n0).
template <typename E>
__device__ __forceinline__ void merge_rows(const MergeArgs &m, int i0, int n0, int nl,
                                           const int *s_pid, const float *s_cf,
                                           float (*Bs)[kMT + 4], float (*As)[kMT + 4],
                                           float (&acc)[4][4]) {
  const int tid = threadIdx.x;
  const int tx = tid & 15, ty = tid >> 4;
  const E *Ap = static_cast<const E *>(m.a_pages);
  const E *Bp = static_cast<const E *>(m.b_pages);
  for (int j0 = 0; j0 < nl; j0 += kMR) {
    const int nr = min(kMR, nl - j0);
    // stage 32 rank rows x 64 columns of B (scaled) and of A, 4 values per thread each
#pragma unroll
    for (int q = 0; q < kMR * kMT / (4 * 256); ++q) {
      const int idx = tid + q * 256;
      const int jj = idx / (kMT / 4), cc = (idx % (kMT / 4)) * 4;
      float bv[4] = {0.f, 0.f, 0.f, 0.f}, av[4] = {0.f, 0.f, 0.f, 0.f};
      if (jj < nr) {
        const int64_t pg = s_pid[j0 + jj];
        const float c = s_cf[j0 + jj];
        W4<E>::load(Bp + pg * m.d_out + n0 + cc, bv);
        W4<E>::load(Ap + pg * m.d_in + i0 + cc, av);
#pragma unroll
        for (int u = 0; u < 4; ++u) bv[u] *= c;
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        Bs[jj][cc + u] = bv[u];
        As[jj][cc + u] = av[u];
      }
    }
    __syncthreads();
    for (int jj = 0; jj < nr; ++jj) {
      const float4 b4 = *reinterpret_cast<const float4 *>(&Bs[jj][ty * 4]);
      const float4 a4 = *reinterpret_cast<const float4 *>(&As[jj][tx * 4]);
      const float bb[4] = {b4.x, b4.y, b4.z, b4.w}, aa[4] = {a4.x, a4.y, a4.z, a4.w};
#pragma unroll
      for (int y = 0; y < 4; ++y)
#pragma unroll
        for (int x = 0; x < 4; ++x) acc[y][x] = fmaf(bb[y], aa[x], acc[y][x]);
    }
    __syncthreads();
  }
}

// Persistent: each workgroup walks tiles blockIdx.x, + gridDim.x, ...  When
// the whole merge list fits one LDS list it is built once per workgroup.
template <typename E>
__global__ __launch_bounds__(256) void merge_kernel(MergeArgs m) {
  __shared__ float Bs[kMR][kMT + 4];
  __shared__ float As[kMR][kMT + 4];
  __shared__ int s_pid[kMList];
  __shared__ float s_cf[kMList];
  __shared__ int s_tot[4];
  const int tid = threadIdx.x;
  const int tx = tid & 15, ty = tid >> 4;
  const int tiles_i = m.d_in / kMT;
  const int ntiles = tiles_i * (m.d_out / kMT);
  E *W = static_cast<E *>(m.W);
  const bool one_list = m.m <= kMAd;
  int total = 0;
  if (one_list) total = merge_list(m, 0, 0, s_pid, s_cf, s_tot);
  const bool resident = one_list && total <= kMList;
  for (int t = blockIdx.x; t < ntiles; t += gridDim.x) {
    const int i0 = (t % tiles_i) * kMT;   // d_in columns
    const int n0 = (t / tiles_i) * kMT;   // d_out rows
    // the tile's W values, loaded first so their round trip overlaps the staging
    float w[4][4];
#pragma unroll
    for (int y = 0; y < 4; ++y) W4<E>::load(W + int64_t(n0 + ty * 4 + y) * m.d_in + i0 + tx * 4, w[y]);
    float acc[4][4] = {};
    if (resident) {
      merge_rows<E>(m, i0, n0, total, s_pid, s_cf, Bs, As, acc);
    } else {
      for (int e0 = 0; e0 < m.m; e0 += kMAd) {
        const int tot = merge_list(m, e0, 0, s_pid, s_cf, s_tot);
        for (int lb = 0; lb < tot; lb += kMList) {
          if (lb > 0) merge_list(m, e0, lb, s_pid, s_cf, s_tot);
          merge_rows<E>(m, i0, n0, min(kMList, tot - lb), s_pid, s_cf, Bs, As, acc);
        }
      }
    }
#pragma unroll
    for (int y = 0; y < 4; ++y) {
#pragma unroll
      for (int x = 0; x < 4; ++x) w[y][x] += acc[y][x];
      W4<E>::store(W + int64_t(n0 + ty * 4 + y) * m.d_in + i0 + tx * 4, w[y]);
    }
  }
}

}  // namespace

hipError_t launch_merge(const MergeArgs &a, int dtype, hipStream_t s) {
  const int ntiles = (a.d_in / kMT) * (a.d_out / kMT);
  const dim3 grid(unsigned(ntiles < 1024 ? ntiles : 1024));
  if (dtype == LORA_BF16) hipLaunchKernelGGL(merge_kernel<uint16_t>, grid, dim3(256), 0, s, a);
  else hipLaunchKernelGGL(merge_kernel<float>, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace lora
