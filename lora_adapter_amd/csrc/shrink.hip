// Segmented shrink: the LoRA down projection for every planned pair, with no
// padding and one launch for all adapters.
//
// S-LoRA (section 批处理) computes every request's x.A.B with custom kernels
// instead of padded batched GEMMs; AdaFuse (section 关键设计 item 3) groups
// rows by adapter (segmented gather).  Here one wave owns one rank row j of
// one segment's adapter: it streams that A page (d contiguous elements, the
// page of S-LoRA's Unified Paging) once from HBM with 16-byte coalesced
// loads and dots it with the rows of every token of the segment (read from
// L2: they are small and shared).  Rank rows of all segments are laid end to
// end (seg_row_off) and waves stride over them, so no adapter is padded to
// another's rank and no launch depends on the number of adapters.
//
// The same kernel computes the gradient's dY.B^T (pages = B, Z = dY).
#include "lora_internal.h"

namespace lora {
namespace {

constexpr int kShrinkThreads = 256;
constexpr int kShrinkPairs = 4;   // token rows dotted per A-chunk load

template <typename E, bool kMask>
__global__ __launch_bounds__(kShrinkThreads) void shrink_rows_kernel(ShrinkArgs s) {
  const int32_t *hdr = s.plan.hdr;
  const int S = hdr[LORA_PH_SEGS];
  const int R_used = hdr[LORA_PH_RUSED];
  const int64_t R_pairs = hdr[LORA_PH_RPAIRS];
  if (R_pairs > s.out_cap) {
    if (blockIdx.x == 0 && threadIdx.x == 0) atomicOr(s.err_word, LORA_DEVERR_CAPACITY);
    return;
  }
  const int lane = threadIdx.x & 63;
  const int waves = kShrinkThreads / 64;
  const int gw = blockIdx.x * waves + (threadIdx.x >> 6);
  const int nw = gridDim.x * waves;
  const E *Z = static_cast<const E *>(s.Z);
  const E *pages = static_cast<const E *>(s.pages);
  const int d = s.d;

  for (int g = gw; g < R_used; g += nw) {
    // segment owning rank row g: last s with seg_row_off[s] <= g
    int lo = 0, hi = S;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (s.plan.seg_row_off[mid] <= g) lo = mid; else hi = mid;
    }
    const int seg = lo;
    const int ad = s.plan.seg_adapter[seg];
    const int j = g - s.plan.seg_row_off[seg];
    const int64_t page = s.page_ids[s.page_start[ad] + j];
    const int p0 = s.plan.seg_off[seg], p1 = s.plan.seg_off[seg + 1];
    const float sc = s.scale[ad] * s.extra_scale;
    const E *arow = pages + page * d;

    for (int q = p0; q < p1; q += kShrinkPairs) {
      const int nq = min(kShrinkPairs, p1 - q);
      int tk[kShrinkPairs];
      const E *zr[kShrinkPairs];
      const uint8_t *mr[kShrinkPairs];
#pragma unroll
      for (int i = 0; i < kShrinkPairs; ++i) {
        tk[i] = s.plan.pair_tk[q + min(i, nq - 1)];
        const int64_t t = tk[i] / s.K;
        zr[i] = Z + t * d;
        mr[i] = kMask ? s.mask + t * d : nullptr;
      }
      float acc[kShrinkPairs] = {0.f, 0.f, 0.f, 0.f};
      for (int c = lane * 8; c < d; c += 64 * 8) {
        float av[8];
        Elem<E>::load8(arow + c, av);
#pragma unroll
        for (int i = 0; i < kShrinkPairs; ++i) {
          if (i < nq) {
            float zv[8];
            Elem<E>::load8(zr[i] + c, zv);
            if (kMask) {
              const uint2 mb = *reinterpret_cast<const uint2 *>(mr[i] + c);
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                if (((mb.x >> (8 * e)) & 0xffu) == 0) zv[e] = 0.f;
                if (((mb.y >> (8 * e)) & 0xffu) == 0) zv[4 + e] = 0.f;
              }
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[i] = fmaf(zv[e], av[e], acc[i]);
          }
        }
      }
#pragma unroll
      for (int i = 0; i < kShrinkPairs; ++i) acc[i] = wave_sum(acc[i]);
      if (lane == 0) {
#pragma unroll
        for (int i = 0; i < kShrinkPairs; ++i) {
          if (i < nq) s.out[s.plan.u_off[q + i] + j] = s.gates[tk[i]] * sc * acc[i];
        }
      }
    }
  }
}

}  // namespace

hipError_t launch_shrink(const ShrinkArgs &a, int dtype, int64_t rows_bound, hipStream_t st) {
  const int64_t waves = rows_bound < 1 ? 1 : rows_bound;
  int64_t blocks = (waves + 3) / 4;
  if (blocks > 4096) blocks = 4096;
  const dim3 grid{static_cast<unsigned>(blocks), 1, 1};
  const dim3 block{kShrinkThreads, 1, 1};
  if (dtype == LORA_BF16) {
    if (a.mask) hipLaunchKernelGGL((shrink_rows_kernel<uint16_t, true>), grid, block, 0, st, a);
    else hipLaunchKernelGGL((shrink_rows_kernel<uint16_t, false>), grid, block, 0, st, a);
  } else {
    if (a.mask) hipLaunchKernelGGL((shrink_rows_kernel<float, true>), grid, block, 0, st, a);
    else hipLaunchKernelGGL((shrink_rows_kernel<float, false>), grid, block, 0, st, a);
  }
  return hipGetLastError();
}

}  // namespace lora
