// Segmented shrink: the LoRA down projection of every planned pair, with no
// padding and a fixed number of launches whatever the number of adapters.
//
// S-LoRA (section 批处理) computes every request's x.A.B with custom kernels
// instead of padded batched GEMMs; AdaFuse (section 关键设计 item 3) groups
// rows by adapter (segmented gather); LoRAForge (section LoRAForge的核心设计)
// keeps each adapter's exact retained rank.  The output is
//   out[u_off[p] + j] = coef_p . sum_i Z[t_p][i] . m[t_p][i] . page_j[i]
// with coef_p = gates[t_p][k_p] . scale[a] . extra_scale, for every planned
// pair p and rank row j of its adapter (page_j = A column j, stored
// contiguously as one page of the pool).
//
// Two kernels, split by segment size:
//   * units kernel (every segment, except those the tile kernel takes): a
//     persistent grid of kShrinkWaves waves over the plan's unit schedule
//     (see shrink_units_kernel); A pages stream from HBM with 16-byte
//     coalesced loads, token rows come from L2.
//   * tile kernel (the whole 32-pair tiles of segments of kBigSegPairs
//     pairs or more, bf16, large batches, i.e. prefill; the units kernel
//     takes each such segment's last len % 32 pairs, so there are at most
//     T*K / 32 tiles and a batch of 8192 pairs fills exactly 256
//     workgroups): two MFMA blocks of 16 tokens x 16 rank rows
//     (v_mfma_f32_16x16x32_bf16) sharing each A page fragment, token rows
//     and A pages read straight from global memory as MFMA fragments, the
//     dropout mask applied to the bf16 fragment (exact), the four waves of a
//     workgroup splitting d and adding through LDS.  X is read once from HBM
//     per rank-row block; the A pages, from L2, once per 32 pairs.
// When the tile kernel is on and d <= 6144, both run in one launch
// (shrink_both_kernel): its tiles first, then the units schedule.
// The same kernels compute the gradient's dY.B^T (Z = dY, pages = B) where
// the gradient does not form it on MFMA.
#include "lora_internal.h"
#include "shrink_units.h"

namespace lora {
namespace {

constexpr int kTileRank = 16;       // rank rows per MFMA tile
constexpr int kTileAhead = 4;       // K steps per batch of loads

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ bool capacity_ok(const ShrinkArgs &s) {
  if (int64_t(s.plan.hdr[LORA_PH_RPAIRS]) <= s.out_cap) return true;
  if (blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) atomicOr(s.err_word, LORA_DEVERR_CAPACITY);
  return false;
}

// Standalone decode shrink: one 64-lane workgroup per wave of the schedule.
template <typename E, bool kMask, int kCh, bool kResident>
__global__ __launch_bounds__(64) void shrink_units_kernel(ShrinkArgs s) {
  shrink_units_wave<E, kMask, kCh, kResident>(s, blockIdx.x);
}

// Finds the big segment and the 32-pair tile of workgroup b, the tiles of the
// big list numbered in list order (a wave-wide scan over 64 entries at a
// time).  Returns false past the last tile.
__device__ __forceinline__ bool tile_of(const PlanView &pv, int b, int lane, int &seg, int &q0, int &pe) {
  const int nb = pv.big_list[0];
  int base = 0;
  for (int c0 = 0; c0 < nb; c0 += 64) {
    const int i = c0 + lane;
    int sg = 0, nt = 0, pb_ = 0, pe_ = 0;
    if (i < nb) {
      sg = pv.big_list[1 + i];
      pb_ = pv.seg_desc[2 * sg].w;
      pe_ = pv.seg_desc[2 * sg + 1].x;
      nt = (pe_ - pb_) / kTileTok;                  // whole tiles only
    }
    int incl = nt;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int v = __shfl_up(incl, o, 64);
      if (lane >= o) incl += v;
    }
    const uint64_t hit = __ballot(i < nb && base + incl > b);
    if (hit) {
      const int l = __ffsll(static_cast<unsigned long long>(hit)) - 1;
      seg = __shfl(sg, l, 64);
      const int first = base + __shfl(incl - nt, l, 64);
      q0 = __shfl(pb_, l, 64) + (b - first) * kTileTok;
      pe = __shfl(pe_, l, 64);
      return true;
    }
    base += __shfl(incl, 63, 64);
  }
  return false;
}

// One workgroup per 32-pair tile of the big segments, numbered across the
// list so that consecutive workgroups (which the dispatcher spreads over the
// XCDs) cover every segment evenly.
template <bool kMask>
__device__ __forceinline__ void shrink_tile_wg(const ShrinkArgs &s, const int b) {
  if (!capacity_ok(s)) return;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int seg = 0, q0 = 0, pe = 0;
  if (!tile_of(s.plan, b, lane, seg, q0, pe)) return;
  const int4 d0 = s.plan.seg_desc[2 * seg];
  const int ad = d0.x, r = d0.y, ps = d0.z;
  const int nq = min(kTileTok, pe - q0);

  // two 16-pair MFMA row blocks per tile share every A page fragment
  __shared__ f32x4_t red[4][2][64];
  const int d = s.d;
  const int kw = d / 4;                          // this wave's part of d (multiple of 16)
  const int kbeg = wave * kw;
  const uint16_t *Z = static_cast<const uint16_t *>(s.Z);
  const uint16_t *pages = static_cast<const uint16_t *>(s.pages);
  // A operand of block h: token row (lane % 16) of its 16 pairs, 8 values
  // at k + (lane / 16) * 8
  const int trow = lane & 15, kofs = (lane >> 4) * 8;
  const int64_t t0 = s.plan.pair_tk[q0 + min(trow, nq - 1)] / s.K;
  const int64_t t1 = s.plan.pair_tk[q0 + min(16 + trow, nq - 1)] / s.K;
  const uint16_t *zrow0 = Z + t0 * d, *zrow1 = Z + t1 * d;
  const uint8_t *mrow0 = kMask ? s.mask + t0 * d : nullptr;
  const uint8_t *mrow1 = kMask ? s.mask + t1 * d : nullptr;
  const float sc = s.scale[ad] * s.extra_scale;

  // the keep mask (bytes 0 or 1) on a bf16 fragment: the bytes of elements
  // 2i and 2i + 1 go to bits 0 and 16 (one byte permute), times 0xffff
  auto masked = [&](uint4 z, uint2 m) {
    if constexpr (kMask) {
      uint32_t w[4] = {z.x, z.y, z.z, z.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t x = __builtin_amdgcn_perm(0u, i < 2 ? m.x : m.y, (i & 1) ? 0x0c030c02u : 0x0c010c00u);
        w[i] &= (x << 16) - x;
      }
      z = make_uint4(w[0], w[1], w[2], w[3]);
    }
    return z;
  };
  // K steps of 32 in batches of kTileAhead, the next batch's loads in flight
  // while the current batch's MFMAs run (kw is a multiple of 32)
  const int nsteps = kw / 32;
  for (int jb = 0; jb < r; jb += kTileRank) {
    // B operand: rank row jb + (lane % 16), same k offsets
    const int jr = jb + (lane & 15);
    const uint16_t *arow = pages + int64_t(s.page_ids[ps + min(jr, r - 1)]) * d;
    f32x4_t acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
    uint4 za0[kTileAhead], za1[kTileAhead], pa[kTileAhead];
    uint4 zb0[kTileAhead], zb1[kTileAhead], pb2[kTileAhead];
    uint2 ma0[kTileAhead], ma1[kTileAhead], mb0[kTileAhead], mb1[kTileAhead];
    auto load_batch = [&](uint4 (&z0)[kTileAhead], uint4 (&z1)[kTileAhead], uint4 (&p)[kTileAhead],
                          uint2 (&m0)[kTileAhead], uint2 (&m1)[kTileAhead], int i0) {
#pragma unroll
      for (int u = 0; u < kTileAhead; ++u) {
        const int k = kbeg + min(i0 + u, nsteps - 1) * 32 + kofs;
        z0[u] = *reinterpret_cast<const uint4 *>(zrow0 + k);
        z1[u] = *reinterpret_cast<const uint4 *>(zrow1 + k);
        p[u] = *reinterpret_cast<const uint4 *>(arow + k);
        if (kMask) {
          m0[u] = *reinterpret_cast<const uint2 *>(mrow0 + k);
          m1[u] = *reinterpret_cast<const uint2 *>(mrow1 + k);
        }
      }
    };
    auto mfma_batch = [&](const uint4 (&z0)[kTileAhead], const uint4 (&z1)[kTileAhead],
                          const uint4 (&p)[kTileAhead], const uint2 (&m0)[kTileAhead],
                          const uint2 (&m1)[kTileAhead], int i0) {
#pragma unroll
      for (int u = 0; u < kTileAhead; ++u) {
        if (i0 + u >= nsteps) break;
        const uint4 x0 = masked(z0[u], m0[u]), x1 = masked(z1[u], m1[u]);
        bf16x8_t fa0, fa1, fb;
        __builtin_memcpy(&fa0, &x0, 16);
        __builtin_memcpy(&fa1, &x1, 16);
        __builtin_memcpy(&fb, &p[u], 16);
        acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa0, fb, acc0, 0, 0, 0);
        acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa1, fb, acc1, 0, 0, 0);
      }
    };
    load_batch(za0, za1, pa, ma0, ma1, 0);
    for (int i0 = 0; i0 < nsteps; i0 += 2 * kTileAhead) {
      load_batch(zb0, zb1, pb2, mb0, mb1, i0 + kTileAhead);
      mfma_batch(za0, za1, pa, ma0, ma1, i0);
      if (i0 + kTileAhead >= nsteps) break;
      load_batch(za0, za1, pa, ma0, ma1, i0 + 2 * kTileAhead);
      mfma_batch(zb0, zb1, pb2, mb0, mb1, i0 + kTileAhead);
    }
    red[wave][0][lane] = acc0;
    red[wave][1][lane] = acc1;
    __syncthreads();
    if (wave < 2) {
      // wave h adds block h over the four K quarters
      f32x4_t v = red[0][wave][lane];
#pragma unroll
      for (int w = 1; w < 4; ++w) {
        const f32x4_t o = red[w][wave][lane];
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] += o[i];
      }
      // lane holds rank column (lane % 16) and token rows 4 * (lane / 16) + i
      const int j = jb + (lane & 15);
      if (j < r) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int tr = 16 * wave + (lane >> 4) * 4 + i;
          if (tr < nq) {
            const int p = q0 + tr;
            s.out[s.plan.u_off[p] + j] = s.plan.pair_gate[p] * sc * v[i];
          }
        }
      }
    }
    __syncthreads();
  }
}

template <bool kMask>
__global__ __launch_bounds__(256) void shrink_tile_kernel(ShrinkArgs s) {
  shrink_tile_wg<kMask>(s, blockIdx.x);
}

// Both shrinks in one launch (bf16 batches with big segments): workgroups
// 0 .. n_tile-1 run the tile kernel's tiles, the others the units
// schedule, one schedule wave per wave.  The two write disjoint pairs.
template <bool kMask, int kCh>
__global__ __launch_bounds__(256) void shrink_both_kernel(ShrinkArgs s, int n_tile) {
  const int b = int(blockIdx.x);
  if (b < n_tile) {
    shrink_tile_wg<kMask>(s, b);
    return;
  }
  shrink_units_wave<uint16_t, kMask, kCh, true>(s, (b - n_tile) * 4 + int(threadIdx.x >> 6));
}

// Workgroups of the tile shrink: the whole 32-pair tiles of the big
// segments, at most T*K / 32 (at least one workgroup).
int shrink_tile_wgs(int64_t TK, int64_t n_adapters) {
  (void)n_adapters;
  return int(TK / kTileTok > 0 ? TK / kTileTok : 1);
}

}  // namespace

hipError_t launch_shrink(const ShrinkArgs &a, int dtype, int64_t TK, int64_t n_adapters,
                         int d_in, int d_out, hipStream_t st) {
  const int64_t segs = TK < n_adapters ? TK : n_adapters;
  if (segs <= 0) return hipSuccess;
  ShrinkArgs s = a;
  s.big_segments = shrink_tile_enabled(dtype, TK, d_in, d_out) ? 1 : 0;
  if (s.big_segments && s.d <= 12 * 512) {
    // one launch for both (the units part resident: d fits its chunks)
    static_assert(kShrinkWaves % 4 == 0, "four schedule waves per workgroup");
    const int n_tile = shrink_tile_wgs(TK, n_adapters);
    const dim3 g2{unsigned(n_tile + kShrinkWaves / 4), 1, 1}, b2{256, 1, 1};
    if (s.d <= 8 * 512) {
      if (s.mask) hipLaunchKernelGGL((shrink_both_kernel<true, 8>), g2, b2, 0, st, s, n_tile);
      else hipLaunchKernelGGL((shrink_both_kernel<false, 8>), g2, b2, 0, st, s, n_tile);
    } else {
      if (s.mask) hipLaunchKernelGGL((shrink_both_kernel<true, 12>), g2, b2, 0, st, s, n_tile);
      else hipLaunchKernelGGL((shrink_both_kernel<false, 12>), g2, b2, 0, st, s, n_tile);
    }
    return hipGetLastError();
  }
  const dim3 grid{unsigned(kShrinkWaves), 1, 1}, block{64, 1, 1};
#define LORA_SHRINK_UNITS(E, M, CH, RES) \
  hipLaunchKernelGGL((shrink_units_kernel<E, M, CH, RES>), grid, block, 0, st, s)
  const int d = s.d;
  if (dtype == LORA_BF16) {
    if (d <= 8 * 512) {
      if (s.mask) LORA_SHRINK_UNITS(uint16_t, true, 8, true); else LORA_SHRINK_UNITS(uint16_t, false, 8, true);
    } else if (d <= 12 * 512) {
      if (s.mask) LORA_SHRINK_UNITS(uint16_t, true, 12, true); else LORA_SHRINK_UNITS(uint16_t, false, 12, true);
    } else {
      if (s.mask) LORA_SHRINK_UNITS(uint16_t, true, 8, false); else LORA_SHRINK_UNITS(uint16_t, false, 8, false);
    }
  } else {
    // fp32: 8 elements are 32 bytes, two loads per chunk
    if (d <= 4 * 512) {
      if (s.mask) LORA_SHRINK_UNITS(float, true, 4, true); else LORA_SHRINK_UNITS(float, false, 4, true);
    } else {
      if (s.mask) LORA_SHRINK_UNITS(float, true, 4, false); else LORA_SHRINK_UNITS(float, false, 4, false);
    }
  }
#undef LORA_SHRINK_UNITS
  const hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  return launch_shrink_big(s, dtype, TK, n_adapters, d_in, d_out, st);
}

hipError_t launch_shrink_big(const ShrinkArgs &a, int dtype, int64_t TK, int64_t n_adapters,
                             int d_in, int d_out, hipStream_t st) {
  if (!shrink_tile_enabled(dtype, TK, d_in, d_out)) return hipSuccess;
  ShrinkArgs s = a;
  s.big_segments = 1;
  const dim3 g2{unsigned(shrink_tile_wgs(TK, n_adapters)), 1, 1}, b2{256, 1, 1};
  if (s.mask) hipLaunchKernelGGL((shrink_tile_kernel<true>), g2, b2, 0, st, s);
  else hipLaunchKernelGGL((shrink_tile_kernel<false>), g2, b2, 0, st, s);
  return hipGetLastError();
}

}  // namespace lora
