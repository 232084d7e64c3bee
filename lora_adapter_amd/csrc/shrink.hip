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
//   * rows kernel (segments with fewer than kBigSeg pairs, i.e. decode):
//     one wave per (segment, 4 rank rows).  It reads the segment's packed
//     descriptor (adapter, rank, page_start, pair range), streams its A pages
//     from HBM with 16-byte coalesced loads and dots them with each token row
//     of the segment (rows are small and shared, so they come from L2).
//   * tile kernel (segments with kBigSeg pairs or more, i.e. prefill):
//     an MFMA tile of 16 tokens x 16 rank rows (v_mfma_f32_16x16x32_bf16),
//     token rows and A pages read straight from global memory as MFMA
//     fragments, the dropout mask applied to the bf16 fragment (exact), the
//     four waves of a workgroup splitting d and adding through LDS.  X is
//     read once from HBM per rank-row block.
// The same kernels compute the gradient's dY.B^T (Z = dY, pages = B).
#include "lora_internal.h"

namespace lora {
namespace {

constexpr int kRowsPerWave = 2;     // rank rows per wave in the rows kernel
constexpr int kPairsPerPass = 2;    // token rows per pass
constexpr int kChunks = 8;          // 16-byte chunks per lane issued together (4096 bf16)
constexpr int kBigSeg = 64;         // segments this large use the tile kernel
constexpr int kTileTok = 16;        // tokens per MFMA tile
constexpr int kTileRank = 16;       // rank rows per MFMA tile

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ bool capacity_ok(const ShrinkArgs &s) {
  if (int64_t(s.plan.hdr[LORA_PH_RPAIRS]) <= s.out_cap) return true;
  if (blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) atomicOr(s.err_word, LORA_DEVERR_CAPACITY);
  return false;
}

// 8 consecutive elements held raw until they are needed (so that a batch of
// loads can be issued before the first conversion waits on one).
template <typename E> struct Raw;
template <> struct Raw<uint16_t> {
  uint4 v;
  __device__ __forceinline__ void load(const uint16_t *p) { v = *reinterpret_cast<const uint4 *>(p); }
  __device__ __forceinline__ void to8(float o[8]) const {
    o[0] = bf_lo(v.x); o[1] = bf_hi(v.x); o[2] = bf_lo(v.y); o[3] = bf_hi(v.y);
    o[4] = bf_lo(v.z); o[5] = bf_hi(v.z); o[6] = bf_lo(v.w); o[7] = bf_hi(v.w);
  }
};
template <> struct Raw<float> {
  float4 a, b;
  __device__ __forceinline__ void load(const float *p) {
    a = *reinterpret_cast<const float4 *>(p);
    b = *reinterpret_cast<const float4 *>(p + 4);
  }
  __device__ __forceinline__ void to8(float o[8]) const {
    o[0] = a.x; o[1] = a.y; o[2] = a.z; o[3] = a.w; o[4] = b.x; o[5] = b.y; o[6] = b.z; o[7] = b.w;
  }
};

// Zero the elements of 8 gathered values whose keep-mask byte is 0.
__device__ __forceinline__ void apply_mask8(float v[8], uint2 mb) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    if (((mb.x >> (8 * e)) & 0xffu) == 0) v[e] = 0.f;
    if (((mb.y >> (8 * e)) & 0xffu) == 0) v[4 + e] = 0.f;
  }
}

// Control data is fetched lane-parallel (one lane per word, one instruction
// per round trip) and broadcast with shuffles: a decode segment costs three
// dependent round trips (descriptor, page and token ids, then A and X).
template <typename E, bool kMask>
__global__ __launch_bounds__(64) void shrink_rows_kernel(ShrinkArgs s) {
  const int seg = blockIdx.x;
  const int lane = threadIdx.x;
  // round trip 1: segment descriptor (lanes 0-7) and header words (lanes 8, 9);
  // seg < grid size <= T*K keeps the descriptor read in bounds
  int w = 0;
  if (lane < 8) w = reinterpret_cast<const int *>(s.plan.seg_desc)[8 * seg + lane];
  else if (lane == 8) w = s.plan.hdr[LORA_PH_SEGS];
  else if (lane == 9) w = s.plan.hdr[LORA_PH_RPAIRS];
  if (seg >= __shfl(w, 8, 64)) return;
  if (int64_t(__shfl(w, 9, 64)) > s.out_cap) {
    if (seg == 0 && blockIdx.y == 0 && lane == 0) atomicOr(s.err_word, LORA_DEVERR_CAPACITY);
    return;
  }
  const int ad = __shfl(w, 0, 64), r = __shfl(w, 1, 64), ps = __shfl(w, 2, 64);
  const int pb = __shfl(w, 3, 64), pe = __shfl(w, 4, 64);
  if (pe - pb >= kBigSeg && s.big_segments) return;
  const int d = s.d;
  const E *Z = static_cast<const E *>(s.Z);
  const E *pages = static_cast<const E *>(s.pages);
  for (int j0 = blockIdx.y * kRowsPerWave; j0 < r; j0 += gridDim.y * kRowsPerWave) {
  const int nr = min(kRowsPerWave, r - j0);
  // round trip 2: page ids (lanes 0-3) and the adapter scale (lane 4)
  int pw = 0;
  float scw = 0.f;
  if (lane < kRowsPerWave) pw = s.page_ids[ps + j0 + min(lane, nr - 1)];
  else if (lane == kRowsPerWave) scw = s.scale[ad];
  const float sc = __shfl(scw, kRowsPerWave, 64) * s.extra_scale;
  const E *arow[kRowsPerWave];
#pragma unroll
  for (int i = 0; i < kRowsPerWave; ++i) arow[i] = pages + int64_t(__shfl(pw, i, 64)) * d;

  for (int q = pb; q < pe; q += kPairsPerPass) {
    const int nq = min(kPairsPerPass, pe - q);
    // token of each pair (lanes 0-3), then each lane's own gate and U offset
    int tkl = 0;
    if (lane < kPairsPerPass) tkl = s.plan.pair_tk[q + min(lane, nq - 1)];
    float gate = 0.f;
    int uoff = 0;
    if (lane < nq) {
      gate = s.gates[tkl];
      uoff = s.plan.u_off[q + lane];
    }
    int tk[kPairsPerPass];
    const E *zr[kPairsPerPass];
    const uint8_t *mr[kPairsPerPass];
#pragma unroll
    for (int i = 0; i < kPairsPerPass; ++i) {
      tk[i] = __shfl(tkl, i, 64);
      const int64_t t = tk[i] / s.K;
      zr[i] = Z + t * d;
      mr[i] = kMask ? s.mask + t * d : nullptr;
    }
    float acc[kRowsPerWave][kPairsPerPass];
#pragma unroll
    for (int a = 0; a < kRowsPerWave; ++a)
#pragma unroll
      for (int i = 0; i < kPairsPerPass; ++i) acc[a][i] = 0.f;
    // Blocks of kChunks x 512 elements: every load of a block is issued
    // before any is used, from clamped addresses (rows past nr / pairs past nq
    // repeat the last valid one and are never written; chunks past d repeat
    // the last chunk and are skipped below), so no load waits on a branch.
    for (int cb = 0; cb < d; cb += kChunks * 512) {
      Raw<E> ar[kRowsPerWave][kChunks], zrw[kPairsPerPass][kChunks];
      uint2 mk[kPairsPerPass][kChunks];
#pragma unroll
      for (int ch = 0; ch < kChunks; ++ch) {
        const int c = min(cb + ch * 512 + lane * 8, d - 8);
#pragma unroll
        for (int a = 0; a < kRowsPerWave; ++a) ar[a][ch].load(arow[a] + c);
#pragma unroll
        for (int i = 0; i < kPairsPerPass; ++i) {
          zrw[i][ch].load(zr[i] + c);
          if (kMask) mk[i][ch] = *reinterpret_cast<const uint2 *>(mr[i] + c);
        }
      }
#pragma unroll
      for (int ch = 0; ch < kChunks; ++ch) {
        if (cb + ch * 512 + lane * 8 >= d) continue;
        float av[kRowsPerWave][8];
#pragma unroll
        for (int a = 0; a < kRowsPerWave; ++a) ar[a][ch].to8(av[a]);
#pragma unroll
        for (int i = 0; i < kPairsPerPass; ++i) {
          float zv[8];
          zrw[i][ch].to8(zv);
          if (kMask) apply_mask8(zv, mk[i][ch]);
#pragma unroll
          for (int a = 0; a < kRowsPerWave; ++a)
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[a][i] = fmaf(zv[e], av[a][e], acc[a][i]);
        }
      }
    }
#pragma unroll
    for (int a = 0; a < kRowsPerWave; ++a)
#pragma unroll
      for (int i = 0; i < kPairsPerPass; ++i) acc[a][i] = wave_sum(acc[a][i]);
    if (lane < nq) {
      // lane i writes pair q + i; select its sums without dynamic indexing
      float mine[kRowsPerWave];
#pragma unroll
      for (int a = 0; a < kRowsPerWave; ++a) {
        mine[a] = acc[a][0];
#pragma unroll
        for (int i = 1; i < kPairsPerPass; ++i)
          if (lane == i) mine[a] = acc[a][i];
      }
      const float coef = gate * sc;
      float *o = s.out + uoff + j0;
#pragma unroll
      for (int a = 0; a < kRowsPerWave; ++a)
        if (a < nr) o[a] = coef * mine[a];
    }
  }
  }  // rank-row groups
}

// bf16 only: MFMA operands are bf16.
template <bool kMask>
__global__ __launch_bounds__(256) void shrink_tile_kernel(ShrinkArgs s) {
  const int seg = blockIdx.x;
  if (seg >= s.plan.hdr[LORA_PH_SEGS]) return;
  if (!capacity_ok(s)) return;
  const int4 d0 = s.plan.seg_desc[2 * seg];
  const int4 d1 = s.plan.seg_desc[2 * seg + 1];
  const int ad = d0.x, r = d0.y, ps = d0.z, pb = d0.w, pe = d1.x;
  if (pe - pb < kBigSeg) return;
  const int q0 = pb + blockIdx.y * kTileTok;
  if (q0 >= pe) return;
  const int nq = min(kTileTok, pe - q0);

  __shared__ f32x4_t red[4][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int d = s.d;
  const int kw = d / 4;                          // this wave's part of d (multiple of 16)
  const int kbeg = wave * kw, kend = kbeg + kw;
  const uint16_t *Z = static_cast<const uint16_t *>(s.Z);
  const uint16_t *pages = static_cast<const uint16_t *>(s.pages);
  // A operand: token row (lane % 16) of the tile, 8 values at k + (lane / 16) * 8
  const int trow = lane & 15, kofs = (lane >> 4) * 8;
  const int pq = q0 + min(trow, nq - 1);
  const int64_t t = s.plan.pair_tk[pq] / s.K;
  const uint16_t *zrow = Z + t * d;
  const uint8_t *mrow = kMask ? s.mask + t * d : nullptr;
  const float sc = s.scale[ad] * s.extra_scale;

  for (int jb = 0; jb < r; jb += kTileRank) {
    // B operand: rank row jb + (lane % 16), same k offsets
    const int jr = jb + (lane & 15);
    const uint16_t *arow = pages + int64_t(s.page_ids[ps + min(jr, r - 1)]) * d;
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 8
    for (int k = kbeg; k < kend; k += 32) {
      uint4 xa = *reinterpret_cast<const uint4 *>(zrow + k + kofs);
      const uint4 ab = *reinterpret_cast<const uint4 *>(arow + k + kofs);
      if (kMask) {
        const uint2 mb = *reinterpret_cast<const uint2 *>(mrow + k + kofs);
        uint32_t w[4] = {xa.x, xa.y, xa.z, xa.w};
        const uint32_t mw[2] = {mb.x, mb.y};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          if (((mw[e >> 2] >> (8 * (e & 3))) & 0xffu) == 0) w[e >> 1] &= (e & 1) ? 0x0000ffffu : 0xffff0000u;
        }
        xa = make_uint4(w[0], w[1], w[2], w[3]);
      }
      bf16x8_t fa, fb;
      __builtin_memcpy(&fa, &xa, 16);
      __builtin_memcpy(&fb, &ab, 16);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa, fb, acc, 0, 0, 0);
    }
    red[wave][lane] = acc;
    __syncthreads();
    if (wave == 0) {
      f32x4_t v = red[0][lane];
#pragma unroll
      for (int w = 1; w < 4; ++w) {
        const f32x4_t o = red[w][lane];
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] += o[i];
      }
      // lane holds rank column (lane % 16) and token rows 4 * (lane / 16) + i
      const int j = jb + (lane & 15);
      if (j < r) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int tr = (lane >> 4) * 4 + i;
          if (tr < nq) {
            const int p = q0 + tr;
            s.out[s.plan.u_off[p] + j] = s.gates[s.plan.pair_tk[p]] * sc * v[i];
          }
        }
      }
    }
    __syncthreads();
  }
}

}  // namespace

hipError_t launch_shrink(const ShrinkArgs &a, int dtype, int64_t TK, int64_t n_adapters,
                         int max_rank, hipStream_t st) {
  const int64_t segs = TK < n_adapters ? TK : n_adapters;
  if (segs <= 0) return hipSuccess;
  const unsigned gx = unsigned(segs);
  const unsigned gy = unsigned((max_rank + kRowsPerWave - 1) / kRowsPerWave);
  const dim3 grid{gx, gy > 0 ? gy : 1u, 1}, block{64, 1, 1};
  ShrinkArgs s = a;
  s.big_segments = (dtype == LORA_BF16 && TK >= 512 && s.d % 128 == 0) ? 1 : 0;
  if (dtype == LORA_BF16) {
    if (s.mask) hipLaunchKernelGGL((shrink_rows_kernel<uint16_t, true>), grid, block, 0, st, s);
    else hipLaunchKernelGGL((shrink_rows_kernel<uint16_t, false>), grid, block, 0, st, s);
  } else {
    if (s.mask) hipLaunchKernelGGL((shrink_rows_kernel<float, true>), grid, block, 0, st, s);
    else hipLaunchKernelGGL((shrink_rows_kernel<float, false>), grid, block, 0, st, s);
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || !s.big_segments) return err;
  const dim3 g2{gx, unsigned((TK + kTileTok - 1) / kTileTok), 1}, b2{256, 1, 1};
  if (s.mask) hipLaunchKernelGGL((shrink_tile_kernel<true>), g2, b2, 0, st, s);
  else hipLaunchKernelGGL((shrink_tile_kernel<false>), g2, b2, 0, st, s);
  return hipGetLastError();
}

}  // namespace lora
