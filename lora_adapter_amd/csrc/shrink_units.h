// Decode shrink as a wave-level routine, shared by its own kernel and by the
// decode GEMM launch that runs it beside the GEMM's workgroups.
// Internal to liblora (gfx950 only).
#pragma once

#include "lora_internal.h"

namespace lora {
namespace {

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

typedef __bf16 su_bf16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float dot2_bf16(uint32_t x, uint32_t a, float acc) {
  su_bf16x2_t xv, av;
  __builtin_memcpy(&xv, &x, 4);
  __builtin_memcpy(&av, &a, 4);
  return __builtin_amdgcn_fdot2_f32_bf16(xv, av, acc, false);
}

// acc + the dot product of 8 token values with 8 rank-row values, and the
// keep mask applied to the token values (exact: masked values become 0).
// bf16: v_dot2 on the packed words (each product of two bf16 is exact in
// fp32, accumulation in fp32), no conversion of either operand.
template <typename E> struct Dot8;
template <> struct Dot8<uint16_t> {
  static __device__ __forceinline__ float run(const Raw<uint16_t> &x, const Raw<uint16_t> &a, float acc) {
    acc = dot2_bf16(x.v.x, a.v.x, acc);
    acc = dot2_bf16(x.v.y, a.v.y, acc);
    acc = dot2_bf16(x.v.z, a.v.z, acc);
    acc = dot2_bf16(x.v.w, a.v.w, acc);
    return acc;
  }
  static __device__ __forceinline__ void mask(Raw<uint16_t> &x, uint2 mb) {
    uint32_t w[4] = {x.v.x, x.v.y, x.v.z, x.v.w};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t byte = ((e < 4 ? mb.x : mb.y) >> (8 * (e & 3))) & 0xffu;
      if (byte == 0) w[e >> 1] &= (e & 1) ? 0x0000ffffu : 0xffff0000u;
    }
    x.v = make_uint4(w[0], w[1], w[2], w[3]);
  }
};
template <> struct Dot8<float> {
  static __device__ __forceinline__ float run(const Raw<float> &x, const Raw<float> &a, float acc) {
    float xv[8], av[8];
    x.to8(xv);
    a.to8(av);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc = fmaf(xv[e], av[e], acc);
    return acc;
  }
  static __device__ __forceinline__ void mask(Raw<float> &x, uint2 mb) {
    float v[8];
    x.to8(v);
#pragma unroll
    for (int e = 0; e < 8; ++e)
      if ((((e < 4 ? mb.x : mb.y) >> (8 * (e & 3))) & 0xffu) == 0) v[e] = 0.f;
    x.a = make_float4(v[0], v[1], v[2], v[3]);
    x.b = make_float4(v[4], v[5], v[6], v[7]);
  }
};

// Decode shrink.  Its work is a list of units (segment, group of kShrinkRows
// rank rows, pair), counted per segment as pairs x groups and numbered group
// by group; the plan splits them into equal runs, one per wave of a fixed
// grid of kShrinkWaves waves, and records each run's first segment, unit and
// descriptor.  A wave therefore starts with one load, then per group of rank
// rows: one lane-parallel load of the page ids and of the control words of up
// to 64 pairs (token, gate, U offset), then the group's A rows go into
// registers (when d fits in kCh x 512 elements) and the token rows of its
// pairs stream through, the next pair's row in flight while the current one
// is reduced.  A segment with many pairs is thus spread over as many waves as
// its work needs, with no idle grid slots.
template <typename E, bool kMask, int kCh, bool kResident>
__device__ __forceinline__ void shrink_units_wave(const ShrinkArgs &s, const int wv) {
  constexpr int RW = kShrinkRows;
  constexpr int KB = kCh * 512;                 // elements per d-block
  const int lane = threadIdx.x & 63;
  // round trip 1: this wave's start (lanes 0-7) and header words (lanes 8-10)
  int v = 0;
  if (lane < 8) v = reinterpret_cast<const int *>(s.plan.wave_start)[8 * wv + lane];
  else if (lane == 8) v = s.plan.hdr[kPhUnits];
  else if (lane == 9) v = s.plan.hdr[kPhUnitsPerWave];
  else if (lane == 10) v = s.plan.hdr[LORA_PH_RPAIRS];
  else if (lane == 11) v = s.plan.hdr[kPhSched];
  else if (lane == 12) v = s.plan.hdr[LORA_PH_SEGS];
  if (int64_t(__builtin_amdgcn_readlane(v, 10)) > s.out_cap) {
    if (wv == 0 && lane == 0) atomicOr(s.err_word, LORA_DEVERR_CAPACITY);
    return;
  }
  const int units = __builtin_amdgcn_readlane(v, 8), upw = __builtin_amdgcn_readlane(v, 9);
  // only waves with work have a start record (this plan's, not a stale one)
  if (int64_t(wv) * upw >= units) return;
  int seg, loc, ad, r, ps, pb, pe;
  if (__builtin_amdgcn_readlane(v, 11) != 0) {
    seg = __builtin_amdgcn_readlane(v, 0);
    loc = __builtin_amdgcn_readlane(v, 1);
    ad = __builtin_amdgcn_readlane(v, 2);
    r = __builtin_amdgcn_readlane(v, 3);
    ps = __builtin_amdgcn_readlane(v, 4);
    pb = __builtin_amdgcn_readlane(v, 5);
    pe = __builtin_amdgcn_readlane(v, 6);
  } else {
    // no wave records in this plan: the last segment whose first unit is
    // <= this wave's first unit u0, by a 64-way search over the segments'
    // first units (seg_uoff[0] = 0 <= u0, seg_uoff[S] = units > u0)
    const int S = __builtin_amdgcn_readlane(v, 12);
    const int u0 = wv * upw;
    int lo = 0, first = 0, step = 1;
    while (int64_t(step) * 64 <= S) step *= 64;
    for (; step > 0; step /= 64) {
      const int idx = lo + lane * step;
      const int val = s.plan.seg_uoff[min(idx, S)];
      const uint64_t m = __ballot(idx <= S && val <= u0);
      const int last = 63 - __clzll(static_cast<long long>(m));
      first = __shfl(val, last, 64);
      lo += last * step;
    }
    seg = lo;
    loc = u0 - first;
    int w2 = 0;
    if (lane < 8) w2 = reinterpret_cast<const int *>(s.plan.seg_desc)[8 * seg + lane];
    ad = __builtin_amdgcn_readlane(w2, 0);
    r = __builtin_amdgcn_readlane(w2, 1);
    ps = __builtin_amdgcn_readlane(w2, 2);
    pb = __builtin_amdgcn_readlane(w2, 3);
    pe = __builtin_amdgcn_readlane(w2, 4);
  }
  int left = min(upw, units - wv * upw);
  const int d = s.d;
  const E *Z = static_cast<const E *>(s.Z);
  const E *pages = static_cast<const E *>(s.pages);

  while (left > 0) {
    const int n = pe - pb;
    const int G = (r + RW - 1) / RW;
    // the MFMA shrink takes the whole 32-pair tiles of a big segment: the
    // units cover its last n % 32 pairs only (every pair of a small one)
    const int n_tiled = s.big_segments && n >= kBigSegPairs ? n / kTileTok * kTileTok : 0;
    const int nu = n - n_tiled;
    const int here = min(left, nu * G - loc);
    int g = here > 0 ? loc / nu : 0, i = here > 0 ? loc % nu : 0;
    int rem = here;
    while (rem > 0) {
      const int j0 = g * RW, nr = min(RW, r - j0);
      const int i_end = min(nu, i + rem);
      for (int ib = i; ib < i_end; ib += 64) {
        const int nb = min(64, i_end - ib);
        // round trip 2: page ids (lanes < RW), scale (lane RW), and per pair
        // of this block (one per lane): token row, gate, U offset
        int pw = 0;
        float scw = 0.f;
        if (lane < RW) pw = s.page_ids[ps + j0 + min(lane, nr - 1)];
        else if (lane == RW) scw = s.scale[ad];
        const int q = pb + n_tiled + ib + min(lane, nb - 1);
        const int tkl = s.plan.pair_tk[q];
        const float gl = s.plan.pair_gate[q];
        const int ul = s.plan.u_off[q];
        const int rowl = tkl / s.K;
        const float scale =
            __int_as_float(__builtin_amdgcn_readlane(__float_as_int(scw), RW)) * s.extra_scale;
        const E *arow[RW];
#pragma unroll
        for (int a2 = 0; a2 < RW; ++a2)
          arow[a2] = pages + int64_t(__builtin_amdgcn_readlane(pw, a2)) * d;

        // one pair: dot its token row with the group's rank rows, reduce, store
        auto finish = [&](float (&acc)[RW], int k) {
#pragma unroll
          for (int a2 = 0; a2 < RW; ++a2) acc[a2] = wave_sum(acc[a2]);
          const float coef = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(gl), k)) * scale;
          const int uo = __builtin_amdgcn_readlane(ul, k);
          if (lane < nr) {
            float mine = acc[0];
#pragma unroll
            for (int a2 = 1; a2 < RW; ++a2)
              if (lane == a2) mine = acc[a2];
            s.out[uo + j0 + lane] = coef * mine;
          }
        };
        if constexpr (kResident) {
          // d <= KB: the group's rank rows stay in registers for all pairs
          Raw<E> ar[RW][kCh];
#pragma unroll
          for (int ch = 0; ch < kCh; ++ch) {
            const int c = min(ch * 512 + lane * 8, d - 8);
#pragma unroll
            for (int a2 = 0; a2 < RW; ++a2) ar[a2][ch].load(arow[a2] + c);
          }
          Raw<E> xa[kCh], xb[kCh];
          uint2 ma[kCh], mb[kCh];
          auto load_x = [&](Raw<E> (&x)[kCh], uint2 (&m)[kCh], int k) {
            const int64_t t = __builtin_amdgcn_readlane(rowl, k);
#pragma unroll
            for (int ch = 0; ch < kCh; ++ch) {
              const int c = min(ch * 512 + lane * 8, d - 8);
              x[ch].load(Z + t * d + c);
              if (kMask) m[ch] = *reinterpret_cast<const uint2 *>(s.mask + t * d + c);
            }
          };
          auto dot = [&](const Raw<E> (&x)[kCh], const uint2 (&m)[kCh], float (&acc)[RW]) {
#pragma unroll
            for (int a2 = 0; a2 < RW; ++a2) acc[a2] = 0.f;
#pragma unroll
            for (int ch = 0; ch < kCh; ++ch) {
              if (ch * 512 + lane * 8 >= d) continue;
              Raw<E> xv = x[ch];
              if (kMask) Dot8<E>::mask(xv, m[ch]);
#pragma unroll
              for (int a2 = 0; a2 < RW; ++a2) acc[a2] = Dot8<E>::run(xv, ar[a2][ch], acc[a2]);
            }
          };
          // pairs two at a time: the other buffer's token row is always in
          // flight (clamped to the last pair, so no load sits behind a branch)
          load_x(xa, ma, 0);
          for (int k = 0; k < nb; k += 2) {
            load_x(xb, mb, min(k + 1, nb - 1));
            float acc[RW];
            dot(xa, ma, acc);
            finish(acc, k);
            load_x(xa, ma, min(k + 2, nb - 1));
            if (k + 1 < nb) {
              dot(xb, mb, acc);
              finish(acc, k + 1);
            }
          }
        } else {
          // wide rows: blocks of KB elements, rank rows re-read per pair (L2)
          for (int k = 0; k < nb; ++k) {
            const int64_t t = __builtin_amdgcn_readlane(rowl, k);
            float acc[RW];
#pragma unroll
            for (int a2 = 0; a2 < RW; ++a2) acc[a2] = 0.f;
            for (int cb = 0; cb < d; cb += KB) {
              Raw<E> ar[RW][kCh], xr[kCh];
              uint2 mk[kCh];
#pragma unroll
              for (int ch = 0; ch < kCh; ++ch) {
                const int c = min(cb + ch * 512 + lane * 8, d - 8);
#pragma unroll
                for (int a2 = 0; a2 < RW; ++a2) ar[a2][ch].load(arow[a2] + c);
                xr[ch].load(Z + t * d + c);
                if (kMask) mk[ch] = *reinterpret_cast<const uint2 *>(s.mask + t * d + c);
              }
#pragma unroll
              for (int ch = 0; ch < kCh; ++ch) {
                if (cb + ch * 512 + lane * 8 >= d) continue;
                Raw<E> xv = xr[ch];
                if (kMask) Dot8<E>::mask(xv, mk[ch]);
#pragma unroll
                for (int a2 = 0; a2 < RW; ++a2) acc[a2] = Dot8<E>::run(xv, ar[a2][ch], acc[a2]);
              }
            }
            finish(acc, k);
          }
        }
      }
      rem -= i_end - i;
      i = 0;
      ++g;
    }
    left -= here;
    if (left <= 0) break;
    // the run continues in the next segment: its descriptor
    ++seg;
    loc = 0;
    int w2 = 0;
    if (lane < 8) w2 = reinterpret_cast<const int *>(s.plan.seg_desc)[8 * seg + lane];
    ad = __builtin_amdgcn_readlane(w2, 0);
    r = __builtin_amdgcn_readlane(w2, 1);
    ps = __builtin_amdgcn_readlane(w2, 2);
    pb = __builtin_amdgcn_readlane(w2, 3);
    pe = __builtin_amdgcn_readlane(w2, 4);
  }
}

// Per-slot decode shrink, no plan needed (each slot gathers its own
// adapter's rank rows, so the launch that builds the plan can run it too).
// Four workgroups (4 waves each) per slot i = t*K + k: part q, wave w takes
// rank rows 4q + w, 4q + w + 16, ..., one row at a time with every load of
// the row (token row and A page) in one round trip, so the slot's rows go
// out from 16 waves at once.  Each lane adds its 16-byte chunks in
// ascending order with v_dot2, then the wave sum and coef = gate . (scale .
// extra): the same operations in the same order as shrink_units_wave, so U
// is identical to the plan-driven shrink's.
//
// Part 0's first wave also writes the slot's descriptor for the epilogue:
// active when its id is in range, its gate is not 0, its adapter's rank is
// in 1..LORA_MAX_RANK with a consistent page_start and every page id in
// range (the plan's rule for keeping a slot).
constexpr int kSlotParts = 4;    // workgroups per slot

template <bool kMask>
__device__ __forceinline__ void slot_shrink_part(const SlotShrinkArgs &s, const int i, const int q) {
  constexpr int kCh = 4;                        // 512-element chunks per load batch
  constexpr int KB = kCh * 512;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int id = s.ids[i];
  const float gate = s.gates[i];
  int r = 0, ps = 0;
  bool act = id >= 0 && id < s.N && gate != 0.0f && s.n_pages > 0;
  if (act) {
    r = s.rank[id];
    ps = s.page_start[id];
    const int pe = s.page_start[id + 1];
    act = r > 0 && r <= LORA_MAX_RANK && ps >= 0 && int64_t(pe) - ps == r && pe <= s.n_page_ids;
  }
  if (!act) {
    if (q == 0 && threadIdx.x == 0) s.sdesc[i] = make_int4(-1, 0, 0, 0);
    return;
  }
  if (q == 0 && w == 0) {
    // every page id of the adapter in range (lane-parallel), then the
    // descriptor; the other waves only guard their own loads
    bool bad = false;
    for (int j = lane; j < r; j += 64) {
      const int pid = s.page_ids[ps + j];
      bad |= pid < 0 || pid >= s.n_pages;
    }
    const bool any_bad = __ballot(bad) != 0;
    if (lane == 0)
      s.sdesc[i] = any_bad ? make_int4(-1, 0, 0, 0) : make_int4(i, r, i * s.stride, ps);
  }
  const float coef = gate * (s.scale[id] * s.extra_scale);
  const int d = s.d;
  const int64_t t = i / s.K;
  const uint16_t *zrow = static_cast<const uint16_t *>(s.Z) + t * d;
  const uint8_t *mrow = kMask ? s.mask + t * d : nullptr;
  const uint16_t *pages = static_cast<const uint16_t *>(s.pages);
  for (int j = kSlotParts * q + w; j < r; j += 4 * kSlotParts) {
    const int pid = s.page_ids[ps + j];
    const bool in = pid >= 0 && pid < s.n_pages;
    const uint16_t *arow = pages + int64_t(in ? pid : 0) * d;
    float acc = 0.f;
    for (int cb = 0; cb < d; cb += 2 * KB) {
      // two batches of kCh chunks in flight, added in ascending order
      Raw<uint16_t> ar[2 * kCh], xr[2 * kCh];
      uint2 mk[2 * kCh];
#pragma unroll
      for (int ch = 0; ch < 2 * kCh; ++ch) {
        const int c = min(cb + ch * 512 + lane * 8, d - 8);
        xr[ch].load(zrow + c);
        if (kMask) mk[ch] = *reinterpret_cast<const uint2 *>(mrow + c);
        ar[ch].load(arow + c);
      }
#pragma unroll
      for (int ch = 0; ch < 2 * kCh; ++ch) {
        if (cb + ch * 512 + lane * 8 >= d) continue;
        Raw<uint16_t> xv = xr[ch];
        if (kMask) Dot8<uint16_t>::mask(xv, mk[ch]);
        acc = Dot8<uint16_t>::run(xv, ar[ch], acc);
      }
    }
    acc = wave_sum(acc);
    if (lane == 0 && in) s.out[int64_t(i) * s.stride + j] = coef * acc;
  }
}

}  // namespace
}  // namespace lora
