// Base GEMM Y = X.W with the LoRA expand in its epilogue.
//
// S-LoRA (section 批处理) batches the base-model product over all requests
// and adds each request's x.A.B separately without padding; LoRAFusion
// (section Kernel 层：图分裂融合) keeps the compute-bound GEMM main loop intact
// and consumes the small A.X intermediate in place.  Here the main loop is a
// plain gfx950 bf16 MFMA GEMM (v_mfma_f32_32x32x16_bf16, fp32 accumulators,
// both operands K-contiguous: X[M][K] and W_t[N][K]); the expand
//   acc[t][n] += sum over t's planned pairs p, rank rows j:  U[u_off[p]+j] . B_a[j][n]
// is added to the fp32 accumulators of each output tile before the single
// rounding to the output dtype, so the main loop never sees the adapters.
//
// Two epilogue placements, chosen from the shape:
//   * fused: when the tile grid alone fills the GPU (prefill), each tile
//     adds the expand to its accumulators (MFMA blocks for rank <= 16, one
//     slot per token; row by row with the adapter's B slice cached in
//     registers otherwise), stages them through LDS and stores; the input
//     gradient uses the same epilogue with its keep mask on the LoRA term;
//   * split-K: decode shapes have too few output tiles to stream W at full
//     bandwidth, so K is split across workgroups that write fp32 partial
//     products; the epilogue kernel then sums the partials in a fixed order,
//     adds the expand with wide (512-column) coalesced B-row reads, rounds
//     and stores.  The reduction order is fixed: results are deterministic,
//     and rows without active slots equal the base-only result bit for bit.
#include "lora_internal.h"
#include "plan_build.h"
#include "shrink_units.h"

namespace lora {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

// ------------------------------------------------------------ vector loads/stores
template <typename E, int CPL> struct Cols;
template <> struct Cols<uint16_t, 1> {
  static __device__ __forceinline__ void load(const uint16_t *p, float v[1]) { v[0] = bf2f(*p); }
  static __device__ __forceinline__ void store(uint16_t *p, const float v[1]) { *p = f2bf(v[0]); }
};
template <> struct Cols<uint16_t, 2> {
  static __device__ __forceinline__ void load(const uint16_t *p, float v[2]) {
    const uint32_t w = *reinterpret_cast<const uint32_t *>(p);
    v[0] = bf_lo(w); v[1] = bf_hi(w);
  }
  static __device__ __forceinline__ void store(uint16_t *p, const float v[2]) {
    *reinterpret_cast<uint32_t *>(p) = f2bf2(v[0], v[1]);
  }
};
template <> struct Cols<uint16_t, 8> {
  static __device__ __forceinline__ void load(const uint16_t *p, float v[8]) { Elem<uint16_t>::load8(p, v); }
  static __device__ __forceinline__ void store(uint16_t *p, const float v[8]) {
    uint4 w;
    w.x = f2bf2(v[0], v[1]);
    w.y = f2bf2(v[2], v[3]);
    w.z = f2bf2(v[4], v[5]);
    w.w = f2bf2(v[6], v[7]);
    *reinterpret_cast<uint4 *>(p) = w;
  }
};
// 8 bf16 values, one 16-byte streaming store (Y is written once and not
// read back by the layer)
__device__ __forceinline__ void store8_nt(uint16_t *p, const float v[8]) {
  typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
  u32x4_t w;
  w.x = f2bf2(v[0], v[1]);
  w.y = f2bf2(v[2], v[3]);
  w.z = f2bf2(v[4], v[5]);
  w.w = f2bf2(v[6], v[7]);
  __builtin_nontemporal_store(w, reinterpret_cast<u32x4_t *>(p));
}
template <> struct Cols<float, 8> {
  static __device__ __forceinline__ void load(const float *p, float v[8]) { Elem<float>::load8(p, v); }
  static __device__ __forceinline__ void store(float *p, const float v[8]) {
    *reinterpret_cast<float4 *>(p) = make_float4(v[0], v[1], v[2], v[3]);
    *reinterpret_cast<float4 *>(p + 4) = make_float4(v[4], v[5], v[6], v[7]);
  }
};

__device__ __forceinline__ void load_f8(const float *p, float v[8]) { Elem<float>::load8(p, v); }

// ------------------------------------------------------------ expand of one row
// v[c] += sum over the row's active slots k (in slot order) and rank rows j
// (ascending) of U[u_off[p] + j] * B_a[j][col + c].  Wave-uniform control flow:
// every lane handles the same row; lanes own consecutive columns.  `col` must
// be a valid column (callers clamp it and mask their store), so the B loads
// are unconditional and eight of them are in flight at a time.
// 8 consecutive elements held raw until used, so a batch of loads is in
// flight before the first conversion waits.
template <typename E> struct Raw8;
template <> struct Raw8<uint16_t> {
  uint4 v;
  __device__ __forceinline__ void load(const uint16_t *p) { v = *reinterpret_cast<const uint4 *>(p); }
  __device__ __forceinline__ void to8(float o[8]) const { Elem<uint16_t>::load8(reinterpret_cast<const uint16_t *>(&v), o); }
};
template <> struct Raw8<float> {
  float4 a, b;
  __device__ __forceinline__ void load(const float *p) {
    a = *reinterpret_cast<const float4 *>(p);
    b = *reinterpret_cast<const float4 *>(p + 4);
  }
  __device__ __forceinline__ void to8(float o[8]) const {
    o[0] = a.x; o[1] = a.y; o[2] = a.z; o[3] = a.w; o[4] = b.x; o[5] = b.y; o[6] = b.z; o[7] = b.w;
  }
};

// One row, 8 columns per lane.  Control data is gathered lane-parallel and
// broadcast: the row's slot descriptors ({pair, rank, u_off, page_start},
// lane k = slot k; the caller loads them, so their round trip can overlap
// its own loads), then the page ids and U values of up to 64 rank rows (lane
// j = row j), then the B rows stream in batches of 8, the next batch in
// flight while the current one is added.  Rank rows are added in ascending
// order, slot by slot.
template <typename E>
__device__ __forceinline__ int4 expand_row_desc(int t, const ExpandArgs &e) {
  int4 sd = make_int4(-1, 0, 0, 0);
  if (lane_id() < e.K) sd = e.slot_desc[t * e.K + lane_id()];
  return sd;
}

template <typename E>
__device__ __forceinline__ void expand_row8(float (&v)[8], int4 sd, int col, const ExpandArgs &e) {
  constexpr int NB = 8;                  // B rows per batch; two batches in flight
  const E *B = static_cast<const E *>(e.b_pages);
  const int lane = lane_id();
  for (int k = 0; k < e.K; ++k) {
    // the slot's descriptor, the same in every lane: scalar registers, so
    // that the loops below branch uniformly
    if (__builtin_amdgcn_readfirstlane(__shfl(sd.x, k, 64)) < 0) continue;
    const int r = __builtin_amdgcn_readfirstlane(__shfl(sd.y, k, 64));
    const int uo = __builtin_amdgcn_readfirstlane(__shfl(sd.z, k, 64));
    const int ps = __builtin_amdgcn_readfirstlane(__shfl(sd.w, k, 64));
    for (int jb = 0; jb < r; jb += 64) {
      const int nrb = min(64, r - jb);
      const int jl = jb + min(lane, nrb - 1);
      const int pid = e.page_ids[ps + jl];
      const float uv = e.U[uo + jl];
      Raw8<E> ba[NB], bb[NB];
      auto loadb = [&](Raw8<E> (&dst)[NB], int q0) {
#pragma unroll
        for (int q = 0; q < NB; ++q)
          dst[q].load(B + int64_t(__shfl(pid, min(q0 + q, nrb - 1), 64)) * e.d_out + col);
      };
      auto addb = [&](const Raw8<E> (&src)[NB], int q0) {
#pragma unroll
        for (int q = 0; q < NB; ++q) {
          if (q0 + q < nrb) {
            float b[8];
            src[q].to8(b);
            const float uj = __shfl(uv, q0 + q, 64);
#pragma unroll
            for (int c = 0; c < 8; ++c) v[c] = fmaf(uj, b[c], v[c]);
          }
        }
      };
      // both batches' loads are issued unconditionally (rows past nrb
      // re-read row nrb - 1, a cache hit, and are not added): a load under
      // a condition leaves the compiler unable to count what is in flight,
      // and it then waits for every load, the batch just issued included
      loadb(ba, 0);
      for (int q0 = 0; q0 < nrb; q0 += 2 * NB) {
        loadb(bb, q0 + NB);
        addb(ba, q0);
        loadb(ba, q0 + 2 * NB);
        addb(bb, q0 + NB);
      }
    }
  }
}

// Same sums in the same order, with the B slice of the last page range (rank
// <= RB) kept in registers: consecutive prefill rows usually share an adapter.
template <int CPL, int RB>
struct BCache {
  int ps, r;
  float b[RB][CPL];
};

template <int CPL, int RB>
__device__ __forceinline__ void expand_row_cached(float (&v)[CPL], int t, int col,
                                                  const ExpandArgs &e, BCache<CPL, RB> &cache) {
  const uint16_t *B = static_cast<const uint16_t *>(e.b_pages);
  for (int k = 0; k < e.K; ++k) {
    const int4 sd = e.slot_desc[t * e.K + k];
    if (sd.x < 0) continue;
    const int r = sd.y;
    const float *u = e.U + sd.z;
    const int32_t *pid = e.page_ids + sd.w;
    if (r <= RB) {
      if (sd.w != cache.ps || r != cache.r) {
        // rows past r reload row r-1; they are never used
#pragma unroll
        for (int j = 0; j < RB; ++j)
          Cols<uint16_t, CPL>::load(B + int64_t(pid[min(j, r - 1)]) * e.d_out + col, cache.b[j]);
        cache.ps = sd.w;
        cache.r = r;
      }
#pragma unroll
      for (int j = 0; j < RB; ++j) {
        if (j < r) {
          const float uj = u[j];
#pragma unroll
          for (int c = 0; c < CPL; ++c) v[c] = fmaf(uj, cache.b[j][c], v[c]);
        }
      }
    } else {
      for (int j = 0; j < r; ++j) {
        float bv[CPL];
        Cols<uint16_t, CPL>::load(B + int64_t(pid[j]) * e.d_out + col, bv);
        const float uj = u[j];
#pragma unroll
        for (int c = 0; c < CPL; ++c) v[c] = fmaf(uj, bv[c], v[c]);
      }
    }
  }
}

__device__ __forceinline__ bool expand_enabled(const ExpandArgs &e) {
  return e.U != nullptr && int64_t(e.hdr[LORA_PH_RPAIRS]) <= e.u_cap;
}

// ------------------------------------------------------------ LDS copies and waits
// LDS byte address of a __shared__ object.
__device__ __forceinline__ uint32_t lds_addr(const void *p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>(
      (const __attribute__((address_space(3))) char *)(p)));
}

// global_load_lds_dwordx4: each of the 64 lanes copies 16 bytes from its
// global address to LDS at lds + 16 * lane.  Issued from inline asm so that
// the compiler does not put a blanket vmcnt(0) in front of every later LDS
// read (it cannot tell which LDS stage an in-flight copy writes); the
// instruction has no register result, and the kernel waits for these copies
// itself (wait_vmcnt) before the barrier that precedes reading the stage.
// On this architecture family an LDS DMA needs one wait state after a
// scalar write of m0, which the compiler cannot insert inside the asm
// block: the s_nop provides it.
__device__ __forceinline__ void lds_dma16(const void *gptr, uint32_t lds) {
  const uint32_t lds_s = __builtin_amdgcn_readfirstlane(lds);   // wave-uniform LDS base
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(gptr), "s"(lds_s)
               : "memory", "m0");
}

// s_waitcnt with only vmcnt constrained (gfx9 encoding: vmcnt bits 3:0 and 15:14).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Workgroup barrier for LDS only.  The stage copies are LDS DMA issued from
// inline asm, so every wave first waits (wait_vmcnt) for its own copies of a
// stage and then meets the others here; no global load in flight is waited
// for (__syncthreads() waits for all of them).
__device__ __forceinline__ void lds_bar() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// ------------------------------------------------------------ decode GEMM
// Few tokens (M <= 128): the product is a stream of W (d_in x d_out bf16)
// through HBM, and every W byte is used by one wave only.  A workgroup owns
// 128 output columns (32 per wave) and KC = 512 of K, and issues its whole
// W share at once, straight into the MFMA B-operand registers (32 loads of
// 16 bytes per lane, nothing staged in LDS), so a 1-workgroup-per-CU grid
// keeps ~128 KiB per CU in flight.  The token rows (shared by the 4 waves)
// go through LDS.  K is permuted inside each 64-wide group so that a lane's
// W loads are 64 contiguous bytes: in step s, lanes 0-31 contract k = 8s..8s+7
// and lanes 32-63 k = 32+8s..32+8s+7; the X fragments read from LDS use the
// same permutation, so the sum is unchanged.  Partial sums of the K splits go
// to the workspace for the epilogue kernel.
constexpr int kDecodeKC = 512;   // K elements per decode workgroup

// One decode tile: columns bx*128 .. +127, token rows by*32*MB .., K chunk bz.
// xs: LDS of MB*32*kDecodeKC bf16 for the token rows.
template <int MB>
__device__ __forceinline__ void decode_tile(const GemmArgs &g, int bx, int by, int bz,
                                            uint16_t *xs) {
  constexpr int KC = kDecodeKC;
  constexpr int NG = KC / 64;                 // 64-wide K groups
  constexpr int BMr = MB * 32;
  // One token row of the K chunk = 64 slots of 16 bytes.  Row r keeps chunk c
  // in slot c ^ (r & 15): the 16 rows that one quarter of a wave's fragment
  // read touches at once (same chunk) cover the 64 banks exactly once.
  const uint16_t *X = static_cast<const uint16_t *>(g.X);
  const uint16_t *W = static_cast<const uint16_t *>(g.W);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n0 = bx * 128 + wave * 32;
  const int m0 = by * BMr;
  const int k0 = bz * KC;
  const int ng = min(NG, (g.Kd - k0) / 64);
  const int half = lane >> 5;

  // All loads are unconditional, from clamped addresses, so none waits on a
  // branch: rows past M and columns past N only feed outputs that are never
  // stored, and K groups past the end are skipped by the MFMA loop.
  // The token rows (mostly L2) go first, straight into LDS: wave w copies
  // rows w, w+4, ...; lane l of a copy fills slot l of the row.  The copies
  // are issued from inline asm, so the compiler does not hold every LDS read
  // until all loads have landed; the W stream (HBM) follows, and the MFMAs
  // of each 64-wide K group start as soon as its W fragments are in.
#pragma unroll
  for (int i = 0; i < BMr / 4; ++i) {
    const int r = wave + 4 * i;
    const int row = min(m0 + r, g.M - 1);
    const int chunk = lane ^ (r & 15);
    const int col = min(chunk * 8, ng * 64 - 8);
    lds_dma16(X + int64_t(row) * g.Kd + k0 + col, lds_addr(xs + r * KC));
  }
  // W fragments: row n0 + lane%32, k0 + 64*grp + 32*half + [0, 32)
  uint4 wf[NG][4];
  const uint16_t *wrow = W + int64_t(min(n0 + (lane & 31), g.N - 1)) * g.Kd + k0 + half * 32;
#pragma unroll
  for (int gq = 0; gq < NG; ++gq)
#pragma unroll
    for (int q = 0; q < 4; ++q)
      wf[gq][q] = *reinterpret_cast<const uint4 *>(wrow + min(gq, ng - 1) * 64 + q * 8);
  __builtin_amdgcn_sched_barrier(0);
  wait_vmcnt<NG * 4>();   // this wave's token rows have landed (its W loads came after them)
  lds_bar();              // and every wave's
  f32x16_t acc[MB];
#pragma unroll
  for (int b = 0; b < MB; ++b)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[b][v] = 0.f;
#pragma unroll
  for (int gq = 0; gq < NG; ++gq) {
    if (gq < ng) {
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        bf16x8_t bfrag;
        __builtin_memcpy(&bfrag, &wf[gq][s], 16);
#pragma unroll
        for (int b = 0; b < MB; ++b) {
          const int r = b * 32 + (lane & 31);
          const int chunk = (gq * 64 + half * 32 + s * 8) / 8;
          const bf16x8_t afrag =
              *reinterpret_cast<const bf16x8_t *>(xs + r * KC + ((chunk ^ (r & 15)) * 8));
          acc[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(afrag, bfrag, acc[b], 0, 0, 0);
        }
      }
    }
  }
  // partials are read once, by the epilogue: streaming (non-temporal) stores
  float *Pz = g.partial + int64_t(bz) * g.M * g.N;
  const int col = n0 + (lane & 31);
  if (col < g.N) {
#pragma unroll
    for (int b = 0; b < MB; ++b)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int row = m0 + b * 32 + (v >> 2) * 8 + half * 4 + (v & 3);
        if (row < g.M) __builtin_nontemporal_store(acc[b][v], Pz + int64_t(row) * g.N + col);
      }
  }
}

template <int MB>
__global__ __launch_bounds__(256) void gemm_decode_kernel(GemmArgs g) {
  __shared__ __attribute__((aligned(16))) uint16_t xs[MB * 32 * kDecodeKC];
  decode_tile<MB>(g, blockIdx.x, blockIdx.y, blockIdx.z, xs);
}

// Decode GEMM and decode shrink in one launch.  Workgroups [0, n_gemm) are
// GEMM tiles (bx fastest, then by, then bz); the others run the shrink
// schedule, one schedule wave per wave, striding over all kShrinkWaves.  The
// two halves stream disjoint HBM data (W, A pages) side by side and share
// the token rows through L2, and the shrink no longer costs a launch of its
// own on the decode critical path.
template <int MB, bool kMask, int kCh>
__global__ __launch_bounds__(256, 2) void decode_gemm_shrink_kernel(GemmArgs g, ShrinkArgs s,
                                                                 int gx, int gy, int n_gemm) {
  __shared__ __attribute__((aligned(16))) uint16_t xs[MB * 32 * kDecodeKC];
  const int b = blockIdx.x;
  if (b < n_gemm) {
    decode_tile<MB>(g, b % gx, (b / gx) % gy, b / (gx * gy), xs);
    return;
  }
  const int nsw = (int(gridDim.x) - n_gemm) * 4;
  for (int w = (b - n_gemm) * 4 + (threadIdx.x >> 6); w < kShrinkWaves; w += nsw)
    shrink_units_wave<uint16_t, kMask, kCh, true>(s, w);
}

// Workgroup 0 builds the plan, workgroups 1 .. n_gemm are the decode GEMM
// tiles, the per-slot shrink parts (four per slot) follow.  No part reads
// what another writes, and neither the shrink nor the GEMM needs the plan.
// GEMM tiles first: they are dispatched one per CU whatever the shrink does.
// With the shrink parts first, a batch whose slots are all inactive (parts
// that end at once) had its tiles packed unevenly onto CUs: the q_proj
// decode batch (64 tokens, 4096 -> 4096, 64 rank-16 adapters) with an empty
// plan took 22.3 us per step against 17.3 us this way, and
// the full step is the same either way (21.9 us).
template <int MB, bool kMask, bool kLds>
__global__ __launch_bounds__(256) void decode_gemm_slot_kernel(GemmArgs g, SlotShrinkArgs ss,
                                                                PlanArgs pa, int gx, int gy,
                                                                int n_gemm) {
  __shared__ __attribute__((aligned(16))) uint16_t xs[MB * 32 * kDecodeKC];
  const int b = int(blockIdx.x);
  if (b == 0) {
    // the plan, in the LDS the GEMM tiles use for token rows; dispatched
    // first, so its one global round trip goes out ahead of the W stream
    plan_build<kLds>(pa, reinterpret_cast<int *>(xs));
    return;
  }
  if (b - 1 < n_gemm) {
    const int t = b - 1;
    decode_tile<MB>(g, t % gx, (t / gx) % gy, t / (gx * gy), xs);
    return;
  }
  slot_shrink_part<kMask>(ss, (b - 1 - n_gemm) / kSlotParts, (b - 1 - n_gemm) % kSlotParts);
}

// ------------------------------------------------------------ pipelined tile GEMM
// The main GEMM for more than 128 tokens.  Tile BM x BN, K step 64, WM x WN
// waves each owning (BM/WM) x (BN/WN) as 32x32x16 MFMA blocks.  The 256 x 256
// tile runs 8 waves (2 x 4, each 128 x 64; two per SIMD, so one wave's
// waits are covered by the other's MFMAs), measured about 1-2 % faster
// than 4 waves of 128 x 128 on the prefill product and its input gradient
// despite 1.5x the fragment reads per MFMA; the stream-K 256 x 128 tile runs 4.
//   * Operands go global -> LDS with global_load_lds_dwordx4 (no VGPR
//     staging): one instruction moves 8 tile rows of 128 bytes.  Two LDS
//     stages; the loads of K tile kt+1 are in flight while tile kt feeds the
//     MFMAs, and explicit vmcnt waits release each stage.
//   * In LDS a tile row (128 bytes) keeps 16-byte chunk c in slot
//     tswz(row, c) = c ^ (row & 7) ^ ((row >> 3) & 1): the 16 rows that one
//     quarter of a wave's fragment read touches at once (same chunk) cover
//     the 64 banks exactly once.  With c ^ (row & 7) alone, rows r and r + 8
//     collide, and every fragment read took two passes.
//   * Tiles are ordered so that the workgroups the hardware places on one XCD
//     (workgroup ids equal mod 8) take consecutive tiles, walked 4 tile rows at
//     a time: concurrently running tiles on an XCD share X rows and W columns
//     through that XCD's L2.
// LDS slot of 16-byte chunk c (0..7) in tile row `row`.
__device__ __forceinline__ int tswz(int row, int c) { return c ^ (row & 7) ^ ((row >> 3) & 1); }

template <int BM, int BN, int WM, int WN>
struct TileCfg {
  static constexpr int NW = WM * WN, NT = NW * 64;
  static constexpr int ROWB = 128;                        // bytes per 64-wide K row
  static constexpr int STAGE = (BM + BN) * ROWB;          // bytes per LDS stage
  static constexpr int TM = BM / (WM * 32), TN = BN / (WN * 32);
  static constexpr int A_INS = BM / 8 / NW, B_INS = BN / 8 / NW;
  static constexpr int LPW = A_INS + B_INS;               // loads per wave per stage
  static_assert(A_INS * 8 * NW == BM && B_INS * 8 * NW == BN, "tile rows / waves");
  static_assert(LPW < 64, "vmcnt field holds at most 63");
};

__device__ __forceinline__ void tile_coords(int T, int tiles_m, int tiles_n, int &tm, int &tn) {
  constexpr int G = 4;
  const int gsize = G * tiles_n;
  const int grp = T / gsize;
  const int first = grp * G;
  const int gm = min(G, tiles_m - first);
  const int in = T - grp * gsize;
  tm = first + in % gm;
  tn = in / gm;
}

// Operands of the fused epilogue's MFMA expand that do not depend on the
// product: the slot descriptors of the tile's rows and the page ids of the
// first adapter of the wave's first block.  They are fetched while the K loop
// runs (the descriptors before its first copies, the page ids once those have
// landed); after the loop each would be a round trip of its own with the MFMA
// pipe idle.  U is not held across the loop (32 more registers would spill):
// the epilogue issues it together with the B values, one round trip for both.
template <int TM>
struct EpiPre {
  int4 sd[TM];        // slot descriptor of row frow of each 32-row block
  int pid;            // lanes 0-15: page id of rank row `lane` of (kps, kr)
  int kps, kr;        // page start and rank of block 0's first adapter (-1: none)
};

// The descriptors (none when U is absent or K > 1: those tiles take the row
// path or no LoRA term).
template <int BM, int BN, int WM, int WN>
__device__ __forceinline__ void epi_fetch_desc(const GemmArgs &g, int m0,
                                               EpiPre<TileCfg<BM, BN, WM, WN>::TM> &p) {
  constexpr int TM = TileCfg<BM, BN, WM, WN>::TM;
  const int lane = threadIdx.x & 63, wm = (threadIdx.x >> 6) / WN;
  const bool want = g.ex.U != nullptr && g.ex.K == 1;
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    const int row = m0 + wm * TM * 32 + i * 32 + (lane & 31);
    p.sd[i] = want ? g.ex.slot_desc[min(row, g.M - 1)] : make_int4(-1, 0, 0, 0);
    if (row >= g.M) p.sd[i].x = -1;
  }
  p.kps = -1;
  p.kr = -1;
  p.pid = 0;
}

// The page ids of block 0's first adapter (the load the epilogue would issue
// for it).
template <int TM>
__device__ __forceinline__ void epi_fetch_pid(const GemmArgs &g, EpiPre<TM> &p) {
  const int lane = threadIdx.x & 63;
  const unsigned long long m = __ballot(p.sd[0].x >= 0) & 0xffffffffull;
  if (m && expand_enabled(g.ex)) {
    const int leader = __ffsll(m) - 1;
    p.kps = __shfl(p.sd[0].w, leader, 64);
    p.kr = __shfl(p.sd[0].y, leader, 64);
    if (lane < 16) p.pid = g.ex.page_ids[p.kps + min(lane, p.kr - 1)];
  }
}

// Fused epilogue of a tile: add the expand to the fp32 accumulators, round
// once, store Y.
//   * One slot per token (K = 1) and ranks <= 16 -- prefill: the expand of a
//     32-row block is done by MFMAs, U_block (32 x r, fp32 split exactly into
//     bf16 hi + lo, error < 2^-16 of U) times the adapter's B slice (r x 32 per
//     MFMA block), accumulated into the base product's registers.  A block
//     spanning several adapters takes one pass per adapter, with the U rows
//     of the other adapters zero.  The B fragments of the last adapter are
//     kept, so a long segment loads them once.  The slot descriptors, U and
//     the first adapter's page ids come prefetched (EpiPre); B values are
//     the one round trip left after the K loop.
//   * Blocks with higher ranks or several slots per token add the expand row
//     by row (all lanes on one row).
//   * Every block is staged in LDS and stored with 16-byte stores when it
//     needs no row-by-row expand.
// The per-block loop is unrolled, so every block's accumulators, descriptors
// and U values are addressed by compile-time indices (a rolled loop that
// rotated the blocks down into position 0 needed 11 dwords of scratch per
// block for the rotation temporaries).
// kMask (the input gradient, whose LoRA term is multiplied by the keep mask
// g.mask [M][N]): the LoRA term is accumulated apart from the base product
// and added times the mask bytes, one rounding, as the split-K epilogue does.
// An MFMA block stages its base product first, accumulates the LoRA term in
// the same registers, and moves it through a second, 8-row staging region a
// quarter at a time; the row path keeps the term in registers of its own.
template <int BM, int BN, int WM, int WN, bool kMask>
__device__ __forceinline__ void fused_epilogue(const GemmArgs &g,
                                               f32x16_t (&acc)[TileCfg<BM, BN, WM, WN>::TM]
                                                              [TileCfg<BM, BN, WM, WN>::TN],
                                               char *lds0, char *lds1, int m0, int n0,
                                               const EpiPre<TileCfg<BM, BN, WM, WN>::TM> &pre) {
  using C = TileCfg<BM, BN, WM, WN>;
  constexpr int TM = C::TM, TN = C::TN;
  constexpr int WC = TN * 32;                // columns of this wave's sub-tile
  constexpr int SC = WC + 4;                 // staged floats per row (padded, 16-byte rows)
  constexpr int CPL = WC / 64;               // columns per lane in the row-by-row path
  static_assert(CPL == 1 || CPL == 2, "fused epilogue handles 64 or 128 columns per wave");
  static_assert(WC % 8 == 0 && 64 % (WC / 8) == 0, "16-byte store layout");
  // waves 0..NW/2-1 stage in lds0, the others in lds1
  static_assert((C::NW / 2) * (kMask ? 40 : 32) * SC * 4 <= C::STAGE, "staging must fit in LDS");
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave / WN, wn = wave % WN;
  const int frow = lane & 31, half = lane >> 5;
  const bool lora_on = expand_enabled(g.ex);
  const bool mfma_ok = lora_on && g.ex.K == 1;
  const uint16_t *Bp = static_cast<const uint16_t *>(g.ex.b_pages);

  // slot descriptor of row frow of every block (fetched during the K loop),
  // and that row's U values (rank rows 8*half .. +7), whose loads share their
  // round trip with the first B values
  const int4 (&sdv)[TM] = pre.sd;
  float uv[TM][8];
  unsigned rowwise = lora_on && !mfma_ok ? (1u << TM) - 1 : 0u;   // blocks for the row path
  if (mfma_ok) {
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const bool act = sdv[i].x >= 0;
      if (__ballot(act && sdv[i].y > 16) != 0) rowwise |= 1u << i;
      // 32 consecutive pairs of one adapter of rank 8 or 16 hold their U as
      // one run of 32 r floats: the wave loads it in 16-byte pieces (lane l
      // floats 8l .. 8l+7, i.e. row l r/8 ... ) and hands each row's values
      // to its lanes by shuffles.  Otherwise each lane loads its 8 values
      // one by one (every such load touches 16 cache lines).
      const int r0 = __shfl(sdv[i].y, 0, 64), z0 = __shfl(sdv[i].z, 0, 64);
      const int w0 = __shfl(sdv[i].w, 0, 64);
      const bool in_run = act && sdv[i].y == r0 && sdv[i].w == w0 && sdv[i].z == z0 + r0 * frow;
      const bool run = __ballot(!in_run) == 0 && (r0 == 8 || r0 == 16) &&
                       (reinterpret_cast<uintptr_t>(g.ex.U + z0) & 15) == 0;
      if (run) {
        const float4 *src = reinterpret_cast<const float4 *>(g.ex.U + z0) + 2 * min(lane, 4 * r0 - 1);
        const float4 lo4 = src[0], hi4 = src[1];
        const float v8[8] = {lo4.x, lo4.y, lo4.z, lo4.w, hi4.x, hi4.y, hi4.z, hi4.w};
        // row frow's rank rows 8*half .. +7 sit in lane frow * r/8 + half
        const int from = min(frow * (r0 / 8) + half, 63);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float x = __shfl(v8[e], from, 64);
          uv[i][e] = half * 8 < r0 ? x : 0.f;
        }
      } else {
        const int r = act ? min(sdv[i].y, 16) : 1;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int ja = half * 8 + e;
          uv[i][e] = act ? g.ex.U[sdv[i].z + min(ja, r - 1)] : 0.f;
          if (ja >= r) uv[i][e] = 0.f;
        }
      }
    }
  }

  float *stage = reinterpret_cast<float *>(wave < C::NW / 2 ? lds0 : lds1) +
                 (wave % (C::NW / 2)) * 32 * SC;
  // kMask: 8 rows of the LoRA term, past every wave's staging region
  float *lstage = reinterpret_cast<float *>(wave < C::NW / 2 ? lds0 : lds1) +
                  (C::NW / 2) * 32 * SC + (wave % (C::NW / 2)) * 8 * SC;
  uint16_t *Y = static_cast<uint16_t *>(g.Y);
  const int cbase = n0 + wn * WC;
  // row-by-row path: lane owns CPL consecutive columns
  const int col_raw = cbase + lane * CPL;
  const bool col_ok = col_raw < g.N;
  const int col = col_ok ? col_raw : g.N - CPL;     // loads stay in bounds
  // 16-byte path: lane owns 8 columns of one of 64 / (WC / 8) rows per step
  constexpr int LPR = WC / 8, RPS = 64 / LPR;
  static_assert(RPS <= 8, "the kMask quarter holds 8 rows");
  const int vr = lane / LPR, vc = (lane % LPR) * 8;
  const bool c8 = cbase + vc + 8 <= g.N;
  BCache<CPL, 16> cache;
  cache.ps = -1;
  cache.r = -1;
  int bkey_ps = -1, bkey_r = -1;             // adapter slice held in bfr
  bf16x8_t bfr[TN] = {};
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    bool lterm = false;                      // kMask: acc[i] holds the LoRA term
    if (mfma_ok && !((rowwise >> i) & 1u)) {
      // one MFMA pass per adapter present in the block (lanes 0-31 = rows)
      const int4 sd = sdv[i];
      unsigned long long pending = __ballot(sd.x >= 0) & 0xffffffffull;
      if constexpr (kMask) {
        lterm = pending != 0;
        if (lterm) {
          // the staging region is this wave's own (see below)
#pragma unroll
          for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
              const int r = (v >> 2) * 8 + half * 4 + (v & 3);
              stage[r * SC + j * 32 + frow] = acc[i][j][v];
              acc[i][j][v] = 0.f;
            }
        }
      }
      while (pending) {
        const int leader = __ffsll(pending) - 1;
        const int kps = __shfl(sd.w, leader, 64), kr = __shfl(sd.y, leader, 64);
        const bool mine = sd.x >= 0 && sd.w == kps && sd.y == kr;
        pending &= ~__ballot(mine);
        if (kps != bkey_ps || kr != bkey_r) {
          // B operand: lane (column frow of block j, rank rows 8*half .. +7)
          int pidl = 0;
          if (kps == pre.kps && kr == pre.kr) pidl = pre.pid;
          else if (lane < 16) pidl = g.ex.page_ids[kps + min(lane, kr - 1)];
#pragma unroll
          for (int j = 0; j < TN; ++j) {
            const int cj = min(n0 + wn * TN * 32 + j * 32 + frow, g.N - 1);
            uint32_t w4[4];
#pragma unroll
            for (int e = 0; e < 8; e += 2) {
              const int ja = half * 8 + e, jb = ja + 1;
              const int pa = __shfl(pidl, min(ja, 15), 64), pb = __shfl(pidl, min(jb, 15), 64);
              uint32_t lo = Bp[int64_t(pa) * g.ex.d_out + cj];
              uint32_t hi = Bp[int64_t(pb) * g.ex.d_out + cj];
              if (ja >= kr) lo = 0;
              if (jb >= kr) hi = 0;
              w4[e >> 1] = lo | (hi << 16);
            }
            const uint4 packed = make_uint4(w4[0], w4[1], w4[2], w4[3]);
            __builtin_memcpy(&bfr[j], &packed, 16);
          }
          bkey_ps = kps;
          bkey_r = kr;
        }
        // A operand: U of row frow (zero unless the row is on this adapter),
        // rank rows 8*half .. +7, as bf16 hi + lo
        uint32_t hw[4], lw[4];
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          const float ua = mine ? uv[i][e] : 0.f, ub = mine ? uv[i][e + 1] : 0.f;
          const uint32_t h2 = f2bf2(ua, ub);
          hw[e >> 1] = h2;
          lw[e >> 1] = f2bf2(ua - bf_lo(h2), ub - bf_hi(h2));
        }
        bf16x8_t ahi, alo;
        const uint4 ph = make_uint4(hw[0], hw[1], hw[2], hw[3]);
        const uint4 pl = make_uint4(lw[0], lw[1], lw[2], lw[3]);
        __builtin_memcpy(&ahi, &ph, 16);
        __builtin_memcpy(&alo, &pl, 16);
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ahi, bfr[j], acc[i][j], 0, 0, 0);
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(alo, bfr[j], acc[i][j], 0, 0, 0);
        }
      }
    }
    // the staging region is this wave's own, and the K loop ended with a
    // workgroup barrier: no barrier here (LDS accesses of one wave stay in
    // order)
    if (!(kMask && lterm)) {
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int r = (v >> 2) * 8 + half * 4 + (v & 3);
          stage[r * SC + j * 32 + frow] = acc[i][j][v];
        }
    }
    const int rbase = m0 + wm * TM * 32 + i * 32;
    if (kMask && lterm) {
      // quarter qr: MFMA registers v = 4qr .. 4qr+3 hold rows 8qr .. 8qr+7
#pragma unroll
      for (int qr = 0; qr < 4; ++qr) {
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
          for (int v = 4 * qr; v < 4 * qr + 4; ++v)
            lstage[(half * 4 + (v & 3)) * SC + j * 32 + frow] = acc[i][j][v];
#pragma unroll
        for (int q = 0; q < 8 / RPS; ++q) {
          const int lr = q * RPS + vr;
          const int rr = qr * 8 + lr;
          const int row = rbase + rr;
          if (row < g.M && c8) {
            const float *sb = stage + rr * SC + vc, *sl = lstage + lr * SC + vc;
            const float4 b0 = *reinterpret_cast<const float4 *>(sb);
            const float4 b1 = *reinterpret_cast<const float4 *>(sb + 4);
            const float4 l0 = *reinterpret_cast<const float4 *>(sl);
            const float4 l1 = *reinterpret_cast<const float4 *>(sl + 4);
            const float b8[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
            const float l8[8] = {l0.x, l0.y, l0.z, l0.w, l1.x, l1.y, l1.z, l1.w};
            const uint2 mw = *reinterpret_cast<const uint2 *>(g.mask + int64_t(row) * g.N + cbase + vc);
            float v8[8];
#pragma unroll
            for (int c = 0; c < 8; ++c) {
              const uint32_t word = c < 4 ? mw.x : mw.y;
              v8[c] = b8[c] + float((word >> (8 * (c & 3))) & 0xffu) * l8[c];
            }
            store8_nt(Y + int64_t(row) * g.N + cbase + vc, v8);
          }
        }
      }
    } else if (!((rowwise >> i) & 1u)) {
#pragma unroll
      for (int rr0 = 0; rr0 < 32; rr0 += RPS) {
        const int rr = rr0 + vr;
        const int row = rbase + rr;
        if (row < g.M && c8) {
          const float4 lo = *reinterpret_cast<const float4 *>(stage + rr * SC + vc);
          const float4 hi = *reinterpret_cast<const float4 *>(stage + rr * SC + vc + 4);
          const float v8[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
          store8_nt(Y + int64_t(row) * g.N + cbase + vc, v8);
        }
      }
    } else {
      for (int rr = 0; rr < 32; ++rr) {
        const int row = rbase + rr;
        if (row >= g.M) break;
        float v[CPL];
#pragma unroll
        for (int c = 0; c < CPL; ++c) v[c] = stage[rr * SC + lane * CPL + c];
        if constexpr (kMask) {
          float l[CPL];
#pragma unroll
          for (int c = 0; c < CPL; ++c) l[c] = 0.f;
          expand_row_cached<CPL, 16>(l, row, col, g.ex, cache);
          const uint8_t *mr = g.mask + int64_t(row) * g.N + col;
#pragma unroll
          for (int c = 0; c < CPL; ++c) v[c] += float(mr[c]) * l[c];
        } else {
          expand_row_cached<CPL, 16>(v, row, col, g.ex, cache);
        }
        if (col_ok) Cols<uint16_t, CPL>::store(Y + int64_t(row) * g.N + col, v);
      }
    }
  }
}

// Fragment read slot i of a K step (A blocks 0 .. TM-1 are fragments
// 0 .. TM-1, B blocks TM ..): block (i, j) takes MFMA i * TN + j, so the
// next step needs A 0 and B 0 first, then B 1 .. TN-1, then A 1, A 2, ...;
// read in that order, one after each of the first TM + TN MFMAs of a step,
// every fragment has at least TM * TN - 2 MFMAs between its read and its
// first use.
template <int TM, int TN>
__device__ __forceinline__ constexpr int frag_order(int i) {
  return i == 0 ? 0 : i <= TN ? TM + i - 1 : i - TN;
}

// One K tile of MFMAs from an LDS stage.  pre_step(s) runs before each of
// the four 16-wide K steps (the ring pipeline issues a quarter of the next
// tile's copies there, so that they queue while the MFMAs execute).
struct NoStep {
  __device__ __forceinline__ void operator()(int) const {}
};

template <int BM, int BN, int WM, int WN, typename F = NoStep>
__device__ __forceinline__ void tile_mfma(const char *As,
                                          f32x16_t (&acc)[TileCfg<BM, BN, WM, WN>::TM]
                                                         [TileCfg<BM, BN, WM, WN>::TN],
                                          const F &pre_step = F()) {
  using C = TileCfg<BM, BN, WM, WN>;
  constexpr int TM = C::TM, TN = C::TN;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave / WN, wn = wave % WN;
  const int frow = lane & 31, half = lane >> 5;
  // Fragments are pipelined inside the tile: the LDS reads of K step s + 1
  // go out under the first MFMAs of step s (two register sets) in the order
  // that step s + 1 uses them, each step's instructions pinned in this order
  // (sched_barrier).
  bf16x8_t fa0[TM], fb0[TN], fa1[TM], fb1[TN];
  // fragment q (A blocks 0 .. TM-1, then B blocks) of K step s
  auto frag = [&](int s, int q) __attribute__((always_inline)) {
    const int row = q < TM ? wm * TM * 32 + q * 32 + frow : BM + wn * TN * 32 + (q - TM) * 32 + frow;
    return *reinterpret_cast<const bf16x8_t *>(As + row * C::ROWB + (tswz(frow, 2 * s + half) << 4));
  };
  auto kstep = [&](auto nxt, int s, bf16x8_t (&xa)[TM], bf16x8_t (&xb)[TN], bf16x8_t (&ya)[TM],
                   bf16x8_t (&yb)[TN]) __attribute__((always_inline)) {
    constexpr bool kNext = decltype(nxt)::value;
    constexpr int NM = TM * TN, NF = TM + TN;
    static_assert(NF <= NM, "one fragment read after each of the first MFMAs");
    pre_step(s);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int m = 0; m < NM; ++m) {
      acc[m / TN][m % TN] =
          __builtin_amdgcn_mfma_f32_32x32x16_bf16(xa[m / TN], xb[m % TN], acc[m / TN][m % TN], 0, 0, 0);
      if constexpr (kNext) {
        const int q = frag_order<TM, TN>(m);
        if (m < NF) {
          if (q < TM) ya[q] = frag(s + 1, q);
          else yb[q - TM] = frag(s + 1, q);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };
#pragma unroll
  for (int q = 0; q < TM + TN; ++q) {
    if (q < TM) fa0[q] = frag(0, q);
    else fb0[q - TM] = frag(0, q);
  }
  kstep(std::true_type{}, 0, fa0, fb0, fa1, fb1);
  kstep(std::true_type{}, 1, fa1, fb1, fa0, fb0);
  kstep(std::true_type{}, 2, fa0, fb0, fa1, fb1);
  kstep(std::false_type{}, 3, fa1, fb1, fa0, fb0);
}

// Wait until at most n (0 <= n <= NS - 2) K tiles' copies are still in flight.
template <int LPW, int NS>
__device__ __forceinline__ void wait_tiles(int n) {
  if constexpr (NS >= 4) {
    if (n >= 2) { wait_vmcnt<2 * LPW>(); return; }
  }
  if constexpr (NS >= 3) {
    if (n >= 1) { wait_vmcnt<LPW>(); return; }
  }
  wait_vmcnt<0>();
}

// One output tile (m0, n0) over K tiles [k_begin / 64, + nk): the K loop
// and the epilogue (fp32 partials into slot `slot`, or the fused expand).
template <int BM, int BN, int WM, int WN, int NS, bool kFused, bool kMask = false>
__device__ __forceinline__ void tile_run(const GemmArgs &g, char *smem, int m0, int n0,
                                         int k_begin, int nk, int slot) {
  using C = TileCfg<BM, BN, WM, WN>;
  constexpr int TM = C::TM, TN = C::TN;
  char *const st0 = smem;
  char *const st1 = smem + C::STAGE;
  const uint16_t *X = static_cast<const uint16_t *>(g.X);
  const uint16_t *W = static_cast<const uint16_t *>(g.W);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;

  // per-lane source rows, as 32-bit element offsets from the tile's first row
  // (clamped: rows past M / N feed outputs that are never stored)
  const int lrow = lane >> 3;
  const uint16_t *abase = X + int64_t(m0) * g.Kd + k_begin;
  const uint16_t *bbase = W + int64_t(n0) * g.Kd + k_begin;
  uint32_t aoff[C::A_INS], boff[C::B_INS];
#pragma unroll
  for (int i = 0; i < C::A_INS; ++i) {
    const int row = (wave * C::A_INS + i) * 8 + lrow;
    aoff[i] = uint32_t(min(row, g.M - 1 - m0)) * uint32_t(g.Kd) + tswz(row, lane & 7) * 8;
  }
#pragma unroll
  for (int i = 0; i < C::B_INS; ++i) {
    const int row = (wave * C::B_INS + i) * 8 + lrow;
    boff[i] = uint32_t(min(row, g.N - 1 - n0)) * uint32_t(g.Kd) + tswz(row, lane & 7) * 8;
  }
  auto issue = [&](char *base, int kt) {
    const uint16_t *a = abase + kt * 64;
    const uint16_t *b = bbase + kt * 64;
    const uint32_t lds = lds_addr(base);
#pragma unroll
    for (int i = 0; i < C::A_INS; ++i)
      lds_dma16(a + aoff[i], lds + (wave * C::A_INS + i) * 1024);
#pragma unroll
    for (int i = 0; i < C::B_INS; ++i)
      lds_dma16(b + boff[i], lds + BM * C::ROWB + (wave * C::B_INS + i) * 1024);
  };
  // quarter q of issue(base, kt): copies [q * LPW / 4, (q + 1) * LPW / 4) of
  // the wave's A-then-B list, in the same order as issue()
  static_assert(NS == 2 || C::LPW % 4 == 0, "copies split over the four K steps");
  auto issue_quarter = [&](char *base, int kt, int q) {
    const uint16_t *a = abase + kt * 64;
    const uint16_t *b = bbase + kt * 64;
    const uint32_t lds = lds_addr(base);
#pragma unroll
    for (int c = 0; c < C::LPW / 4; ++c) {
      const int i = q * (C::LPW / 4) + c;
      if (i < C::A_INS) lds_dma16(a + aoff[i], lds + (wave * C::A_INS + i) * 1024);
      else lds_dma16(b + boff[i - C::A_INS], lds + BM * C::ROWB + (wave * C::B_INS + i - C::A_INS) * 1024);
    }
  };

  f32x16_t acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  // the fused epilogue's descriptors go out ahead of the first copies
  EpiPre<TM> pre;
  if constexpr (kFused) epi_fetch_desc<BM, BN, WM, WN>(g, m0, pre);

  const int frow = lane & 31, half = lane >> 5;
  // NS >= 3 stages in a ring: K tile kt lives in stage kt % NS.  At the top
  // of step kt, once tile kt has landed and every wave has left step kt - 1,
  // tile kt + NS - 1 is issued into the stage step kt - 1 used, so NS - 1
  // tiles' copies are in flight while tile kt feeds the MFMAs.
  if constexpr (NS == 2) {
    // Two stages, pipelined at fragment level.  The fragments of K step
    // s + 1 are read from LDS while the MFMAs of step s run (two register
    // sets: fa0/fb0 for even steps, fa1/fb1 for odd ones).  Before the last
    // step of K tile kt one barrier both frees the stage just read (the
    // copies of tile kt + 2 go into it, one after each MFMA of that step)
    // and publishes tile kt + 1, whose first fragments are read at once; so
    // the MFMA pipe is never left waiting on a fragment read.  Each step's
    // instructions are pinned in this order (sched_barrier): left alone, the
    // compiler keeps one register set and reads a step's fragments only
    // after the previous step's MFMAs have issued.
    bf16x8_t fa0[TM], fb0[TN], fa1[TM], fb1[TN];
    // fragment q (A blocks 0 .. TM-1, then B blocks) of K step s
    auto frag = [&](const char *base, int s, int q) __attribute__((always_inline)) {
      const int row = q < TM ? wm * TM * 32 + q * 32 + frow : BM + wn * TN * 32 + (q - TM) * 32 + frow;
      return *reinterpret_cast<const bf16x8_t *>(base + row * C::ROWB + (tswz(frow, 2 * s + half) << 4));
    };
    // copy i of the wave's A-then-B list for K tile kt into stage base
    auto dma_one = [&](char *base, int kt, int i) __attribute__((always_inline)) {
      const uint32_t lds = lds_addr(base);
      if (i < C::A_INS) lds_dma16(abase + kt * 64 + aoff[i], lds + (wave * C::A_INS + i) * 1024);
      else lds_dma16(bbase + kt * 64 + boff[i - C::A_INS], lds + BM * C::ROWB + (wave * C::B_INS + i - C::A_INS) * 1024);
    };
    // One K step: MFMA m on block (m / TN, m % TN) from (xa, xb), each
    // followed by one of the next step's fragment reads from src (into ya,
    // yb, in frag_order; mode bit 0) and its share of the copies of K tile
    // kn into dst (bit 1).
    auto kstep = [&](auto mode, bf16x8_t (&xa)[TM], bf16x8_t (&xb)[TN], bf16x8_t (&ya)[TM],
                     bf16x8_t (&yb)[TN], const char *src, int s_next, char *dst,
                     int kn) __attribute__((always_inline)) {
      constexpr int MD = decltype(mode)::value;
      constexpr int NM = TM * TN, NQ = TM + TN;
      static_assert(NQ <= NM, "one fragment read after each of the first MFMAs");
#pragma unroll
      for (int m = 0; m < NM; ++m) {
        acc[m / TN][m % TN] =
            __builtin_amdgcn_mfma_f32_32x32x16_bf16(xa[m / TN], xb[m % TN], acc[m / TN][m % TN], 0, 0, 0);
        if constexpr ((MD & 1) != 0) {
          const int q = frag_order<TM, TN>(m);
          if (m < NQ) {
            if (q < TM) ya[q] = frag(src, s_next, q);
            else yb[q - TM] = frag(src, s_next, q);
          }
        }
        if constexpr ((MD & 2) != 0) {
#pragma unroll
          for (int c = m * C::LPW / NM; c < (m + 1) * C::LPW / NM; ++c) dma_one(dst, kn, c);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    if (nk > 0) issue(st0, 0);
    if (nk > 1) {
      issue(st1, 1);
      wait_vmcnt<C::LPW>();
    } else {
      wait_vmcnt<0>();
    }
    lds_bar();
    if (nk > 0) {
#pragma unroll
      for (int q = 0; q < TM + TN; ++q) {
        if (q < TM) fa0[q] = frag(st0, 0, q);
        else fb0[q - TM] = frag(st0, 0, q);
      }
    }
    // K tile kt from stage cur, its step-0 fragments in fa0/fb0 on entry.
    // The last step reads the first fragments of tile kt + 1 from nxt and
    // copies tile kt + 2 into cur.  Past the end the body stays the same
    // (no branch inside the loop): the copy repeats the last tile into a
    // stage no one reads again, and the reads of nxt go unused.
    for (int kt = 0; kt < nk; ++kt) {
      char *const cur = (kt & 1) ? st1 : st0;
      char *const nxt = (kt & 1) ? st0 : st1;
      kstep(std::integral_constant<int, 1>{}, fa0, fb0, fa1, fb1, cur, 1, cur, 0);
      kstep(std::integral_constant<int, 1>{}, fa1, fb1, fa0, fb0, cur, 2, cur, 0);
      kstep(std::integral_constant<int, 1>{}, fa0, fb0, fa1, fb1, cur, 3, cur, 0);
      wait_vmcnt<0>();   // tile kt + 1, the only copies in flight, has landed
      lds_bar();         // for every wave, and every wave has read cur
      // fused: the descriptors have landed with the first copies; the page
      // ids go out now and land under the following K tiles
      if constexpr (kFused) {
        if (kt == 0) epi_fetch_pid(g, pre);
      }
      kstep(std::integral_constant<int, 3>{}, fa1, fb1, fa0, fb0, nxt, 0, cur, min(kt + 2, nk - 1));
    }
    if constexpr (kFused) {
      if (nk <= 0) epi_fetch_pid(g, pre);
    }
    // the copies of the last step have landed and every wave is done with
    // the stages before anything else uses this LDS
    wait_vmcnt<0>();
    lds_bar();
  } else {
#pragma unroll
    for (int i = 0; i < NS - 1; ++i)
      if (i < nk) issue(smem + i * C::STAGE, i);
    for (int kt0 = 0; kt0 < nk; kt0 += NS) {
#pragma unroll
      for (int u = 0; u < NS; ++u) {
        const int kt = kt0 + u;
        if (kt < nk) {
          wait_tiles<C::LPW, NS>(min(NS - 2, nk - 1 - kt));
          lds_bar();
          char *const nxt = smem + ((u + NS - 1) % NS) * C::STAGE;
          const bool more = kt + NS - 1 < nk;
          tile_mfma<BM, BN, WM, WN>(smem + u * C::STAGE, acc, [&](int q) {
            if (more) issue_quarter(nxt, kt + NS - 1, q);
          });
        }
      }
    }
    if constexpr (kFused) epi_fetch_pid(g, pre);
    __syncthreads();   // the epilogue reuses the stages
  }

  if constexpr (!kFused) {
    // partials are read once, by the epilogue: streaming (non-temporal) stores
    float *Pz = g.partial + int64_t(slot) * g.M * g.N;
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int col = n0 + wn * TN * 32 + j * 32 + frow;
        if (col >= g.N) continue;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int row = m0 + wm * TM * 32 + i * 32 + (v >> 2) * 8 + half * 4 + (v & 3);
          if (row < g.M) __builtin_nontemporal_store(acc[i][j][v], Pz + int64_t(row) * g.N + col);
        }
      }
  } else {
    fused_epilogue<BM, BN, WM, WN, kMask>(g, acc, st0, st1, m0, n0, pre);
  }
}

// Stream-K: workgroup w of G = g.sk_g takes the units (tile, K tile)
// [w U / G, (w + 1) U / G) of the U = tiles x KT units, in order, across tile
// boundaries; each maximal run inside one tile is a piece, stored in slot
// w - (first workgroup of that tile).  The epilogue adds a tile's pieces in
// K order.
template <int BM, int BN, int WM, int WN, int NS>
__device__ __forceinline__ void stream_k(const GemmArgs &g, char *smem, int w) {
  const int tiles_n = (g.N + BN - 1) / BN;
  const int ntiles = ((g.M + BM - 1) / BM) * tiles_n;
  const int KT = g.Kd / 64;
  const int64_t U = int64_t(ntiles) * KT;
  const int G = g.sk_g;
  int64_t u = int64_t(w) * U / G;
  const int64_t u1 = int64_t(w + 1) * U / G;
  while (u < u1) {
    const int t = int(u / KT), kb = int(u % KT);
    const int ke = int(min<int64_t>(KT, kb + (u1 - u)));
    const int wf = int(((int64_t(t) * KT + 1) * G - 1) / U);
    tile_run<BM, BN, WM, WN, NS, false>(g, smem, (t / tiles_n) * BM, (t % tiles_n) * BN, kb * 64,
                                        ke - kb, w - wf);
    u += ke - kb;
  }
}

template <int BM, int BN, int WM, int WN, int NS, bool kFused, bool kMask = false>
__global__ __launch_bounds__(WM * WN * 64, 1) void gemm_tile_kernel(GemmArgs g) {
  using C = TileCfg<BM, BN, WM, WN>;
  static_assert(NS >= 2 && (NS - 2) * C::LPW < 64, "stages / vmcnt range");
  __shared__ __attribute__((aligned(16))) char smem[NS * C::STAGE];
  const int tiles_m = (g.M + BM - 1) / BM, tiles_n = (g.N + BN - 1) / BN;
  const int ntiles = tiles_m * tiles_n;
  if constexpr (!kFused && NS >= 3) {
    if (g.sk_g > 0) {
      stream_k<BM, BN, WM, WN, NS>(g, smem, blockIdx.x);
      return;
    }
  }
  const int per = (ntiles + 7) / 8;
  int b = int(blockIdx.x), half = -1;
  if constexpr (kFused && NS == 2 && BN == 256) {
    // A grid larger than 8 * per asks for the last, partial round of tiles
    // (the workgroups past the last multiple of 256) as two 256 x 128 halves
    // each: that round then takes half a tile's time on twice the CUs.
    const int nb = 8 * per, n_first = nb - nb % 256;
    if (int(gridDim.x) > nb && b >= n_first) {
      half = (b - n_first) & 1;
      b = n_first + (b - n_first) / 2;
    }
  }
  const int t = (b & 7) * per + (b >> 3);
  if (t >= ntiles) return;
  int tm, tn;
  tile_coords(t, tiles_m, tiles_n, tm, tn);
  const int k_begin = blockIdx.y * g.k_split;
  const int k_end = min(g.Kd, k_begin + g.k_split);
  if constexpr (kFused && NS == 2 && BN == 256) {
    if (half >= 0) {
      // a second half wholly past the last column has nothing to do (and its
      // operand rows must not be clamped from below N)
      const int n0 = tn * BN + half * (BN / 2);
      if (n0 >= g.N) return;
      // the same waves as a 4 x 2 grid when the full tile's is 2 x 4 (each
      // wave then keeps 64 columns, which the fused epilogue needs)
      constexpr int HWM = WN == 4 ? 4 : WM, HWN = WN == 4 ? 2 : WN;
      tile_run<BM, BN / 2, HWM, HWN, NS, kFused, kMask>(g, smem, tm * BM, n0, k_begin,
                                                        (k_end - k_begin) / 64, blockIdx.y);
      return;
    }
  }
  tile_run<BM, BN, WM, WN, NS, kFused, kMask>(g, smem, tm * BM, tn * BN, k_begin,
                                              (k_end - k_begin) / 64, blockIdx.y);
}

// Stream-K GEMM over workgroups 0 .. G-1, with the plan built by workgroup
// G in the LDS the others use for their stages (one CU of its own).
template <int BM, int BN, int WM, int WN, int NS, bool kLds>
__global__ __launch_bounds__(WM * WN * 64, 1) void gemm_tile_plan_kernel(GemmArgs g, PlanArgs pa) {
  using C = TileCfg<BM, BN, WM, WN>;
  __shared__ __attribute__((aligned(16))) char smem[NS * C::STAGE];
  // block 0 builds the plan (dispatched first, its loads go out ahead of
  // the W stream); blocks 1..G are the stream-K workgroups
  if (blockIdx.x == 0) {
    plan_build<kLds>(pa, reinterpret_cast<int *>(smem));
    return;
  }
  stream_k<BM, BN, WM, WN, NS>(g, smem, int(blockIdx.x) - 1);
}

// ------------------------------------------------------------ fp32 GEMM
// Plain LDS-tiled fp32 product (the fp32 layer is small): 64x64 output tile,
// 256 threads each owning 4x4 outputs, K split over blockIdx.z (partials
// summed in order by the epilogue).  A 64-wide K chunk of both operands is
// loaded in one round trip (16 values per thread each), the next chunk's
// loads in flight while the current one is used.
// Workgroup b < tiles_x * tiles_y * splits takes tile (b % tiles_x,
// (b / tiles_x) % tiles_y) and split b / (tiles_x * tiles_y); with kPlan the
// last workgroup builds the plan (1: arrays in LDS, 2: in the plan buffer).
template <int kPlan>
__global__ __launch_bounds__(256) void gemm_f32_kernel(const float *X, const float *W, float *P,
                                                        int M, int N, int Kd, int k_split,
                                                        int tiles_x, int tiles_y, PlanArgs pa) {
  constexpr int KC = 64;
  __shared__ float As[KC][64 + 4];
  __shared__ float Bs[KC][64 + 4];
  if constexpr (kPlan != 0) {
    if (blockIdx.x == gridDim.x - 1) {
      extern __shared__ int fdyn[];
      plan_build<kPlan == 1>(pa, fdyn);
      return;
    }
  }
  const int b = blockIdx.x;
  const int bz = b / (tiles_x * tiles_y);
  const int tid = threadIdx.x;
  const int tx = tid & 15, ty = tid >> 4;
  const int m0 = ((b / tiles_x) % tiles_y) * 64, n0 = (b % tiles_x) * 64;
  const int k_begin = bz * k_split, k_end = min(Kd, k_begin + k_split);
  float acc[4][4] = {};
  float an[16], bn[16];
  auto load = [&](int k0) {
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int idx = tid + e * 256;
      const int rr = idx >> 6, kk = idx & 63;
      an[e] = X[int64_t(min(m0 + rr, M - 1)) * Kd + k0 + kk];
      bn[e] = W[int64_t(min(n0 + rr, N - 1)) * Kd + k0 + kk];
    }
  };
  if (k_begin < k_end) load(k_begin);
  for (int k0 = k_begin; k0 < k_end; k0 += KC) {
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int idx = tid + e * 256;
      As[idx & 63][idx >> 6] = an[e];
      Bs[idx & 63][idx >> 6] = bn[e];
    }
    __syncthreads();
    if (k0 + KC < k_end) load(k0 + KC);
#pragma unroll 8
    for (int kk = 0; kk < KC; ++kk) {
      float av[4], bv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) { av[i] = As[kk][ty * 4 + i]; bv[i] = Bs[kk][tx * 4 + i]; }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(av[i], bv[j], acc[i][j]);
    }
    __syncthreads();
  }
  float *Pz = P + int64_t(bz) * M * N;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = m0 + ty * 4 + i;
    if (row >= M) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int col = n0 + tx * 4 + j;
      if (col < N) Pz[int64_t(row) * N + col] = acc[i][j];
    }
  }
}

// ------------------------------------------------------------ epilogue kernel
// One wave per output row and 512-column chunk: sum the split partials in
// order, add the expand, round once, store.  16-byte B-row loads, 1 KiB per
// wave instruction.
//
// On lora_forward's decode path (a.sdesc set) the expand reads the per-slot U
// and slot descriptors that the previous launch's per-slot shrink wrote, and
// the first column chunk of each row also moves that row's U to the u_off
// places of the plan the previous launch's workgroup 0 built.  As in
// lora_apply, the LoRA term is skipped (and LORA_DEVERR_CAPACITY set) when the
// plan's U does not fit the workspace.
template <typename E, int NW, bool kMask = false>
__global__ __launch_bounds__(NW * 64) void epilogue_kernel(EpilogueArgs a) {
  constexpr int CPL = 8;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int row, cx;
  if (a.pair_tk) {
    const int i = blockIdx.x;
    if (i < a.n_a) {
      // pair groups from the last: the plan orders segments by ascending rank
      // bucket, so the longest rows are dispatched first and short ones fill
      // the tail
      const int np = a.ex.hdr[LORA_PH_PAIRS];
      const int ng = (np + NW - 1) / NW;
      const int gi = i / a.n_x;
      if (gi >= ng) return;
      const int q = (ng - 1 - gi) * NW + wave;
      cx = i % a.n_x;
      if (q >= np) return;
      row = a.pair_tk[q];                               // one slot per token
    } else {
      const int j = i - a.n_a;
      cx = j % a.n_x;
      row = (j / a.n_x) * NW + wave;
      if (row >= a.M) return;
      if (a.ex.slot_desc[row].x >= 0) return;           // taken in pair order
    }
  } else {
    row = blockIdx.y * NW + wave;
    cx = blockIdx.x;
    if (row >= a.M) return;
  }
  // decode: the first column chunk of each row also moves the row's per-slot
  // U to the plan's u_off places; the loads for its first slot (first 64 rank
  // rows) go out now so that their round trips overlap the rest
  const bool do_copy = a.u_out != nullptr && cx == 0;
  int4 cpd0 = make_int4(-1, 0, 0, 0);
  float cpv0 = 0.f;
  int64_t rpairs = 0;
  if (do_copy) {
    rpairs = a.plan_hdr[LORA_PH_RPAIRS];
    const int64_t i = int64_t(row) * a.ex.K;
    cpd0 = a.plan_sdesc[i];
    cpv0 = a.ex.U[i * a.slot_stride + lane];          // rank rows < 64 <= LORA_MAX_RANK
  }
  const int col_raw = (cx * 64 + lane) * CPL;
  const bool col_ok = col_raw < a.N;
  const int col = col_ok ? col_raw : a.N - CPL;      // loads stay in bounds
  // decode forward: the same rule as expand_enabled, with the plan's R_pairs
  // against the capacity of the packed U the plan layout is stored into
  const bool lora_on = a.sdesc ? (a.ex.U != nullptr &&
                                  (a.u_out == nullptr || int64_t(a.plan_hdr[LORA_PH_RPAIRS]) <= a.u_cap))
                               : expand_enabled(a.ex);
  // the row's slot descriptors first: their round trip overlaps the partials'
  int4 sd = make_int4(-1, 0, 0, 0);
  if (lora_on) {
    if (a.sdesc) {
      if (lane < a.ex.K) sd = a.sdesc[row * a.ex.K + lane];
    } else {
      sd = expand_row_desc<E>(row, a.ex);
    }
  }
  float v[CPL];
#pragma unroll
  for (int c = 0; c < CPL; ++c) v[c] = 0.f;
  // pieces of this lane's output: the K splits, or under stream-K the
  // workgroups that covered its tile (w(x) = workgroup holding unit x)
  int np = a.splits;
  if (a.sk_g > 0) {
    const int tiles_n = (a.N + a.bn - 1) / a.bn;
    const int t = (row / a.bm) * tiles_n + col / a.bn;
    const int64_t U = int64_t((a.M + a.bm - 1) / a.bm) * tiles_n * a.sk_kt;
    const int64_t x0 = int64_t(t) * a.sk_kt, x1 = x0 + a.sk_kt - 1;
    np = int(((x1 + 1) * a.sk_g - 1) / U - ((x0 + 1) * a.sk_g - 1) / U) + 1;
  }
  // partials: issue up to 8 at once, add in piece order
  for (int z0 = 0; z0 < a.splits; z0 += 8) {
    Raw8<float> pr[8];
#pragma unroll
    for (int z = 0; z < 8; ++z)
      pr[z].load(a.partial + (int64_t(min(z0 + z, np - 1)) * a.M + row) * a.N + col);
#pragma unroll
    for (int z = 0; z < 8; ++z) {
      if (z0 + z < np) {
        float pv[8];
        pr[z].to8(pv);
#pragma unroll
        for (int c = 0; c < CPL; ++c) v[c] += pv[c];
      }
    }
  }
  if (lora_on) {
    if constexpr (kMask) {
      // the expand term alone, then times the row's keep-mask bytes
      float l[CPL];
#pragma unroll
      for (int c = 0; c < CPL; ++c) l[c] = 0.f;
      expand_row8<E>(l, sd, col, a.ex);
      const uint2 mw = *reinterpret_cast<const uint2 *>(a.mask + int64_t(row) * a.N + col);
#pragma unroll
      for (int c = 0; c < CPL; ++c) {
        const uint32_t word = c < 4 ? mw.x : mw.y;
        v[c] += float((word >> (8 * (c & 3))) & 0xffu) * l[c];
      }
    } else {
      expand_row8<E>(v, sd, col, a.ex);
    }
  }
  if (col_ok) Cols<E, CPL>::store(static_cast<E *>(a.Y) + int64_t(row) * a.N + col, v);
  if (do_copy) {
    // this row's per-slot U to the places the plan gave its active slots
    if (rpairs > a.u_cap) {
      if (row == 0 && lane == 0) atomicOr(a.plan_hdr + LORA_PH_ERR, LORA_DEVERR_CAPACITY);
      return;
    }
    for (int k = 0; k < a.ex.K; ++k) {
      const int64_t i = int64_t(row) * a.ex.K + k;
      int4 d = cpd0;
      float v0 = cpv0;
      if (k > 0) {
        d = a.plan_sdesc[i];
        v0 = a.ex.U[i * a.slot_stride + lane];
      }
      if (d.x < 0) continue;
      if (lane < d.y) a.u_out[d.z + lane] = v0;
      const float *src = a.ex.U + i * a.slot_stride;
      for (int j = lane + 64; j < d.y; j += 64) a.u_out[d.z + j] = src[j];
    }
  }
}

}  // namespace

GemmConfig choose_gemm(int T, int d_in, int d_out, int dtype) {
  GemmConfig c{};
  if (dtype == LORA_F32) {
    // K split so that each workgroup's K range is a few 64-wide chunks and
    // the small fp32 layer still spreads over more than a handful of CUs
    c.kind = 0; c.bm = 64; c.bn = 64; c.fused = false;
    const int kb = d_in / 64;
    const int want = kb < 8 ? kb : 8;
    const int per = (kb + want - 1) / want;
    c.k_split = per * 64;
    c.splits = (kb + per - 1) / per;
    return c;
  }
  if (T <= 128) {
    // decode: W streamed once, K split in chunks of 512 across workgroups
    c.kind = 4; c.bn = 128;
    c.bm = T <= 32 ? 32 : (T <= 64 ? 64 : 128);
    c.k_split = 512;
    c.splits = (d_in + 511) / 512;
    c.fused = false;
    return c;
  }
  const int kblocks = d_in / 64;
  // enough 256 x 256 tiles to fill the GPU: fused epilogue, no split
  const int64_t big_tiles = int64_t((T + 255) / 256) * ((d_out + 255) / 256);
  if (big_tiles >= 256) {
    c.kind = 5; c.bm = 256; c.bn = 256;
    c.splits = 1; c.k_split = d_in; c.fused = true;
    return c;
  }
  // otherwise 256 x 128 tiles, stream-K over 255 workgroups (one per CU, the
  // last CU left to the plan workgroup when the plan is built in the launch):
  // every workgroup takes the same number of (tile, K tile) units, so no CU
  // runs a second round; a tile is covered by at most ceil(KT / per) + 1
  // workgroups (its pieces)
  c.kind = 6; c.bm = 256; c.bn = 128; c.fused = false;
  const int64_t tiles = int64_t((T + c.bm - 1) / c.bm) * ((d_out + c.bn - 1) / c.bn);
  const int64_t units = tiles * kblocks;
  constexpr int kStreamWgs = 255;       // + 1 plan workgroup in launch_gemm_plan
  if (units >= 4 * kStreamWgs) {
    const int64_t per = units / kStreamWgs;
    c.sk = kStreamWgs;
    c.k_split = 64;
    c.splits = int((kblocks + per - 1) / per) + 1;
    return c;
  }
  // few units: classic split-K with ~256 workgroups
  int64_t want = tiles > 0 ? (256 + tiles - 1) / tiles : 1;
  int64_t most = kblocks / 8 > 1 ? kblocks / 8 : 1;     // every split keeps >= 512 of K
  int splits = int(want < most ? want : most);
  if (splits < 1) splits = 1;
  const int kb_per = (kblocks + splits - 1) / splits;
  c.k_split = kb_per * 64;
  c.splits = (kblocks + kb_per - 1) / kb_per;
  c.sk = 0;
  return c;
}

size_t gemm_partial_bytes(const GemmConfig &c, int T, int d_out) {
  return c.fused ? 0 : size_t(c.splits) * size_t(T) * size_t(d_out) * sizeof(float);
}

hipError_t launch_base_gemm(const GemmConfig &c, const GemmArgs &g, hipStream_t s) {
  if (c.kind == 0) {
    const int tx = (g.N + 63) / 64, ty = (g.M + 63) / 64;
    hipLaunchKernelGGL(gemm_f32_kernel<0>, dim3(unsigned(tx * ty * c.splits)), dim3(256), 0, s,
                       static_cast<const float *>(g.X), static_cast<const float *>(g.W), g.partial,
                       g.M, g.N, g.Kd, c.k_split, tx, ty, PlanArgs{});
    return hipGetLastError();
  }
  if (c.kind == 4) {
    const dim3 grid((g.N + 127) / 128, (g.M + c.bm - 1) / c.bm, c.splits);
    if (c.bm == 32) hipLaunchKernelGGL(gemm_decode_kernel<1>, grid, dim3(256), 0, s, g);
    else if (c.bm == 64) hipLaunchKernelGGL(gemm_decode_kernel<2>, grid, dim3(256), 0, s, g);
    else hipLaunchKernelGGL(gemm_decode_kernel<4>, grid, dim3(256), 0, s, g);
    return hipGetLastError();
  }
  if (g.mask && !(c.kind == 5 && c.fused)) return hipErrorInvalidConfiguration;
  if (c.kind == 5 || c.kind == 6) {
    const int tiles = ((g.M + c.bm - 1) / c.bm) * ((g.N + c.bn - 1) / c.bn);
    const dim3 grid = c.sk > 0 ? dim3(c.sk, 1) : dim3(8 * ((tiles + 7) / 8), c.splits);
    if (c.kind == 5) {
      if (c.fused) {
        // a last partial round of at most 128 tiles runs as 256 x 128 halves
        unsigned gx = grid.x;
        const unsigned nf = gx - gx % 256, rem = gx - nf;
        if (nf > 0 && rem > 0 && rem <= 128) gx = nf + 2 * rem;
        if (g.mask)
          hipLaunchKernelGGL((gemm_tile_kernel<256, 256, 2, 4, 2, true, true>), dim3(gx, grid.y), dim3(512), 0, s, g);
        else
          hipLaunchKernelGGL((gemm_tile_kernel<256, 256, 2, 4, 2, true>), dim3(gx, grid.y), dim3(512), 0, s, g);
      }
      else hipLaunchKernelGGL((gemm_tile_kernel<256, 256, 2, 4, 2, false>), grid, dim3(512), 0, s, g);
    } else {
      if (c.fused) hipLaunchKernelGGL((gemm_tile_kernel<256, 128, 2, 2, 3, true>), grid, dim3(256), 0, s, g);
      else hipLaunchKernelGGL((gemm_tile_kernel<256, 128, 2, 2, 3, false>), grid, dim3(256), 0, s, g);
    }
    return hipGetLastError();
  }
  return hipErrorInvalidConfiguration;
}

bool decode_shrink_fusable(const GemmConfig &c, int d_in) {
  return c.kind == 4 && d_in <= 8 * 512;
}

hipError_t launch_decode_gemm_shrink(const GemmConfig &c, const GemmArgs &g, const ShrinkArgs &sa,
                                     hipStream_t st) {
  const int gx = (g.N + 127) / 128, gy = (g.M + c.bm - 1) / c.bm;
  const int n_gemm = gx * gy * c.splits;
  // shrink workgroups: enough waves that each walks at most two runs of the
  // schedule, and no more than the GEMM's own count (two workgroups per CU
  // fit the 64 KiB of LDS each)
  const int n_shr = kShrinkWaves / 8;
  const dim3 grid(unsigned(n_gemm + n_shr)), block(256);
  const bool m = sa.mask != nullptr;
#define LORA_DGS(MB, M) \
  hipLaunchKernelGGL((decode_gemm_shrink_kernel<MB, M, 8>), grid, block, 0, st, g, sa, gx, gy, n_gemm)
#define LORA_DGS_M(MB) do { if (m) LORA_DGS(MB, true); else LORA_DGS(MB, false); } while (0)
  if (c.bm == 32) LORA_DGS_M(1);
  else if (c.bm == 64) LORA_DGS_M(2);
  else LORA_DGS_M(4);
#undef LORA_DGS_M
#undef LORA_DGS
  return hipGetLastError();
}

bool gemm_plan_fusable(const GemmConfig &c) {
  return c.kind == 0 || c.kind == 4 || (c.kind == 6 && c.sk > 0);
}

// Decode: the plan workgroup uses the decode tile's token-row LDS (bm rows
// of kDecodeKC bf16).  fp32: the launch's dynamic LDS, kept to 64 KiB.
// Stream-K: the tile kernel's stages.
size_t plan_lds_cap(const GemmConfig &c) {
  if (c.kind == 4) return size_t(c.bm) * kDecodeKC * sizeof(uint16_t);
  if (c.kind == 0) return size_t(64) << 10;
  return size_t(3) * TileCfg<256, 128, 2, 2>::STAGE;
}

hipError_t launch_gemm_plan(const GemmConfig &c, const GemmArgs &g, const PlanLaunch &pl,
                            hipStream_t s) {
  if (pl.lds_bytes > plan_lds_cap(c)) return hipErrorInvalidConfiguration;
  if (c.kind == 0) {
    const int tx = (g.N + 63) / 64, ty = (g.M + 63) / 64;
    const dim3 grid(unsigned(tx * ty * c.splits + 1)), block(256);
    const float *X = static_cast<const float *>(g.X), *W = static_cast<const float *>(g.W);
    if (pl.lds)
      hipLaunchKernelGGL(gemm_f32_kernel<1>, grid, block, pl.lds_bytes, s, X, W, g.partial, g.M, g.N,
                         g.Kd, c.k_split, tx, ty, pl.a);
    else
      hipLaunchKernelGGL(gemm_f32_kernel<2>, grid, block, pl.lds_bytes, s, X, W, g.partial, g.M, g.N,
                         g.Kd, c.k_split, tx, ty, pl.a);
    return hipGetLastError();
  }
  if (c.kind != 6 || c.sk <= 0) return hipErrorInvalidConfiguration;
  const dim3 grid(unsigned(1 + c.sk)), block(256);
  if (pl.lds) hipLaunchKernelGGL((gemm_tile_plan_kernel<256, 128, 2, 2, 3, true>), grid, block, 0, s, g, pl.a);
  else hipLaunchKernelGGL((gemm_tile_plan_kernel<256, 128, 2, 2, 3, false>), grid, block, 0, s, g, pl.a);
  return hipGetLastError();
}

hipError_t launch_decode_slot_plan(const GemmConfig &c, const GemmArgs &g,
                                   const SlotShrinkArgs &ss, const PlanLaunch &pl, hipStream_t s) {
  if (c.kind != 4 || pl.lds_bytes > plan_lds_cap(c)) return hipErrorInvalidConfiguration;
  const int gx = (g.N + 127) / 128, gy = (g.M + c.bm - 1) / c.bm;
  const int n_gemm = gx * gy * c.splits;
  const dim3 grid(unsigned(1 + kSlotParts * ss.n_slots + n_gemm)), block(256);
  const bool m = ss.mask != nullptr;
#define LORA_DGS3(MB, M, L) \
  hipLaunchKernelGGL((decode_gemm_slot_kernel<MB, M, L>), grid, block, 0, s, g, ss, pl.a, gx, gy, n_gemm)
#define LORA_DGS2(MB, M) do { if (pl.lds) LORA_DGS3(MB, M, true); else LORA_DGS3(MB, M, false); } while (0)
#define LORA_DGS(MB) do { if (m) LORA_DGS2(MB, true); else LORA_DGS2(MB, false); } while (0)
  if (c.bm == 32) LORA_DGS(1);
  else if (c.bm == 64) LORA_DGS(2);
  else LORA_DGS(4);
#undef LORA_DGS
#undef LORA_DGS2
#undef LORA_DGS3
  return hipGetLastError();
}

// Row-major epilogue grid: one wave per (row, 512-column chunk), 4 waves a
// workgroup; with so few rows that this leaves CUs idle (decode), one wave a
// workgroup, so that the waves spread over every CU (64 tokens, 4096 ->
// 4096: 8.3 -> 7.7 us for the decode epilogue).
static hipError_t launch_epilogue_rows(const EpilogueArgs &e, const GemmArgs &g, int dtype,
                                       hipStream_t s) {
  const unsigned n_x = unsigned((g.N + 511) / 512);
  if (int64_t(n_x) * ((g.M + 3) / 4) < 256) {
    const dim3 grid(n_x, unsigned(g.M));
    if (dtype == LORA_BF16) hipLaunchKernelGGL((epilogue_kernel<uint16_t, 1>), grid, dim3(64), 0, s, e);
    else hipLaunchKernelGGL((epilogue_kernel<float, 1>), grid, dim3(64), 0, s, e);
  } else {
    const dim3 grid(n_x, unsigned((g.M + 3) / 4));
    if (dtype == LORA_BF16) hipLaunchKernelGGL((epilogue_kernel<uint16_t, 4>), grid, dim3(256), 0, s, e);
    else hipLaunchKernelGGL((epilogue_kernel<float, 4>), grid, dim3(256), 0, s, e);
  }
  return hipGetLastError();
}

hipError_t launch_grad_x_epilogue(const GemmConfig &c, const GemmArgs &g, int dtype,
                                  const uint8_t *mask, hipStream_t s) {
  if (c.fused) return hipErrorInvalidConfiguration;
  EpilogueArgs e{g.partial, c.splits, g.M, g.N, c.sk, g.Kd / 64, c.bm, c.bn, g.Y, g.ex, nullptr,
                 nullptr, 0, 0};
  if (mask == nullptr) return launch_epilogue_rows(e, g, dtype, s);
  e.mask = mask;
  const unsigned n_x = unsigned((g.N + 511) / 512);
  const dim3 grid(n_x, unsigned((g.M + 3) / 4));
  if (dtype == LORA_BF16) hipLaunchKernelGGL((epilogue_kernel<uint16_t, 4, true>), grid, dim3(256), 0, s, e);
  else hipLaunchKernelGGL((epilogue_kernel<float, 4, true>), grid, dim3(256), 0, s, e);
  return hipGetLastError();
}

hipError_t launch_epilogue_ucopy(const GemmConfig &c, const GemmArgs &g, int dtype,
                                 const float *slot_u, const int4 *sdesc, float *u_out,
                                 int64_t u_cap, hipStream_t s) {
  if (c.fused || c.kind != 4) return hipErrorInvalidConfiguration;
  EpilogueArgs e{g.partial, c.splits, g.M, g.N, c.sk, g.Kd / 64, c.bm, c.bn, g.Y, g.ex, sdesc,
                 nullptr, 0, 0};
  e.ex.U = slot_u;
  e.plan_sdesc = g.ex.slot_desc;                 // the plan's slot descriptors and header
  e.plan_hdr = const_cast<int32_t *>(g.ex.hdr);
  e.u_out = u_out;
  e.u_cap = u_cap;
  e.slot_stride = LORA_MAX_RANK;
  return launch_epilogue_rows(e, g, dtype, s);
}

hipError_t launch_epilogue(const GemmConfig &c, const GemmArgs &g, int dtype, hipStream_t s) {
  if (c.fused) return hipSuccess;
  EpilogueArgs e{g.partial, c.splits, g.M, g.N, c.sk, g.Kd / 64, c.bm, c.bn, g.Y, g.ex, nullptr,
                 nullptr, 0, 0};
  if (dtype == LORA_BF16 && c.kind == 6 && g.ex.K == 1 && g.ex.pair_tk) {
    // one slot per token: rows in pair order, 4 per workgroup (see EpilogueArgs;
    // 8-wave workgroups held 16 of the 20 waves a CU takes: 256 tokens,
    // 4096 -> 11008, 1024 adapters of ranks 8-128, 49.0 -> 45.3 us)
    const int n_x = (g.N + 511) / 512;
    e.pair_tk = g.ex.pair_tk;
    e.n_x = n_x;
    e.n_a = ((g.M + 3) / 4) * n_x;
    const dim3 grid(unsigned(2 * e.n_a));
    hipLaunchKernelGGL((epilogue_kernel<uint16_t, 4>), grid, dim3(256), 0, s, e);
    return hipGetLastError();
  }
  return launch_epilogue_rows(e, g, dtype, s);
}

}  // namespace lora
