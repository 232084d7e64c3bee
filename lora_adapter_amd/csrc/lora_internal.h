// Internal definitions shared by the HIP sources of liblora (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "lora.h"

namespace lora {

// ----------------------------------------------------------------- limits
constexpr int64_t kMaxPairs = int64_t(1) << 20;  // T*K: keeps prefix sums of ranks in int32
constexpr int kPlanThreads = 1024;
constexpr int kPlanLdsInts = 24576;               // LDS the plan kernel may use (96 KiB)
constexpr int kGradPairChunk = 256;               // pairs per partial in the gradient reduction
constexpr int kGradRankChunk = 16;                // rank rows per gradient register block
constexpr int kBigSegPairs = 64;                  // segments this large may use the MFMA shrink
constexpr int kTileTok = 32;                      // pairs per MFMA shrink tile (two 16-row blocks)
constexpr int kShrinkRows = 2;                    // rank rows per decode-shrink unit
constexpr int kShrinkWaves = 2048;                // waves of the decode shrink (its units split evenly)

// Plan header words after the LORA_PH_* ones (scheduling data for the shrink).
constexpr int kPhUnits = 8;          // decode-shrink units: sum over its segments of pairs x row groups
constexpr int kPhUnitsPerWave = 9;   // units per wave of the decode shrink
constexpr int kPhBig = 10;           // segments left to the MFMA shrink
constexpr int kPhSched = 11;         // 1: the decode-shrink wave records were built

// Segments of at least kBigSegPairs pairs go to the MFMA shrink when the
// operands are bf16, the batch is large and both projections' widths are
// multiples of 128 (the MFMA shrink splits d over four waves in steps of 32).
__host__ __device__ inline bool shrink_tile_enabled(int dtype, int64_t TK, int d_in, int d_out) {
  return dtype == LORA_BF16 && TK >= 512 && d_in % 128 == 0 && d_out % 128 == 0;
}

// ----------------------------------------------------------------- bf16
__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf2f(uint16_t v) { return __uint_as_float(uint32_t(v) << 16); }

// float32 -> bf16 by the hardware conversion: round to nearest even, a NaN
// gives a quiet NaN.
__device__ __forceinline__ uint16_t f2bf(float f) {
  const __bf16 h = (__bf16)f;          // v_cvt_pk_bf16_f32
  uint16_t u;
  __builtin_memcpy(&u, &h, 2);
  return u;
}

// Two values to bf16 in one hardware conversion (v_cvt_pk_bf16_f32, round to
// nearest even): a in bits 0-15, b in bits 16-31.
__device__ __forceinline__ uint32_t f2bf2(float a, float b) {
  typedef float f32x2_cvt_t __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2_cvt_t __attribute__((ext_vector_type(2)));
  const bf16x2_cvt_t h = __builtin_convertvector((f32x2_cvt_t){a, b}, bf16x2_cvt_t);
  uint32_t u;
  __builtin_memcpy(&u, &h, 4);
  return u;
}

// Element traits: storage type E is float (fp32) or uint16_t (bf16 bits).
template <typename E> struct Elem;
template <> struct Elem<float> {
  // 8 consecutive elements starting at p (32-byte aligned).
  static __device__ __forceinline__ void load8(const float *p, float v[8]) {
    const float4 a = *reinterpret_cast<const float4 *>(p);
    const float4 b = *reinterpret_cast<const float4 *>(p + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
  static __device__ __forceinline__ float load1(const float *p) { return *p; }
  static __device__ __forceinline__ void store1(float *p, float v) { *p = v; }
  static __device__ __forceinline__ float to_f(float v) { return v; }
  static __device__ __forceinline__ float from_f(float v) { return v; }
};
template <> struct Elem<uint16_t> {
  static __device__ __forceinline__ void load8(const uint16_t *p, float v[8]) {
    const uint4 a = *reinterpret_cast<const uint4 *>(p);
    v[0] = bf_lo(a.x); v[1] = bf_hi(a.x); v[2] = bf_lo(a.y); v[3] = bf_hi(a.y);
    v[4] = bf_lo(a.z); v[5] = bf_hi(a.z); v[6] = bf_lo(a.w); v[7] = bf_hi(a.w);
  }
  static __device__ __forceinline__ float load1(const uint16_t *p) { return bf2f(*p); }
  static __device__ __forceinline__ void store1(uint16_t *p, float v) { *p = f2bf(v); }
  static __device__ __forceinline__ float to_f(uint16_t v) { return bf2f(v); }
  static __device__ __forceinline__ uint16_t from_f(float v) { return f2bf(v); }
};

// ----------------------------------------------------------------- wave helpers
__device__ __forceinline__ int lane_id() { return __lane_id(); }

// Sum over the 64 lanes of a wave with a fixed butterfly (deterministic).
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// ----------------------------------------------------------------- plan layout
// Offsets in int32 units inside the plan buffer; every array 64-byte aligned.
struct PlanLayout {
  int64_t hdr, pair_tk, seg_adapter, seg_off, seg_row_off, bucket_seg_off, u_off, slot_pos;
  int64_t pair_adapter;
  int64_t pair_gate;  // [T*K] float bits: gate of each sorted pair
  int64_t seg_uoff;   // [S+1] first decode-shrink unit of each segment
  int64_t wave_start; // [kShrinkWaves] x 8 ints: {seg, unit in seg, adapter, rank}, {page_start, pair_begin, pair_end, 0}
  int64_t big_list;   // [1 + T*K/kBigSegPairs]: count, then the segments left to the MFMA shrink
  int64_t seg_desc;   // [S] x 8 ints: {adapter, rank, page_start, pair_begin, pair_end, u_begin, row_begin, 0}
  int64_t slot_desc;  // [T*K] x 4 ints: {pair or -1, rank, u_off, page_start}
  int64_t cnt, ubias, cur, ps, inf;  // per-adapter scratch (pools too big for LDS)
  int64_t wcnt;                      // per (bucket, round, wave) counts, same case
  int64_t total;
};

__host__ __device__ inline int64_t align16(int64_t x) { return (x + 15) & ~int64_t(15); }

// Per-bucket columns of the plan kernel's (round, wave) count table for any
// block size of 64..kPlanThreads threads: ceil(N / nt) * (nt / 64) <= ceil(N / 64) + 16.
__host__ __device__ inline int64_t plan_count_cols(int64_t N) {
  return (N + 63) / 64 + kPlanThreads / 64 + 1;
}

// Threads of the plan workgroup: one per slot or adapter (the larger count),
// rounded up to a power of two in 64..kPlanThreads, so that small batches run
// in few waves.
inline int plan_threads(int64_t TK, int64_t N) {
  const int64_t work = TK > N ? TK : N;
  int nt = 64;
  while (nt < kPlanThreads && nt < work) nt *= 2;
  return nt;
}

__host__ __device__ inline PlanLayout plan_layout(int64_t TK, int64_t N) {
  PlanLayout L;
  int64_t o = 0;
  L.hdr = o;            o = align16(o + LORA_PLAN_HEADER_INTS);
  L.pair_tk = o;        o = align16(o + TK);
  L.seg_adapter = o;    o = align16(o + TK);
  L.seg_off = o;        o = align16(o + TK + 1);
  L.seg_row_off = o;    o = align16(o + TK + 1);
  L.bucket_seg_off = o; o = align16(o + 16);
  L.u_off = o;          o = align16(o + TK + 1);
  L.slot_pos = o;       o = align16(o + TK);
  L.pair_adapter = o;   o = align16(o + TK);
  L.pair_gate = o;      o = align16(o + TK);
  L.seg_uoff = o;       o = align16(o + TK + 1);
  L.wave_start = o;     o = align16(o + 8 * kShrinkWaves);
  L.big_list = o;       o = align16(o + 1 + TK / kBigSegPairs + 1);
  L.seg_desc = o;       o = align16(o + 8 * TK);
  L.slot_desc = o;      o = align16(o + 4 * TK);
  L.cnt = o;            o = align16(o + N);
  L.ubias = o;          o = align16(o + N);
  L.cur = o;            o = align16(o + N);
  L.ps = o;             o = align16(o + N);
  L.inf = o;            o = align16(o + N);
  L.wcnt = o;           o = align16(o + LORA_N_BUCKETS * plan_count_cols(N));
  L.total = o;
  return L;
}

// Read-only view of a built plan.
struct PlanView {
  const int32_t *hdr, *pair_tk, *seg_adapter, *seg_off, *seg_row_off, *u_off, *slot_pos;
  const int32_t *pair_adapter;
  const int4 *seg_desc;    // two int4 per segment
  const int4 *slot_desc;   // one int4 per slot
  const float *pair_gate;  // gate of each sorted pair
  const int4 *wave_start;  // two int4 per decode-shrink wave
  const int32_t *big_list; // count, then segment ids
  const int32_t *seg_uoff; // first decode-shrink unit of each segment
};

inline PlanView plan_view(const void *plan, int64_t TK, int64_t N) {
  const PlanLayout L = plan_layout(TK, N);
  const int32_t *b = static_cast<const int32_t *>(plan);
  return PlanView{b + L.hdr, b + L.pair_tk, b + L.seg_adapter, b + L.seg_off,
                  b + L.seg_row_off, b + L.u_off, b + L.slot_pos, b + L.pair_adapter,
                  reinterpret_cast<const int4 *>(b + L.seg_desc),
                  reinterpret_cast<const int4 *>(b + L.slot_desc),
                  reinterpret_cast<const float *>(b + L.pair_gate),
                  reinterpret_cast<const int4 *>(b + L.wave_start), b + L.big_list,
                  b + L.seg_uoff};
}

// Device view of an adapter pool.
struct PoolView {
  const void *a_pages, *b_pages;
  const int32_t *rank, *page_start, *page_ids;
  const float *scale;
  int64_t n_pages, n_page_ids;
  int d_in, d_out, n_adapters, dtype;
};

inline PoolView pool_view(const lora_pool_desc *p) {
  return PoolView{p->a_pages, p->b_pages, p->rank, p->page_start, p->page_ids, p->scale,
                  p->n_pages, p->n_page_ids, p->d_in, p->d_out, p->n_adapters, p->dtype};
}

// ----------------------------------------------------------------- kernel arguments

// Segmented shrink: out[u_off[p] + j] = coef_p * sum_i Z[t_p][i] (m[t_p][i]) page_j[i]
// for every planned pair p and rank row j of its adapter, with coef_p =
// gate_p * (scale[a] * extra_scale) (gate_p as recorded by the plan).  Used for
// the LoRA down projection (Z = X, pages = A) and for the gradient's dY.B^T
// (Z = dY, pages = B).
struct ShrinkArgs {
  const void *Z;            // [T][d] activations
  const uint8_t *mask;      // [T][d] 0/1 or null
  float extra_scale;
  int T, K, d;
  const void *pages;        // [n_pages][d]
  const int32_t *rank, *page_start, *page_ids;
  const float *scale;
  const float *gates;       // [T][K]
  PlanView plan;
  int32_t *err_word;        // plan header word for device errors
  float *out;
  int64_t out_cap;          // capacity of out in floats
  int big_segments;         // set by the launcher: large segments go to the MFMA tile kernel
                            // (the plan made the same choice from the same predicate)
};

// Per-slot decode shrink (no plan): out[i * stride + j] for slot i = t*K + k
// and rank row j of the slot's adapter, when the slot is active and its
// adapter's page table is consistent (other entries are left untouched).
struct SlotShrinkArgs {
  const int32_t *ids;       // [T][K]
  const float *gates;       // [T][K]
  int K, N;
  const void *Z;            // [T][d] bf16
  const uint8_t *mask;      // [T][d] 0/1 or null
  float extra_scale;
  int d;
  const void *pages;        // [n_pages][d]
  const int32_t *rank, *page_start, *page_ids;
  const float *scale;
  int64_t n_pages, n_page_ids;
  float *out;
  int stride;               // floats per slot (LORA_MAX_RANK)
  int n_slots;              // T*K
  int4 *sdesc;              // [T*K] {slot, rank, slot*stride, page_start} or {-1,0,0,0}
};

// Everything the expand needs to add sum_j U[u_off[p]+j] * B_a[j][n] to row t.
struct ExpandArgs {
  int K;
  const int4 *slot_desc;    // per slot {pair or -1, rank, u_off, page_start}
  const int32_t *pair_tk;   // the plan's pair order (t*K + k of each sorted pair)
  const int32_t *page_ids;
  const void *b_pages;      // [n_pages][d_out]
  int d_out;
  const float *U;
  const int32_t *hdr;       // plan header (R_pairs)
  int64_t u_cap;
};

struct GemmArgs {
  const void *X;            // [M][Kd]
  const void *W;            // [N][Kd]
  int M, N, Kd;
  int k_split;              // K elements per split (multiple of 64)
  int sk_g;                 // > 0: stream-K over this many workgroups (see the tile GEMM)
  float *partial;           // [splits][M][N]
  void *Y;                  // fused epilogue output [M][N]
  ExpandArgs ex;
  // not null (fused 256 x 256 tiles only): keep mask [M][N] of 0/1 bytes that
  // multiplies the expand term before the rounding (the input gradient)
  const uint8_t *mask;
};

struct EpilogueArgs {
  const float *partial;     // [splits][M][N]
  int splits, M, N;
  int sk_g, sk_kt, bm, bn;  // stream-K: workgroups, K tiles per output tile, tile shape
  void *Y;
  ExpandArgs ex;
  // not null: ex.U holds U per slot and sdesc the slot descriptors written by
  // the per-slot shrink; the plan is not read (lora_forward's decode path)
  const int4 *sdesc;
  // not null (one slot per token, plan available): rows in the plan's pair
  // order, 4 consecutive pairs per workgroup (one per wave), so the rows of
  // one adapter in a workgroup share its B lines in the CU's caches (1-D
  // grid: n_a workgroups of pair rows over n_x column chunks, then the rows
  // without an active slot in token order)
  const int32_t *pair_tk;
  int n_x, n_a;
  // not null (decode, with sdesc): the plan built by the previous launch;
  // the first column chunk of each row copies the row's per-slot U (ex.U,
  // rows of slot_stride floats) to the plan's u_off places, when the plan's
  // R_pairs fits u_cap (else LORA_DEVERR_CAPACITY in plan_hdr's error word)
  const int4 *plan_sdesc;
  int32_t *plan_hdr;
  float *u_out;
  int64_t u_cap;
  int slot_stride;
  // not null (input gradient dX): the expand term (G . A pages) is multiplied
  // element-wise by this [M][N] 0/1 keep mask before it is added
  const uint8_t *mask;
};

struct MergeArgs {
  void *W;                  // [d_out][d_in]
  int d_in, d_out;
  const void *a_pages, *b_pages;
  const int32_t *rank, *page_start, *page_ids;
  const float *scale;
  int64_t n_pages, n_page_ids;
  int n_adapters;
  const int32_t *ids;
  const float *coeffs;
  int m;
};

// Gradient outer-product reduction over the pairs of each segment:
// out_page(a, j)[c] = sum_{p of a} coef[u_off[p] + j] * Z[t_p][c] (* m[t_p][c]).
struct SegOuterArgs {
  const void *Z;            // [T][d]
  const uint8_t *mask;      // [T][d] or null
  int T, K, d;
  const float *coef;        // packed like U
  int64_t coef_cap;         // floats available at coef
  PlanView plan;
  const int32_t *rank, *page_start, *page_ids;
  float *part;              // [pieces][max_rank][d]
  int max_rank;
  float *out_pages;         // [n_pages][d]
  int32_t *err_word;
  // not null (dB pass of the MFMA form): also the partial dY.B^T of every
  // pair over each 256-column tile, gpart[tile][pair][max_rank], from the
  // staged dY rows and the B pages (b_pages)
  float *gpart;
  const void *b_pages;
};

// G from gpart: G[u_off[p] + j] = (gate_p . scale_a . extra_scale) .
// sum over the column tiles (in tile order) of gpart[tile][p][j].
struct GReduceArgs {
  const float *gpart;
  int n_tiles;
  int64_t TK;
  int max_rank;
  PlanView plan;
  const int32_t *rank;
  const float *scale;
  float extra_scale;
  float *G;
  int64_t g_cap;
};

// Arguments of the plan workgroup (plan_build).
struct PlanArgs {
  const int32_t *ids;
  const float *gates;
  int T, K, N;
  const int32_t *rank, *page_start, *page_ids;
  int64_t n_pages, n_page_ids;
  int32_t *plan;
  int slot_cache;    // 1: per-slot adapters and gates cached in LDS
  int use_tile;      // 1: segments of >= kBigSegPairs pairs go to the MFMA shrink
  int page_cache;    // 1: the page table is copied to LDS (after the slot cache)
  int no_sched;      // 1: skip the decode-shrink wave records (header word kPhSched = 0)
  int place_table;   // placement counts in LDS (after the page table) per 1: (wave, adapter),
                     // 2: (chunk of slots, wave, adapter); 0: none
  // not null: U per slot (stride slot_stride) to be stored in the u_off layout
  // at u_out when the plan's R_pairs <= u_cap (else LORA_DEVERR_CAPACITY)
  const float *slot_u;
  float *u_out;
  int64_t u_cap;
  int slot_stride;
};

// A plan workgroup's arguments and LDS use for a block of nt threads with
// lds_cap bytes of LDS: the per-adapter arrays go to LDS (lds) when they fit
// there, else to the plan buffer's scratch; the per-slot adapter cache, then
// the page table, go to LDS when they fit too.  lds_bytes: LDS the plan
// workgroup uses.
struct PlanLaunch {
  PlanArgs a;
  bool lds;
  size_t lds_bytes;
};
PlanLaunch plan_setup(const int32_t *ids, const float *gates, int T, int K, const PoolView &pool,
                      int32_t *plan, int nt, size_t lds_cap);

// ----------------------------------------------------------------- launchers
// Each returns hipSuccess or the launch error.
hipError_t launch_plan(const int32_t *ids, const float *gates, int T, int K, const PoolView &pool,
                       int32_t *plan, hipStream_t s);
// d_in and d_out of the pool decide, with dtype and T*K, whether the MFMA
// shrink takes the big segments (shrink_tile_enabled, as in the plan).
hipError_t launch_shrink(const ShrinkArgs &a, int dtype, int64_t TK, int64_t n_adapters,
                         int d_in, int d_out, hipStream_t s);

// Base GEMM configuration chosen from the shape (host-side, deterministic).
struct GemmConfig {
  int kind;      // 0: fp32 tiles; 4: bf16 decode; 5: bf16 256x256 fused; 6: bf16 256x128 split
  int bm, bn;
  int splits;    // partial slots per output element
  int k_split;
  int sk;        // > 0: stream-K workgroups (splits = most pieces of one tile)
  bool fused;    // expand + rounding in the GEMM epilogue (splits == 1 only)
};
GemmConfig choose_gemm(int T, int d_in, int d_out, int dtype);
size_t gemm_partial_bytes(const GemmConfig &c, int T, int d_out);
hipError_t launch_base_gemm(const GemmConfig &c, const GemmArgs &g, hipStream_t s);
hipError_t launch_epilogue(const GemmConfig &c, const GemmArgs &g, int dtype, hipStream_t s);
// The decode GEMM (kind 4) can run the decode shrink in the same launch when
// d_in <= 4096 (the shrink's rank rows then stay in registers within the
// register budget of two workgroups per CU).
bool decode_shrink_fusable(const GemmConfig &c, int d_in);
// Decode GEMM + decode shrink (the big-segment MFMA shrink, if enabled, is
// launched separately by the caller).
hipError_t launch_decode_gemm_shrink(const GemmConfig &c, const GemmArgs &g, const ShrinkArgs &sa,
                                     hipStream_t s);
// lora_forward's launches for split GEMMs.  Decode (kind 4): the plan
// (built by the launch's first workgroup, in the token-row LDS), the per-slot
// shrink (ss) and the GEMM's partials in one launch (launch_decode_slot_plan),
// then the epilogue from the slot descriptors, which also moves the per-slot
// U to the plan's layout (launch_epilogue_ucopy).  Stream-K (kind 6) and fp32
// (kind 0): the GEMM's partials with the plan built by one more workgroup
// (launch_gemm_plan).  The plan workgroup has 256 threads and the LDS that
// plan_lds_cap(c) gives.
bool gemm_plan_fusable(const GemmConfig &c);
size_t plan_lds_cap(const GemmConfig &c);
hipError_t launch_gemm_plan(const GemmConfig &c, const GemmArgs &g, const PlanLaunch &pl,
                            hipStream_t s);
hipError_t launch_decode_slot_plan(const GemmConfig &c, const GemmArgs &g,
                                   const SlotShrinkArgs &ss, const PlanLaunch &pl, hipStream_t s);
hipError_t launch_epilogue_ucopy(const GemmConfig &c, const GemmArgs &g, int dtype,
                                 const float *slot_u, const int4 *sdesc, float *u_out,
                                 int64_t u_cap, hipStream_t s);
// The MFMA shrink of the big segments alone (no-op unless enabled).
hipError_t launch_shrink_big(const ShrinkArgs &a, int dtype, int64_t TK, int64_t n_adapters,
                             int d_in, int d_out, hipStream_t s);

// Input gradient: the epilogue of the dX GEMM (dY . W^T as split partials),
// with the expand term from G and the A pages times the keep mask (if any).
hipError_t launch_grad_x_epilogue(const GemmConfig &c, const GemmArgs &g, int dtype,
                                  const uint8_t *mask, hipStream_t s);
// dst[c][r] = src[r][c] for a rows x cols matrix of the dtype.
hipError_t launch_transpose(const void *src, void *dst, int rows, int cols, int dtype,
                            hipStream_t s);

// Batched tall-skinny QR (see tsqr.hip).
bool tsqr_shape_ok(int M, int m, int n);
size_t tsqr_workspace_bytes(int M, int m, int n);
hipError_t launch_tsqr(const void *src, int dtype, const int32_t *cols, int M, int m, int n,
                       float *Qt, float *R, void *ws, hipStream_t s);

// Retained-rank recompression (see compress.hip).
size_t compress_workspace_bytes(int M, int d_in, int d_out, int n);
hipError_t launch_compress(const PoolView &pool, const int32_t *adapters, int M, int n, int policy,
                           float ratio, float energy, int floor_rank, void *out_a, void *out_b,
                           int32_t *out_rank, float *out_sigma, void *ws, hipStream_t s);

hipError_t launch_merge(const MergeArgs &a, int dtype, hipStream_t s);
// n layers' merges (same list, each layer's own W and pool): one launch per
// LORA_MERGE_MAX_LAYERS layers when every layer takes the MFMA form.
hipError_t launch_merge_layers(const MergeArgs *layers, int n, int dtype, hipStream_t s);
int64_t grad_pieces(int64_t TK, int64_t n_adapters);
// The MFMA outer-product form (and the fused dY.B^T partials) applies.
bool grad_mfma_form(int dtype, int64_t TK, int d_out);
int grad_gpart_tiles(int d_out);
// The outer products, then the chunk partials' reduction; with g, the
// reduction launch also forms G from gpart.
hipError_t launch_seg_outer(const SegOuterArgs &a, int dtype, int64_t TK, int64_t n_adapters,
                            hipStream_t s, const GReduceArgs *g = nullptr);

}  // namespace lora
