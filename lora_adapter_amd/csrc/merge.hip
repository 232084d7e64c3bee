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
    *reinterpret_cast<uint2 *>(p) = make_uint2(f2bf2(v[0], v[1]),
                                               f2bf2(v[2], v[3]));
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

// ------------------------------------------------------------ bf16 MFMA form
// The delta of W_t is a product with the rank rows as K:
//   delta[n][i] = sum_j A_j[i] . (c_j B_j[n])
// computed with v_mfma_f32_32x32x16_bf16, M = i, N = n.  A pages are bf16
// already (exact operands); c_j B_j[n] is formed in float32 and split into
// bf16 high and low parts (two MFMAs), which keeps ~16 bits of it.  MFMA
// rows are assigned to W columns so that every lane ends with 16 consecutive
// columns of one W row: its W values load and store as 16-byte pieces.
// One workgroup per 128 x 128 rectangle of W_t: its W values are requested
// first, then the rectangle's slices of the listed A and B rows are staged in
// LDS (transposed, rank rows contiguous), 64 rank rows at a time; wave w
// owns rows 32 w .. 32 w + 31 of the rectangle.
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

constexpr int kQN = 128;           // W rows per workgroup (4 waves x 32)
constexpr int kQI = 128;           // W columns per workgroup
constexpr int kQR = 64;            // rank rows per staged chunk
constexpr int kQB = kQI / 32;      // 32-column MFMA blocks per wave

// 16-byte chunk c (8 rank rows) of staged row x sits at chunk c ^ ((x >> 1) & 7):
// 16 consecutive rows read the same chunk without bank conflicts.
__device__ __forceinline__ int qswz(int x, int c) { return c ^ ((x >> 1) & 7); }

// 8 x 8 bf16 transpose in registers: in[r] holds row r (8 values, 2 per
// word); out[c] holds column c.  Each output word takes one half of a word
// of two input rows (v_perm_b32).
__device__ __forceinline__ uint32_t word_of(const uint4 &v, int q) {
  return q == 0 ? v.x : q == 1 ? v.y : q == 2 ? v.z : v.w;
}
__device__ __forceinline__ void transpose8(const uint4 (&in)[8], uint4 (&out)[8]) {
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    uint32_t w[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t lo = word_of(in[2 * q], c >> 1), hi = word_of(in[2 * q + 1], c >> 1);
      // even c: the low halves of (lo, hi); odd c: the high halves
      w[q] = __builtin_amdgcn_perm(hi, lo, (c & 1) ? 0x07060302u : 0x05040100u);
    }
    out[c] = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

// Stages listed rank rows [j0, j0 + nl) (zero past nl):
//   s_at[i][j] = A_j[i0 + i]                          i < 128
//   s_bh[n][j] + s_bl[n][j] = c_j B_j[n0 + n]          n < 128
// Threads 0..127 transpose one (8 rows, 8 columns) block of A each, threads
// 128..255 one block of B.
__device__ __forceinline__ void qstage(const MergeArgs &m, int i0, int n0, int j0, int nl,
                                       const int *s_pid, const float *s_cf,
                                       uint4 (*s_at)[8], uint4 (*s_bh)[8], uint4 (*s_bl)[8]) {
  const int tid = threadIdx.x;
  const bool is_b = tid >= 128;
  const int jg = tid & 7, xg = (tid & 127) >> 3;
  const uint16_t *src = static_cast<const uint16_t *>(is_b ? m.b_pages : m.a_pages);
  const int64_t len = is_b ? m.d_out : m.d_in;
  const int x0 = (is_b ? n0 : i0) + xg * 8;
  uint4 rw[8], t[8];
  float cf[8];
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    const int j = jg * 8 + r;
    const bool ok = j < nl;
    cf[r] = ok ? s_cf[j0 + j] : 0.f;
    rw[r] = make_uint4(0u, 0u, 0u, 0u);
    if (ok) rw[r] = *reinterpret_cast<const uint4 *>(src + int64_t(s_pid[j0 + j]) * len + x0);
  }
  if (!is_b) {
    transpose8(rw, t);
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const int i = xg * 8 + c;
      s_at[i][qswz(i, jg)] = t[c];
    }
    return;
  }
  // c_j B_j[n] in float32 (after the transpose: word q of column c holds rank
  // rows 2q and 2q + 1), split into bf16 high and low parts
  transpose8(rw, t);
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    const int n = xg * 8 + c;
    const uint32_t w[4] = {t[c].x, t[c].y, t[c].z, t[c].w};
    uint32_t hw[4], lw[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float x0 = cf[2 * q] * bf_lo(w[q]), x1 = cf[2 * q + 1] * bf_hi(w[q]);
      hw[q] = f2bf2(x0, x1);
      lw[q] = f2bf2(x0 - bf_lo(hw[q]), x1 - bf_hi(hw[q]));
    }
    s_bh[n][qswz(n, jg)] = make_uint4(hw[0], hw[1], hw[2], hw[3]);
    s_bl[n][qswz(n, jg)] = make_uint4(lw[0], lw[1], lw[2], lw[3]);
  }
}

// acc[b] += the staged chunk's product for MFMA block b (columns 32 b ..) of
// this wave's 32 rows.
__device__ __forceinline__ void qmfma(int nl, const uint4 (*s_at)[8], const uint4 (*s_bh)[8],
                                      const uint4 (*s_bl)[8], f32x16_t (&acc)[kQB]) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int m = lane & 31, g = lane >> 5;
  const int n = wave * 32 + m;
  // MFMA row m -> W column 16 (m >> 4) + 8 ((m >> 2) & 1) + 4 ((m >> 3) & 1) + (m & 3)
  const int icol = 16 * (m >> 4) + 8 * ((m >> 2) & 1) + 4 * ((m >> 3) & 1) + (m & 3);
  for (int k = 0; k < nl; k += 16) {
    const int c = (k >> 3) + g;
    bf16x8_t bh, bl;
    __builtin_memcpy(&bh, &s_bh[n][qswz(n, c)], 16);
    __builtin_memcpy(&bl, &s_bl[n][qswz(n, c)], 16);
#pragma unroll
    for (int b = 0; b < kQB; ++b) {
      const int i = b * 32 + icol;
      bf16x8_t a;
      __builtin_memcpy(&a, &s_at[i][qswz(i, c)], 16);
      acc[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bh, acc[b], 0, 0, 0);
      acc[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bl, acc[b], 0, 0, 0);
    }
  }
}

// Barrier for LDS traffic only: global loads in flight stay in flight.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Streaming form, for merge lists of at most kQR valid rank rows (all staged
// at once): workgroup w takes a contiguous range of 64 x 128 rectangles of
// one 128-column slice (its A slice is staged once) and keeps kSD of them in
// flight in registers: the W rectangle (coalesced 16-byte
// loads, 4 rows x 256 bytes per wave instruction) and the 64 x 64 B block.
// Per rectangle: W goes to LDS (16-byte slots swizzled by row), c.B to
// bf16 high/low parts in LDS, the MFMA delta is added in the lane layout,
// and the rounded rectangle is read back and stored with the same coalesced
// pattern.
constexpr int kSN = 64;            // W rows per rectangle
constexpr int kSD = 3;             // rectangles in flight per workgroup

__device__ __forceinline__ void merge_stream(const MergeArgs &m, int total, uint4 *raw,
                                             const int *s_pid, const float *s_cf, int bid,
                                             int nblk) {
  uint4 (*s_at)[8] = reinterpret_cast<uint4 (*)[8]>(raw);            // [128 i][64 j]
  uint32_t (*s_bh)[32] = reinterpret_cast<uint32_t (*)[32]>(raw + 1024);   // [64 n][64 j]
  uint32_t (*s_bl)[32] = reinterpret_cast<uint32_t (*)[32]>(raw + 1536);
  uint4 (*wbuf)[16] = reinterpret_cast<uint4 (*)[16]>(raw + 2048);   // [64 rows][256 bytes]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nrn = m.d_out / kSN;
  const int gx = m.d_in / kQI;
  // workgroup -> (column slice, part of its rectangles): nblk = gx * gps
  const int gps = nblk / gx;
  const int slice = bid / gps, part = bid % gps;
  const int beg = nrn * part / gps, end = nrn * (part + 1) / gps;   // rectangle rows of the slice
  if (slice >= gx || beg >= end) return;
  const int i0 = slice * kQI;
  uint16_t *W = static_cast<uint16_t *>(m.W);
  const uint16_t *Ap = static_cast<const uint16_t *>(m.a_pages);
  const uint16_t *Bp = static_cast<const uint16_t *>(m.b_pages);
  // this thread's B pieces: rank rows 2 jp and 2 jp + 1, columns n0 + 8 nc .. + 7
  const int jp = tid >> 3, nc = tid & 7;
  const bool oka = 2 * jp < total, okb = 2 * jp + 1 < total;
  const int64_t pga = s_pid[oka ? 2 * jp : 0], pgb = s_pid[okb ? 2 * jp + 1 : 0];
  const float ca = oka ? s_cf[2 * jp] : 0.f, cb = okb ? s_cf[2 * jp + 1] : 0.f;
  // this thread's W pieces: rows (tid / 16) + 16 e, 16-byte chunk tid % 16
  const int wr0 = tid >> 4, wc = tid & 15;
  if (tid < 128) {
    // the A slice: threads 0..127 transpose one (8 rank rows, 8 columns) block each
    const int jg = tid & 7, xg = tid >> 3;
    uint4 rw[8], t[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int j = jg * 8 + q;
      const int64_t pg = s_pid[j < total ? j : 0];
      rw[q] = *reinterpret_cast<const uint4 *>(Ap + pg * m.d_in + i0 + xg * 8);
      if (j >= total) rw[q] = make_uint4(0u, 0u, 0u, 0u);
    }
    transpose8(rw, t);
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const int i = xg * 8 + c;
      s_at[i][qswz(i, jg)] = t[c];
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  auto load_rect = [&](int r, u32x4 (&wv)[4], u32x4 &ba, u32x4 &bb) __attribute__((always_inline)) {
    const int n0 = min(r, end - 1) * kSN;   // past the range: a harmless reload, never used
#pragma unroll
    for (int e = 0; e < 4; ++e)
      wv[e] = *reinterpret_cast<const u32x4 *>(W + int64_t(n0 + wr0 + 16 * e) * m.d_in + i0 + 8 * wc);
    ba = *reinterpret_cast<const u32x4 *>(Bp + pga * m.d_out + n0 + 8 * nc);
    bb = *reinterpret_cast<const u32x4 *>(Bp + pgb * m.d_out + n0 + 8 * nc);
  };
  // MFMA roles: rows 32 (wave & 1) .. of the rectangle, columns 64 (wave >> 1) ..
  const int mrow = lane & 31, g = lane >> 5;
  const int nrow = 32 * (wave & 1) + mrow;
  const int ih = wave >> 1;
  const int icol = 16 * (mrow >> 4) + 8 * ((mrow >> 2) & 1) + 4 * ((mrow >> 3) & 1) + (mrow & 3);
  // Every workgroup runs whole groups of kSD steps (a step past its range
  // only keeps the barriers and reissues a clamped load), so the three slots
  // stay three distinct register sets.
  auto step = [&](int r, u32x4 (&wv)[4], u32x4 &ba, u32x4 &bb) __attribute__((always_inline)) {
    const bool valid = r < end;
    const int n0 = min(r, end - 1) * kSN;
    lds_barrier();                     // the previous rectangle is done with the LDS tiles
    if (valid) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = wr0 + 16 * e;
        wbuf[row][wc ^ (row & 15)] = make_uint4(wv[e][0], wv[e][1], wv[e][2], wv[e][3]);
      }
      const uint32_t wa[4] = {ba[0], ba[1], ba[2], ba[3]}, wb[4] = {bb[0], bb[1], bb[2], bb[3]};
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const uint32_t va = wa[u >> 1], vb = wb[u >> 1];
        const float xa = oka ? ca * ((u & 1) ? bf_hi(va) : bf_lo(va)) : 0.f;
        const float xb = okb ? cb * ((u & 1) ? bf_hi(vb) : bf_lo(vb)) : 0.f;
        const uint32_t h2 = f2bf2(xa, xb);
        const int n = 8 * nc + u;
        const int word = qswz(n, jp >> 2) * 4 + (jp & 3);
        s_bh[n][word] = h2;
        s_bl[n][word] = f2bf2(xa - bf_lo(h2), xb - bf_hi(h2));
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    load_rect(r + kSD, wv, ba, bb);
    __builtin_amdgcn_sched_barrier(0);
    lds_barrier();
    if (valid) {
      f32x16_t acc[2];
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[b][v] = 0.f;
      for (int k = 0; k < total; k += 16) {
        const int c = (k >> 3) + g;
        bf16x8_t bh, bl;
        __builtin_memcpy(&bh, &s_bh[nrow][qswz(nrow, c) * 4], 16);
        __builtin_memcpy(&bl, &s_bl[nrow][qswz(nrow, c) * 4], 16);
#pragma unroll
        for (int b = 0; b < 2; ++b) {
          const int i = 64 * ih + 32 * b + icol;
          bf16x8_t av;
          __builtin_memcpy(&av, &s_at[i][qswz(i, c)], 16);
          acc[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bh, acc[b], 0, 0, 0);
          acc[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bl, acc[b], 0, 0, 0);
        }
      }
      // lane value v of block b: column 64 ih + 32 b + 16 (v / 8) + 8 g + (v % 8) of row nrow
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          const int c = 8 * ih + 4 * b + 2 * q + g;
          uint4 &slot = wbuf[nrow][c ^ (nrow & 15)];
          const uint4 wvv = slot;
          const uint32_t w[4] = {wvv.x, wvv.y, wvv.z, wvv.w};
          uint32_t o[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float lo = bf_lo(w[e]) + acc[b][8 * q + 2 * e];
            const float hi = bf_hi(w[e]) + acc[b][8 * q + 2 * e + 1];
            o[e] = f2bf2(lo, hi);
          }
          slot = make_uint4(o[0], o[1], o[2], o[3]);
        }
    }
    lds_barrier();
    if (valid) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = wr0 + 16 * e;
        // streaming store: the merged W is not read again by this launch
        const uint4 o = wbuf[row][wc ^ (row & 15)];
        const u32x4 ov = {o.x, o.y, o.z, o.w};
        __builtin_nontemporal_store(ov, reinterpret_cast<u32x4 *>(W + int64_t(n0 + row) * m.d_in + i0 + 8 * wc));
      }
    }
  };
  u32x4 w0[4], w1[4], w2[4], b0a, b0b, b1a, b1b, b2a, b2b;
  load_rect(beg, w0, b0a, b0b);
  __builtin_amdgcn_sched_barrier(0);
  load_rect(beg + 1, w1, b1a, b1b);
  __builtin_amdgcn_sched_barrier(0);
  load_rect(beg + 2, w2, b2a, b2b);
  __builtin_amdgcn_sched_barrier(0);
  for (int r = beg; r < end; r += kSD) {
    step(r, w0, b0a, b0b);
    step(r + 1, w1, b1a, b1b);
    step(r + 2, w2, b2a, b2b);
  }
}

// General form (any merge list): workgroup w of G = nblk takes 128 x 128
// rectangles w, w + G, ...; the merge list is built once per workgroup when
// it fits one LDS list.  Lists of at most kQR rank rows take the streaming
// form.
__device__ __forceinline__ void merge_mfma_body(const MergeArgs &m, int bid, int nblk, uint4 *raw,
                                                int *s_pid, float *s_cf, int *s_tot) {
  uint4 (*s_at)[8] = reinterpret_cast<uint4 (*)[8]>(raw);
  uint4 (*s_bh)[8] = reinterpret_cast<uint4 (*)[8]>(raw + 1024);
  uint4 (*s_bl)[8] = reinterpret_cast<uint4 (*)[8]>(raw + 2048);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int gx = m.d_in / kQI;
  const int nrect = gx * (m.d_out / kQN);
  uint16_t *W = static_cast<uint16_t *>(m.W);
  const bool one_list = m.m <= kMAd;
  int total = 0;
  if (one_list) {
    total = merge_list(m, 0, 0, s_pid, s_cf, s_tot);
    if (total == 0) return;                 // nothing valid listed: W stays as it is
    if (total <= kQR) {
      merge_stream(m, total, raw, s_pid, s_cf, bid, nblk);
      return;
    }
  }
  const bool resident = one_list && total <= kMList;
  // lane's W pieces: row n0 + 32 wave + (lane % 32), columns i0 + 32 b + 16 q + 8 (lane / 32)
  auto wptr = [&](int rect) __attribute__((always_inline)) {
    const int i0 = (rect % gx) * kQI, n0 = (rect / gx) * kQN;
    return W + int64_t(n0 + wave * 32 + (lane & 31)) * m.d_in + i0 + 8 * (lane >> 5);
  };
  auto wload = [&](int rect, uint4 (&wv)[kQB][2]) __attribute__((always_inline)) {
    const uint16_t *p = wptr(rect);
#pragma unroll
    for (int b = 0; b < kQB; ++b)
#pragma unroll
      for (int q = 0; q < 2; ++q) wv[b][q] = *reinterpret_cast<const uint4 *>(p + 32 * b + 16 * q);
  };
  uint4 wv[kQB][2];
  bool any = resident;
  for (int rect = bid; rect < nrect; rect += nblk) {
    const int i0 = (rect % gx) * kQI, n0 = (rect / gx) * kQN;
    wload(rect, wv);
    f32x16_t acc[kQB];
#pragma unroll
    for (int b = 0; b < kQB; ++b)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[b][v] = 0.f;
    if (resident) {
      for (int j0 = 0; j0 < total; j0 += kQR) {
        const int nl = min(kQR, total - j0);
        __syncthreads();                    // the previous chunk's reads are done
        qstage(m, i0, n0, j0, nl, s_pid, s_cf, s_at, s_bh, s_bl);
        __syncthreads();
        qmfma(nl, s_at, s_bh, s_bl, acc);
      }
    } else {
      for (int e0 = 0; e0 < m.m; e0 += kMAd) {
        const int tot = merge_list(m, e0, 0, s_pid, s_cf, s_tot);
        for (int lb = 0; lb < tot; lb += kMList) {
          if (lb > 0) merge_list(m, e0, lb, s_pid, s_cf, s_tot);
          const int nlist = min(kMList, tot - lb);
          for (int j0 = 0; j0 < nlist; j0 += kQR) {
            const int nl = min(kQR, nlist - j0);
            __syncthreads();
            qstage(m, i0, n0, j0, nl, s_pid, s_cf, s_at, s_bh, s_bl);
            __syncthreads();
            qmfma(nl, s_at, s_bh, s_bl, acc);
            any = true;
          }
        }
      }
    }
    if (any) {
      // lane value v of block b: column 32 b + 16 (v / 8) + 8 (lane / 32) + (v % 8)
      uint16_t *p = wptr(rect);
#pragma unroll
      for (int b = 0; b < kQB; ++b)
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          const uint32_t w[4] = {wv[b][q].x, wv[b][q].y, wv[b][q].z, wv[b][q].w};
          uint32_t o[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float lo = bf_lo(w[e]) + acc[b][8 * q + 2 * e];
            const float hi = bf_hi(w[e]) + acc[b][8 * q + 2 * e + 1];
            o[e] = f2bf2(lo, hi);
          }
          *reinterpret_cast<uint4 *>(p + 32 * b + 16 * q) = make_uint4(o[0], o[1], o[2], o[3]);
        }
    }
  }
}

__global__ __launch_bounds__(256) void merge_mfma_kernel(MergeArgs m) {
  __shared__ uint4 raw[3072];
  __shared__ int s_pid[kMList];
  __shared__ float s_cf[kMList];
  __shared__ int s_tot[4];
  merge_mfma_body(m, int(blockIdx.x), int(gridDim.x), raw, s_pid, s_cf, s_tot);
}

// Several layers' merges in one launch (AdaFuse notes, section 关键设计 item
// 3: the merges of every layer packed into one batched launch, blocked across
// layers, added in place): layer blockIdx.y, its own workgroup count, the
// same merge list read against that layer's pool.
struct MergeLayers {
  MergeArgs layer[LORA_MERGE_MAX_LAYERS];
  int nblk[LORA_MERGE_MAX_LAYERS];
};

__global__ __launch_bounds__(256) void merge_layers_mfma_kernel(MergeLayers ml) {
  __shared__ uint4 raw[3072];
  __shared__ int s_pid[kMList];
  __shared__ float s_cf[kMList];
  __shared__ int s_tot[4];
  const int l = int(blockIdx.y);
  const int nb = ml.nblk[l];
  if (int(blockIdx.x) >= nb) return;
  merge_mfma_body(ml.layer[l], int(blockIdx.x), nb, raw, s_pid, s_cf, s_tot);
}

// Workgroups of the MFMA merge of one layer: at most 512 (two per CU, one
// round), a whole number per 128-column slice.
int merge_mfma_wgs(const MergeArgs &a) {
  const int gx = a.d_in / kQI, nrn = a.d_out / kSN;
  int gps = 512 / gx;
  gps = gps < 1 ? 1 : gps > nrn ? nrn : gps;
  return gx * gps;
}

bool merge_mfma_ok(const MergeArgs &a, int dtype) {
  return dtype == LORA_BF16 && a.d_in % kQI == 0 && a.d_out % kQN == 0;
}

}  // namespace

hipError_t launch_merge_layers(const MergeArgs *layers, int n, int dtype, hipStream_t s) {
  for (int l0 = 0; l0 < n; l0 += LORA_MERGE_MAX_LAYERS) {
    const int nl = n - l0 < LORA_MERGE_MAX_LAYERS ? n - l0 : LORA_MERGE_MAX_LAYERS;
    bool all_mfma = true;
    for (int l = 0; l < nl; ++l) all_mfma = all_mfma && merge_mfma_ok(layers[l0 + l], dtype);
    if (!all_mfma) {
      // other dtypes or widths: one launch per layer
      for (int l = 0; l < nl; ++l) {
        const hipError_t e = launch_merge(layers[l0 + l], dtype, s);
        if (e != hipSuccess) return e;
      }
      continue;
    }
    MergeLayers ml{};
    int gmax = 1;
    for (int l = 0; l < nl; ++l) {
      ml.layer[l] = layers[l0 + l];
      ml.nblk[l] = merge_mfma_wgs(layers[l0 + l]);
      gmax = ml.nblk[l] > gmax ? ml.nblk[l] : gmax;
    }
    hipLaunchKernelGGL(merge_layers_mfma_kernel, dim3(unsigned(gmax), unsigned(nl)), dim3(256), 0,
                       s, ml);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_merge(const MergeArgs &a, int dtype, hipStream_t s) {
  if (merge_mfma_ok(a, dtype)) {
    hipLaunchKernelGGL(merge_mfma_kernel, dim3(unsigned(merge_mfma_wgs(a))), dim3(256), 0, s, a);
    return hipGetLastError();
  }
  const int ntiles = (a.d_in / kMT) * (a.d_out / kMT);
  const dim3 grid(unsigned(ntiles < 1024 ? ntiles : 1024));
  if (dtype == LORA_BF16) hipLaunchKernelGGL(merge_kernel<uint16_t>, grid, dim3(256), 0, s, a);
  else hipLaunchKernelGGL(merge_kernel<float>, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace lora
