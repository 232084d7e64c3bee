// Batched tall-skinny QR (TSQR) of many m x n matrices, n <= 64.
//
// The LoRAForge page ("LoRAForge：压缩与执行协同，让多LoRA服务更高效", section
// FlashTSQR：批量因子构造的加速器 and its glossary note on TSQR) describes the
// factor construction of post-hoc adapter compression as QR factorisations
// of thousands of tall, skinny matrices, computed by local QRs of row blocks
// whose triangular factors are then merged, with parallelism across modules
// and across row blocks.  Here:
//   * level 0: one workgroup per (matrix, 256-row tile) factors its tile by
//     Householder reflections in LDS (float32, column-major, reductions by a
//     fixed butterfly then a fixed 4-wave sum: deterministic); the tile's
//     n x n triangle becomes n rows of the level-1 matrix, the stack of all
//     tiles' triangles;
//   * the same kernel factors level 1, 2, ... until a level is one tile;
//   * Q is formed top-down: a tile's Q block is its reflectors applied, last
//     to first, to [the tile's n x n block of the level above's Q ; 0]; the
//     top level starts from the diagonal of signs that makes diag(R) >= 0.
// A matrix is given by its n columns, each a row of length m of a source
// array selected through an index table: the pages of an adapter pool (A's
// column j = one page, B^T's column j = one page) are factored where they
// are.  Rows past m in a tile are zero; a zero column (below the diagonal)
// takes no reflection.
#include "lora_internal.h"

namespace lora {
namespace {

constexpr int kTR = 256;        // rows per tile
constexpr int kTN = 64;         // most columns

struct TsqrLevel {
  // input of the level: level 0 gathers column j of matrix i from row
  // cols[i * n + j] of src ([rows][m], dtype); higher levels read
  // X [M][n][m_l] (float32, columns contiguous)
  const void *src;
  const int32_t *cols;
  const float *X;
  int m_l;              // rows of this level's matrices
  int tiles;            // ceil(m_l / kTR)
  int n, M;
  float *V;             // [M][n][m_l] reflectors (v_j = 1 implicit at the diagonal)
  float *tau;           // [M][tiles][n]
  float *Xn;            // next level's input [M][n][tiles * n], or null at the top
  float *R;             // top level: R [M][n][n] with diag >= 0
  float *sgn;           // top level: [M][n] the signs applied
};

__device__ __forceinline__ float block_sum4(float v, float *red) {
  // butterfly within the wave, then the four wave sums in order
  v = wave_sum(v);
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[wave] = v;
  __syncthreads();
  const float s = (red[0] + red[1]) + (red[2] + red[3]);
  __syncthreads();
  return s;
}

// A tile lives in dynamic LDS sized for its n columns (n x 256 floats, 16
// KiB at n = 16 instead of the 64 KiB n = 64 needs), so that many tiles'
// workgroups share a CU: each one is a chain of per-column reductions and
// barriers, and the device runs at the rate of the workgroups in flight.
template <typename E, bool kLevel0>
__global__ __launch_bounds__(256) void tsqr_factor_kernel(TsqrLevel a) {
  extern __shared__ float tsqr_dyn[];
  float (*col)[kTR] = reinterpret_cast<float (*)[kTR]>(tsqr_dyn);   // the tile, column-major
  __shared__ float s_tau[kTN];
  __shared__ float red[4];
  const int tile = blockIdx.x, mat = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = a.n;
  const int r0 = tile * kTR;
  const int rows = min(kTR, a.m_l - r0);
  // load: thread tid owns row tid of every column
  for (int c = 0; c < n; ++c) {
    float v = 0.f;
    if (tid < rows) {
      if constexpr (kLevel0) {
        const int64_t srow = a.cols[int64_t(mat) * n + c];
        v = Elem<E>::to_f(static_cast<const E *>(a.src)[srow * a.m_l + r0 + tid]);
      } else {
        v = a.X[(int64_t(mat) * n + c) * a.m_l + r0 + tid];
      }
    }
    col[c][tid] = v;
  }
  __syncthreads();
  for (int j = 0; j < n; ++j) {
    // reflector for column j, rows j.. of the tile
    const float x = tid >= j ? col[j][tid] : 0.f;
    const float xj = col[j][j];
    const float below = block_sum4(tid > j ? x * x : 0.f, red);
    float beta = xj, tau = 0.f, scl = 0.f;
    if (below > 0.f) {
      const float nrm = sqrtf(xj * xj + below);
      beta = xj >= 0.f ? -nrm : nrm;
      tau = (beta - xj) / beta;
      scl = 1.f / (xj - beta);
    }
    if (tid > j) col[j][tid] = x * scl;       // v (v_j = 1 implicit)
    if (tid == 0) {
      col[j][j] = beta;
      s_tau[j] = tau;
    }
    __syncthreads();
    // apply H_j to columns j+1 .. n-1, one wave per column
    if (tau != 0.f) {
      float v4[kTR / 64];
#pragma unroll
      for (int q = 0; q < kTR / 64; ++q) {
        const int r = lane + 64 * q;
        v4[q] = r > j ? col[j][r] : (r == j ? 1.f : 0.f);
      }
      for (int c = j + 1 + wave; c < n; c += 4) {
        float d = 0.f;
#pragma unroll
        for (int q = 0; q < kTR / 64; ++q) d = fmaf(v4[q], col[c][lane + 64 * q], d);
        const float w = tau * wave_sum(d);
#pragma unroll
        for (int q = 0; q < kTR / 64; ++q) {
          const int r = lane + 64 * q;
          if (r >= j) col[c][r] = fmaf(-w, v4[q], col[c][r]);
        }
      }
    }
    __syncthreads();
  }
  // reflectors and taus out
  float *V = a.V + int64_t(mat) * n * a.m_l;
  for (int c = 0; c < n; ++c)
    if (tid < rows) V[int64_t(c) * a.m_l + r0 + tid] = tid > c ? col[c][tid] : 0.f;
  if (tid < n) a.tau[(int64_t(mat) * a.tiles + tile) * n + tid] = s_tau[tid];
  // the tile's triangle: rows i <= c of column c (zero rows where the tile
  // had fewer rows than columns)
  if (a.Xn) {
    const int mn = a.tiles * n;
    for (int c = 0; c < n; ++c)
      if (tid < n) a.Xn[(int64_t(mat) * n + c) * mn + tile * n + tid] = tid <= c ? col[c][tid] : 0.f;
  } else {
    // top: R with the signs that make its diagonal non-negative
    __shared__ float s_sg[kTN];
    if (tid < n) s_sg[tid] = col[tid][tid] < 0.f ? -1.f : 1.f;
    __syncthreads();
    for (int c = 0; c < n; ++c)
      if (tid < n) a.R[(int64_t(mat) * n + tid) * n + c] = tid <= c ? s_sg[tid] * col[c][tid] : 0.f;
    if (tid < n) a.sgn[int64_t(mat) * n + tid] = s_sg[tid];
  }
}

struct TsqrForm {
  const float *V, *tau;    // this level's reflectors
  int m_l, tiles, n, M;
  const float *Qup;        // [M][n][tiles * n] the level above's Q, or null at the top
  const float *sgn;        // top: [M][n]
  float *Q;                // this level's Q [M][n][m_l] (level 0: the output Qt)
};

__global__ __launch_bounds__(256) void tsqr_form_kernel(TsqrForm a) {
  extern __shared__ float tsqr_dyn[];
  float (*C)[kTR] = reinterpret_cast<float (*)[kTR]>(tsqr_dyn);               // n x 256
  float (*Vs)[kTR] = reinterpret_cast<float (*)[kTR]>(tsqr_dyn + a.n * kTR);  // n x 256
  const int tile = blockIdx.x, mat = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = a.n;
  const int r0 = tile * kTR;
  const int rows = min(kTR, a.m_l - r0);
  const float *V = a.V + int64_t(mat) * n * a.m_l;
  for (int c = 0; c < n; ++c) {
    Vs[c][tid] = tid < rows ? V[int64_t(c) * a.m_l + r0 + tid] : 0.f;
    float b = 0.f;
    if (tid < n) {
      if (a.Qup) b = a.Qup[(int64_t(mat) * n + c) * (int64_t(a.tiles) * n) + tile * n + tid];
      else b = tid == c ? a.sgn[int64_t(mat) * n + c] : 0.f;
    }
    C[c][tid] = b;
  }
  __syncthreads();
  const float *tau = a.tau + (int64_t(mat) * a.tiles + tile) * n;
  for (int j = n - 1; j >= 0; --j) {
    const float t = tau[j];
    if (t != 0.f) {
      float v4[kTR / 64];
#pragma unroll
      for (int q = 0; q < kTR / 64; ++q) {
        const int r = lane + 64 * q;
        v4[q] = r > j ? Vs[j][r] : (r == j ? 1.f : 0.f);
      }
      for (int c = wave; c < n; c += 4) {
        float d = 0.f;
#pragma unroll
        for (int q = 0; q < kTR / 64; ++q) d = fmaf(v4[q], C[c][lane + 64 * q], d);
        const float w = t * wave_sum(d);
#pragma unroll
        for (int q = 0; q < kTR / 64; ++q) {
          const int r = lane + 64 * q;
          if (r >= j) C[c][r] = fmaf(-w, v4[q], C[c][r]);
        }
      }
    }
    __syncthreads();
  }
  float *Q = a.Q + int64_t(mat) * n * a.m_l;
  for (int c = 0; c < n; ++c)
    if (tid < rows) Q[int64_t(c) * a.m_l + r0 + tid] = C[c][tid];
}

// The same factorisation and Q formation with one wave per tile, for n <= 16
// (the ranks of compressed adapters): the tile lives in registers, lane l
// holding rows 4l .. 4l + 3 of every column (one vector load or store per
// column), and every reduction is a DPP sum over the wave (no barrier, no
// LDS).  Four tiles per workgroup.  Same reflectors, taus, triangles and signs as the workgroup
// kernels above, summed in another (fixed) order.
constexpr int kWN = 16;         // most columns of the wave kernels
constexpr int kWQ = kTR / 64;   // rows per lane

// Sum over the 64 lanes with DPP moves (vector ALU, no LDS round trip):
// quad sums, then rows of 16 (row_shr 4, 8), then the row sums carried by
// row_bcast 15 and 31 into lane 63, read back as a wave-uniform value.  A
// fixed order, so deterministic.
__device__ __forceinline__ float wave_total(float v) {
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0xb1, 0xf, 0xf, false));
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x4e, 0xf, 0xf, false));
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x114, 0xf, 0xe, false));
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x118, 0xf, 0xc, false));
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x142, 0xa, 0xf, false));
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x143, 0xc, 0xf, false));
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}

// Four consecutive rows of a column, as floats: one vector load when the
// four are in the tile and aligned (m_l % 4 == 0, 16-byte aligned bases).
template <typename E>
__device__ __forceinline__ void load4(const E *p, int avail, bool vec, float (&v)[4]) {
  if (vec && avail >= 4) {
    if constexpr (sizeof(E) == 2) {
      const uint2 w = *reinterpret_cast<const uint2 *>(p);
      v[0] = bf_lo(w.x); v[1] = bf_hi(w.x); v[2] = bf_lo(w.y); v[3] = bf_hi(w.y);
    } else {
      const float4 w = *reinterpret_cast<const float4 *>(p);
      v[0] = w.x; v[1] = w.y; v[2] = w.z; v[3] = w.w;
    }
  } else {
#pragma unroll
    for (int q = 0; q < 4; ++q) v[q] = q < avail ? Elem<E>::to_f(p[q]) : 0.f;
  }
}

__device__ __forceinline__ void store4(float *p, int avail, bool vec, const float (&v)[4]) {
  if (vec && avail >= 4) {
    *reinterpret_cast<float4 *>(p) = make_float4(v[0], v[1], v[2], v[3]);
  } else {
#pragma unroll
    for (int q = 0; q < 4; ++q)
      if (q < avail) p[q] = v[q];
  }
}

template <typename E, bool kLevel0>
__global__ __launch_bounds__(256) void tsqr_factor_wave_kernel(TsqrLevel a) {
  const int lane = threadIdx.x & 63;
  const int t = int(blockIdx.x) * 4 + int(threadIdx.x >> 6);
  if (t >= a.tiles * a.M) return;
  const int mat = t / a.tiles, tile = t % a.tiles;
  const int n = a.n;
  const int r0 = tile * kTR;
  const int rows = min(kTR, a.m_l - r0);
  const int rl = 4 * lane;                       // the lane's rows: rl .. rl + 3
  const int avail = min(4, max(0, rows - rl));
  const uintptr_t in = kLevel0 ? reinterpret_cast<uintptr_t>(a.src) : reinterpret_cast<uintptr_t>(a.X);
  const bool vec = a.m_l % 4 == 0 && (in | reinterpret_cast<uintptr_t>(a.V)) % 16 == 0;
  float x[kWN][kWQ];
#pragma unroll
  for (int c = 0; c < kWN; ++c) {
    float v[4] = {0.f, 0.f, 0.f, 0.f};
    if (c < n) {
      if constexpr (kLevel0) {
        const int64_t srow = a.cols[int64_t(mat) * n + c];
        load4<E>(static_cast<const E *>(a.src) + srow * a.m_l + r0 + rl, avail, vec, v);
      } else {
        load4<float>(a.X + (int64_t(mat) * n + c) * a.m_l + r0 + rl, avail, vec, v);
      }
    }
#pragma unroll
    for (int q = 0; q < kWQ; ++q) x[c][q] = v[q];
  }
  float taus[kWN];
#pragma unroll
  for (int j = 0; j < kWN; ++j) {
    taus[j] = 0.f;
    if (j >= n) continue;
    // reflector for column j (row j is lane j / 4's row j % 4)
    const float xj = __shfl(x[j][j & 3], j >> 2, 64);
    float part = 0.f;
#pragma unroll
    for (int q = 0; q < kWQ; ++q)
      if (rl + q > j) part = fmaf(x[j][q], x[j][q], part);
    const float below = wave_total(part);
    float beta = xj, tau = 0.f, scl = 0.f;
    if (below > 0.f) {
      const float nrm = sqrtf(xj * xj + below);
      beta = xj >= 0.f ? -nrm : nrm;
      tau = (beta - xj) / beta;
      scl = 1.f / (xj - beta);
    }
    taus[j] = tau;
    // v (v_j = 1 implicit) into column j below the diagonal, beta on it
    float v[kWQ];
#pragma unroll
    for (int q = 0; q < kWQ; ++q) {
      const int r = rl + q;
      if (r > j) x[j][q] *= scl;
      v[q] = r > j ? x[j][q] : (r == j ? 1.f : 0.f);
      if (r == j) x[j][q] = beta;
    }
    if (tau != 0.f) {
      // apply H_j to the later columns: all their dot products first
      float d[kWN];
#pragma unroll
      for (int c = j + 1; c < kWN; ++c) {
        float pc = 0.f;
#pragma unroll
        for (int q = 0; q < kWQ; ++q) pc = fmaf(v[q], x[c][q], pc);
        d[c] = c < n ? wave_total(pc) : 0.f;
      }
#pragma unroll
      for (int c = j + 1; c < kWN; ++c) {
        const float w = tau * d[c];
#pragma unroll
        for (int q = 0; q < kWQ; ++q) x[c][q] = fmaf(-w, v[q], x[c][q]);
      }
    }
  }
  // reflectors and taus out
  float *V = a.V + int64_t(mat) * n * a.m_l;
#pragma unroll
  for (int c = 0; c < kWN; ++c) {
    if (c >= n) continue;
    float v[4];
#pragma unroll
    for (int q = 0; q < kWQ; ++q) v[q] = rl + q > c ? x[c][q] : 0.f;
    store4(V + int64_t(c) * a.m_l + r0 + rl, avail, vec, v);
  }
#pragma unroll
  for (int j = 0; j < kWN; ++j)
    if (j < n && lane == j) a.tau[(int64_t(mat) * a.tiles + tile) * n + j] = taus[j];
  // the triangle: rows t < n (lanes 0 .. 3)
  if (a.Xn) {
    const int mn = a.tiles * n;
#pragma unroll
    for (int c = 0; c < kWN; ++c)
#pragma unroll
      for (int q = 0; q < kWQ; ++q) {
        const int tr = rl + q;
        if (c < n && tr < n) a.Xn[(int64_t(mat) * n + c) * mn + tile * n + tr] = tr <= c ? x[c][q] : 0.f;
      }
  } else {
    float sg[kWQ];
#pragma unroll
    for (int q = 0; q < kWQ; ++q) {
      float diag = 0.f;
#pragma unroll
      for (int c = 0; c < kWN; ++c)
        if (rl + q == c) diag = x[c][q];
      sg[q] = diag < 0.f ? -1.f : 1.f;
    }
#pragma unroll
    for (int c = 0; c < kWN; ++c)
#pragma unroll
      for (int q = 0; q < kWQ; ++q) {
        const int tr = rl + q;
        if (c < n && tr < n) a.R[(int64_t(mat) * n + tr) * n + c] = tr <= c ? sg[q] * x[c][q] : 0.f;
      }
#pragma unroll
    for (int q = 0; q < kWQ; ++q)
      if (rl + q < n) a.sgn[int64_t(mat) * n + rl + q] = sg[q];
  }
}

__global__ __launch_bounds__(256) void tsqr_form_wave_kernel(TsqrForm a) {
  const int lane = threadIdx.x & 63;
  const int t = int(blockIdx.x) * 4 + int(threadIdx.x >> 6);
  if (t >= a.tiles * a.M) return;
  const int mat = t / a.tiles, tile = t % a.tiles;
  const int n = a.n;
  const int r0 = tile * kTR;
  const int rows = min(kTR, a.m_l - r0);
  const int rl = 4 * lane;
  const int avail = min(4, max(0, rows - rl));
  const bool vec = a.m_l % 4 == 0 &&
                   (reinterpret_cast<uintptr_t>(a.V) | reinterpret_cast<uintptr_t>(a.Q)) % 16 == 0;
  const float *V = a.V + int64_t(mat) * n * a.m_l;
  float C[kWN][kWQ];
#pragma unroll
  for (int c = 0; c < kWN; ++c)
#pragma unroll
    for (int q = 0; q < kWQ; ++q) {
      const int r = rl + q;
      float b = 0.f;
      if (c < n && r < n) {
        if (a.Qup) b = a.Qup[(int64_t(mat) * n + c) * (int64_t(a.tiles) * n) + tile * n + r];
        else b = r == c ? a.sgn[int64_t(mat) * n + c] : 0.f;
      }
      C[c][q] = b;
    }
  const float *tau = a.tau + (int64_t(mat) * a.tiles + tile) * n;
#pragma unroll
  for (int jj = 0; jj < kWN; ++jj) {
    const int j = kWN - 1 - jj;            // reflectors last to first
    const float tj = j < n ? tau[j] : 0.f;
    if (tj == 0.f) continue;
    // reflector j (read from the level's V; other waves cover the latency)
    float vr[4];
    load4<float>(V + int64_t(j) * a.m_l + r0 + rl, avail, vec, vr);
    float v[kWQ];
#pragma unroll
    for (int q = 0; q < kWQ; ++q) {
      const int r = rl + q;
      v[q] = r > j ? vr[q] : (r == j ? 1.f : 0.f);
    }
    float d[kWN];
#pragma unroll
    for (int c = 0; c < kWN; ++c) {
      float pc = 0.f;
#pragma unroll
      for (int q = 0; q < kWQ; ++q) pc = fmaf(v[q], C[c][q], pc);
      d[c] = c < n ? wave_total(pc) : 0.f;
    }
#pragma unroll
    for (int c = 0; c < kWN; ++c) {
      const float w = tj * d[c];
#pragma unroll
      for (int q = 0; q < kWQ; ++q) C[c][q] = fmaf(-w, v[q], C[c][q]);
    }
  }
  float *Q = a.Q + int64_t(mat) * n * a.m_l;
#pragma unroll
  for (int c = 0; c < kWN; ++c)
    if (c < n) store4(Q + int64_t(c) * a.m_l + r0 + rl, avail, vec, C[c]);
}

// Rows of each level: m, then tiles * n while more than one tile.
int tsqr_levels(int m, int n, int out_m[16]) {
  int L = 0, ml = m;
  while (true) {
    out_m[L++] = ml;
    const int t = (ml + kTR - 1) / kTR;
    if (t == 1 || L == 16) break;
    ml = t * n;
  }
  return L;
}

}  // namespace

bool tsqr_shape_ok(int M, int m, int n) { return M >= 1 && n >= 1 && n <= kTN && m >= n; }

size_t tsqr_workspace_bytes(int M, int m, int n) {
  int ml[16];
  const int L = tsqr_levels(m, n, ml);
  size_t f = 0;
  for (int l = 0; l < L; ++l) {
    const size_t tiles = size_t((ml[l] + kTR - 1) / kTR);
    f += 2 * size_t(M) * n * ml[l];         // V, and X (level > 0) / Q (level > 0)
    f += size_t(M) * tiles * n;             // tau
  }
  f += size_t(M) * n;                       // signs
  return f * sizeof(float);
}

hipError_t launch_tsqr(const void *src, int dtype, const int32_t *cols, int M, int m, int n,
                       float *Qt, float *R, void *ws, hipStream_t s) {
  int ml[16];
  const int L = tsqr_levels(m, n, ml);
  float *p = static_cast<float *>(ws);
  float *V[16], *X[16], *tau[16];
  for (int l = 0; l < L; ++l) {
    const int tiles = (ml[l] + kTR - 1) / kTR;
    V[l] = p; p += size_t(M) * n * ml[l];
    X[l] = p; p += size_t(M) * n * ml[l];    // level l's input (level 0: unused) and Q (l > 0)
    tau[l] = p; p += size_t(M) * tiles * n;
  }
  float *sgn = p;
  for (int l = 0; l < L; ++l) {
    TsqrLevel a{};
    a.src = src; a.cols = cols; a.X = X[l];
    a.m_l = ml[l]; a.tiles = (ml[l] + kTR - 1) / kTR; a.n = n; a.M = M;
    a.V = V[l]; a.tau = tau[l];
    a.Xn = l + 1 < L ? X[l + 1] : nullptr;
    a.R = R; a.sgn = sgn;
    const dim3 grid(unsigned(a.tiles), unsigned(M)), block(256);
    const size_t lds = size_t(n) * kTR * sizeof(float);
    if (n <= kWN) {
      const dim3 gw(unsigned((int64_t(a.tiles) * M + 3) / 4));
      if (l > 0) hipLaunchKernelGGL((tsqr_factor_wave_kernel<float, false>), gw, block, 0, s, a);
      else if (dtype == LORA_BF16) hipLaunchKernelGGL((tsqr_factor_wave_kernel<uint16_t, true>), gw, block, 0, s, a);
      else hipLaunchKernelGGL((tsqr_factor_wave_kernel<float, true>), gw, block, 0, s, a);
    } else if (l == 0) {
      if (dtype == LORA_BF16) hipLaunchKernelGGL((tsqr_factor_kernel<uint16_t, true>), grid, block, lds, s, a);
      else hipLaunchKernelGGL((tsqr_factor_kernel<float, true>), grid, block, lds, s, a);
    } else {
      hipLaunchKernelGGL((tsqr_factor_kernel<float, false>), grid, block, lds, s, a);
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (!Qt) return hipSuccess;
  // Q top-down; level l > 0 writes its Q over its input X[l] (no longer read)
  for (int l = L - 1; l >= 0; --l) {
    TsqrForm f{};
    f.V = V[l]; f.tau = tau[l]; f.m_l = ml[l]; f.tiles = (ml[l] + kTR - 1) / kTR; f.n = n; f.M = M;
    f.Qup = l + 1 < L ? X[l + 1] : nullptr;
    f.sgn = sgn;
    f.Q = l == 0 ? Qt : X[l];
    if (n <= kWN)
      hipLaunchKernelGGL(tsqr_form_wave_kernel, dim3(unsigned((int64_t(f.tiles) * M + 3) / 4)), dim3(256), 0,
                         s, f);
    else
      hipLaunchKernelGGL(tsqr_form_kernel, dim3(unsigned(f.tiles), unsigned(M)), dim3(256),
                         2 * size_t(n) * kTR * sizeof(float), s, f);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace lora
