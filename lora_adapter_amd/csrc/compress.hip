// Post-hoc recompression of adapters to retained ranks, on the batched QR.
//
// The LoRAForge page ("LoRAForge：压缩与执行协同，让多LoRA服务更高效",
// sections LoRAForge的核心设计 and FlashTSQR：批量因子构造的加速器) compresses
// trained adapters after the fact: low-rank factors are recovered from the
// original matrices through QR factorisations of thousands of modules, and
// each module keeps an explicit retained rank, either a uniform fraction of
// its rank (LoRAForge-U) or by its spectral energy, the squared singular
// values (LoRAForge-S).  For one module, A (d_in x n) and B (n x d_out):
//   A = Q_A.R_A and B^T = Q_B.R_B (the batched QR, on the module's pages),
//   A.B = Q_A.(R_A.R_B^T).Q_B^T, and the n x n core R_A.R_B^T = U.S.V^T,
// so the best rank-k approximation of A.B is A' = Q_A.U_k.sqrt(S_k),
// B' = sqrt(S_k).V_k^T.Q_B^T, without ever forming A.B.
// The core's SVD is one-sided Jacobi in float64 in LDS, one workgroup per
// module: columns of the core are rotated in pairs (round-robin, n/2 disjoint
// pairs per round, fixed order) until a sweep rotates nothing or after 30
// sweeps; singular values are the column norms, sorted by a stable rank.
#include <type_traits>

#include "lora_internal.h"

namespace lora {
namespace {

constexpr int kCN = 64;   // most rank rows per module

// cols[i * n + j] = the page of module i's rank row j; bad modules (rank not
// n, page table or page ids out of range) get page 0 and bad[i] = 1.
__global__ __launch_bounds__(64) void compress_cols_kernel(const int32_t *adapters, int M, int n,
                                                           const int32_t *rank,
                                                           const int32_t *page_start,
                                                           const int32_t *page_ids, int N,
                                                           int64_t n_pages, int64_t n_page_ids,
                                                           int32_t *cols, int32_t *bad) {
  const int i = blockIdx.x, j = threadIdx.x;
  const int a = adapters[i];
  bool ok = a >= 0 && a < N;
  int64_t s0 = 0;
  if (ok) {
    s0 = page_start[a];
    ok = rank[a] == n && s0 >= 0 && int64_t(page_start[a + 1]) - s0 == n && page_start[a + 1] <= n_page_ids;
  }
  int pg = 0;
  if (ok && j < n) {
    pg = page_ids[s0 + j];
    if (pg < 0 || pg >= n_pages) pg = -1;
  }
  const bool all_ok = ok && __ballot(j < n && pg < 0) == 0;
  if (j < n) cols[int64_t(i) * n + j] = all_ok ? pg : 0;
  if (j == 0) bad[i] = all_ok ? 0 : 1;
}

struct CoreArgs {
  const float *Ra, *Rb;   // [M][n][n] row-major, upper triangular
  const int32_t *bad;     // [M]
  int M, n;
  int policy;             // 0 uniform ratio, 1 spectral energy
  float ratio, energy;
  int floor_rank;
  float *Ua, *Vb;         // [M][n][n]: U.sqrt(S) and V.sqrt(S), column j for j < k
  int32_t *out_rank;      // [M]
  float *out_sigma;       // [M][n]
};

// One DPP move of a double (its two halves; lanes without a source read 0).
template <int kCtrl, int kRowMask, int kBankMask>
__device__ __forceinline__ double dpp_d(double v) {
  const uint64_t b = __builtin_bit_cast(uint64_t, v);
  const uint32_t lo = uint32_t(__builtin_amdgcn_update_dpp(0, int(uint32_t(b)), kCtrl, kRowMask, kBankMask, false));
  const uint32_t hi = uint32_t(__builtin_amdgcn_update_dpp(0, int(uint32_t(b >> 32)), kCtrl, kRowMask, kBankMask, false));
  return __builtin_bit_cast(double, (uint64_t(hi) << 32) | lo);
}

// Sum over the 64 lanes by DPP moves (quad sums, rows of 16 by row_shr 4
// and 8, then row_bcast 15 and 31 into lane 63), read back wave-uniform: a
// fixed order without LDS round trips.
__device__ __forceinline__ double wave_sum_d(double v) {
  v += dpp_d<0xb1, 0xf, 0xf>(v);
  v += dpp_d<0x4e, 0xf, 0xf>(v);
  v += dpp_d<0x114, 0xf, 0xe>(v);
  v += dpp_d<0x118, 0xf, 0xc>(v);
  v += dpp_d<0x142, 0xa, 0xf>(v);
  v += dpp_d<0x143, 0xc, 0xf>(v);
  const uint64_t b = __builtin_bit_cast(uint64_t, v);
  const uint32_t lo = uint32_t(__builtin_amdgcn_readlane(int(uint32_t(b)), 63));
  const uint32_t hi = uint32_t(__builtin_amdgcn_readlane(int(uint32_t(b >> 32)), 63));
  return __builtin_bit_cast(double, (uint64_t(hi) << 32) | lo);
}

// CN: the smallest of 16, 32, 64 that holds n (LDS sized for it, so that
// many modules' workgroups share a CU).
template <int CN>
__global__ __launch_bounds__(256) void core_svd_kernel(CoreArgs a) {
  __shared__ double G[CN][CN];     // G[c][r]: column c of the core (rotated in place)
  __shared__ double V[CN][CN];     // V[c][r]: column c of the accumulated rotation
  __shared__ double s_sig[CN];
  __shared__ int s_rot;
  const int mat = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = a.n;
  const int np = n + (n & 1);       // even number of columns (a zero one added)
  const float *Ra = a.Ra + int64_t(mat) * n * n, *Rb = a.Rb + int64_t(mat) * n * n;
  // core C[r][c] = sum_l Ra[r][l] . Rb[c][l]  (R_A . R_B^T)
  for (int e = tid; e < np * np; e += 256) {
    const int r = e % np, c = e / np;
    double v = 0.0;
    if (r < n && c < n)
      for (int l = 0; l < n; ++l) v += double(Ra[r * n + l]) * double(Rb[c * n + l]);
    G[c][r] = v;
    V[c][r] = r == c ? 1.0 : 0.0;
  }
  __syncthreads();
  for (int sweep = 0; sweep < 30; ++sweep) {
    if (tid == 0) s_rot = 0;
    __syncthreads();
    int rotated = 0;
    for (int round = 0; round < np - 1; ++round) {
      // circle method: pair 0 = (np - 1, round), pair i = (round + i, round - i) mod (np - 1)
      for (int pi = wave; pi < np / 2; pi += 4) {
        int p, q;
        if (pi == 0) {
          p = round;
          q = np - 1;
        } else {
          p = (round + pi) % (np - 1);
          q = (round - pi + np - 1) % (np - 1);
        }
        const double gp = lane < np ? G[p][lane] : 0.0, gq = lane < np ? G[q][lane] : 0.0;
        const double alpha = wave_sum_d(gp * gp), beta = wave_sum_d(gq * gq);
        const double gamma = wave_sum_d(gp * gq);
        if (gamma != 0.0 && fabs(gamma) > 1e-15 * sqrt(alpha * beta)) {
          const double zeta = (beta - alpha) / (2.0 * gamma);
          const double t = (zeta >= 0.0 ? 1.0 : -1.0) / (fabs(zeta) + sqrt(1.0 + zeta * zeta));
          const double c = 1.0 / sqrt(1.0 + t * t), s = c * t;
          if (lane < np) {
            G[p][lane] = c * gp - s * gq;
            G[q][lane] = s * gp + c * gq;
            const double vp = V[p][lane], vq = V[q][lane];
            V[p][lane] = c * vp - s * vq;
            V[q][lane] = s * vp + c * vq;
          }
          rotated = 1;
        }
      }
      __syncthreads();
    }
    if (rotated && lane == 0) atomicOr(&s_rot, 1);
    __syncthreads();
    if (s_rot == 0) break;
    __syncthreads();
  }
  // singular values = column norms; sorted descending (ties: lower index first)
  if (wave == 0) {
    for (int c = 0; c < n; ++c) {
      const double g = lane < n ? G[c][lane] : 0.0;
      const double nrm = sqrt(wave_sum_d(g * g));
      if (lane == 0) s_sig[c] = nrm;
    }
  }
  __syncthreads();
  __shared__ int s_pos[CN];
  __shared__ int s_k;
  if (tid < n) {
    int pos = 0;
    for (int l = 0; l < n; ++l)
      pos += (s_sig[l] > s_sig[tid]) || (s_sig[l] == s_sig[tid] && l < tid);
    s_pos[tid] = pos;
  }
  __syncthreads();
  __shared__ double srt[CN];
  if (tid < n) srt[s_pos[tid]] = s_sig[tid];
  __syncthreads();
  if (tid == 0) {
    int k;
    if (a.policy == 0) {
      k = int(ceilf(a.ratio * float(n)));
    } else {
      double tot = 0.0;
      for (int j = 0; j < n; ++j) tot += srt[j] * srt[j];
      const double target = double(a.energy) * tot;
      double acc = 0.0;
      k = n;
      for (int j = 0; j < n; ++j) {
        acc += srt[j] * srt[j];
        if (acc >= target) {
          k = j + 1;
          break;
        }
      }
    }
    k = max(k, max(a.floor_rank, 1));
    k = min(k, n);
    if (a.bad[mat]) k = 0;
    s_k = k;
    a.out_rank[mat] = k;
    for (int j = 0; j < n; ++j) a.out_sigma[int64_t(mat) * n + j] = float(srt[j]);
  }
  __syncthreads();
  // U column j = G column / sigma; both factors take sqrt(sigma)
  float *Ua = a.Ua + int64_t(mat) * n * n, *Vb = a.Vb + int64_t(mat) * n * n;
  for (int e = tid; e < n * n; e += 256) {
    const int l = e % n, c = e / n;             // row l of column c (unsorted order)
    const int j = s_pos[c];
    const double sg = s_sig[c];
    const double u = sg > 0.0 ? G[c][l] / sg : 0.0;
    const double rt = sqrt(sg);
    Ua[l * n + j] = float(u * rt);
    Vb[l * n + j] = float(V[c][l] * rt);
  }
}

// out rows mat * n + j (j < k) of [M * n][m]: column j of Q.W, Q given by its
// columns Qt [M][n][m], W [M][n][n] (row l, column j).
template <typename E, int CN>
__global__ __launch_bounds__(256) void compress_rebuild_kernel(const float *Qt, const float *W,
                                                               const int32_t *rank, int n, int m,
                                                               E *out) {
  __shared__ float w[CN][CN];
  __shared__ float qs[CN][256];           // this chunk of Q's columns
  const int mat = blockIdx.y, tid = threadIdx.x, x = blockIdx.x * 256 + tid;
  const int k = rank[mat];
  for (int e = tid; e < n * n; e += 256) w[e / n][e % n] = W[int64_t(mat) * n * n + e];
  for (int l = 0; l < n; ++l) qs[l][tid] = x < m ? Qt[(int64_t(mat) * n + l) * m + x] : 0.f;
  __syncthreads();
  if (x >= m || k == 0) return;
  for (int j = 0; j < k; ++j) {
    float v = 0.f;
    for (int l = 0; l < n; ++l) v = fmaf(qs[l][tid], w[l][j], v);
    Elem<E>::store1(out + (int64_t(mat) * n + j) * m + x, v);
  }
}

}  // namespace

size_t compress_workspace_bytes(int M, int d_in, int d_out, int n) {
  const size_t tq = tsqr_workspace_bytes(M, d_in > d_out ? d_in : d_out, n);
  return 256 * 8 + size_t(M) * n * 4 * 2 + size_t(M) * n * (size_t(d_in) + d_out) * 4 +
         size_t(M) * n * n * 4 * 4 + tq;
}

hipError_t launch_compress(const PoolView &pool, const int32_t *adapters, int M, int n, int policy,
                           float ratio, float energy, int floor_rank, void *out_a, void *out_b,
                           int32_t *out_rank, float *out_sigma, void *ws, hipStream_t s) {
  auto carve = [](char *&p, size_t bytes) {
    char *r = p;
    p += (bytes + 255) & ~size_t(255);
    return r;
  };
  char *p = static_cast<char *>(ws);
  int32_t *cols = reinterpret_cast<int32_t *>(carve(p, size_t(M) * n * 4));
  int32_t *bad = reinterpret_cast<int32_t *>(carve(p, size_t(M) * 4));
  float *Qa = reinterpret_cast<float *>(carve(p, size_t(M) * n * pool.d_in * 4));
  float *Qb = reinterpret_cast<float *>(carve(p, size_t(M) * n * pool.d_out * 4));
  float *Ra = reinterpret_cast<float *>(carve(p, size_t(M) * n * n * 4));
  float *Rb = reinterpret_cast<float *>(carve(p, size_t(M) * n * n * 4));
  float *Ua = reinterpret_cast<float *>(carve(p, size_t(M) * n * n * 4));
  float *Vb = reinterpret_cast<float *>(carve(p, size_t(M) * n * n * 4));
  void *tws = p;
  hipLaunchKernelGGL(compress_cols_kernel, dim3(unsigned(M)), dim3(64), 0, s, adapters, M, n,
                     pool.rank, pool.page_start, pool.page_ids, pool.n_adapters, pool.n_pages,
                     pool.n_page_ids, cols, bad);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if ((e = launch_tsqr(pool.a_pages, pool.dtype, cols, M, pool.d_in, n, Qa, Ra, tws, s)) != hipSuccess)
    return e;
  if ((e = launch_tsqr(pool.b_pages, pool.dtype, cols, M, pool.d_out, n, Qb, Rb, tws, s)) != hipSuccess)
    return e;
  CoreArgs c{Ra, Rb, bad, M, n, policy, ratio, energy, floor_rank, Ua, Vb, out_rank, out_sigma};
  if (n <= 16) hipLaunchKernelGGL(core_svd_kernel<16>, dim3(unsigned(M)), dim3(256), 0, s, c);
  else if (n <= 32) hipLaunchKernelGGL(core_svd_kernel<32>, dim3(unsigned(M)), dim3(256), 0, s, c);
  else hipLaunchKernelGGL(core_svd_kernel<kCN>, dim3(unsigned(M)), dim3(256), 0, s, c);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const dim3 ga(unsigned((pool.d_in + 255) / 256), unsigned(M)), gb(unsigned((pool.d_out + 255) / 256), unsigned(M));
  auto rebuild = [&](auto tag, auto cn) {
    using E = decltype(tag);
    constexpr int CN = decltype(cn)::value;
    hipLaunchKernelGGL((compress_rebuild_kernel<E, CN>), ga, dim3(256), 0, s, Qa, Ua, out_rank, n,
                       pool.d_in, static_cast<E *>(out_a));
    hipLaunchKernelGGL((compress_rebuild_kernel<E, CN>), gb, dim3(256), 0, s, Qb, Vb, out_rank, n,
                       pool.d_out, static_cast<E *>(out_b));
  };
  if (pool.dtype == LORA_BF16) {
    if (n <= 16) rebuild(uint16_t{}, std::integral_constant<int, 16>{});
    else if (n <= 32) rebuild(uint16_t{}, std::integral_constant<int, 32>{});
    else rebuild(uint16_t{}, std::integral_constant<int, kCN>{});
  } else {
    if (n <= 16) rebuild(float{}, std::integral_constant<int, 16>{});
    else if (n <= 32) rebuild(float{}, std::integral_constant<int, 32>{});
    else rebuild(float{}, std::integral_constant<int, kCN>{});
  }
  return hipGetLastError();
}

}  // namespace lora
