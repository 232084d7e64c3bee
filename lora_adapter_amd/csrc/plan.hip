// Plan kernel: the plan built by a workgroup of its own (plan_build).
#include "plan_build.h"

namespace lora {
namespace {

template <bool kLds>
__global__ __launch_bounds__(kPlanThreads) void plan_kernel(PlanArgs a) {
  extern __shared__ int dyn[];
  plan_build<kLds>(a, dyn);
}

}  // namespace

PlanLaunch plan_setup(const int32_t *ids, const float *gates, int T, int K, const PoolView &pool,
                      int32_t *plan, int nt, size_t lds_cap) {
  const int64_t TK = int64_t(T) * K;
  const int64_t N = pool.n_adapters;
  const int64_t Smax = TK < N ? TK : N;
  PlanLaunch pl{};
  pl.a = PlanArgs{ids, gates, T, K, pool.n_adapters, pool.rank, pool.page_start, pool.page_ids,
                  pool.n_pages, pool.n_page_ids, plan, 0,
                  shrink_tile_enabled(pool.dtype, TK, pool.d_in, pool.d_out) ? 1 : 0, 0, 0, 0,
                  nullptr, nullptr, 0, 0};
  int64_t cap = int64_t(lds_cap / sizeof(int));
  if (cap > kPlanLdsInts) cap = kPlanLdsInts;
  const int64_t adapter_ints = 5 * N + 5 * Smax + 3;
  const int64_t count_cols = (N + nt - 1) / nt * (nt / 64);
  pl.lds = adapter_ints <= cap && count_cols <= kLdsCountCols;
  const int64_t fixed = pl.lds ? adapter_ints : 0;
  pl.a.slot_cache = fixed + 2 * TK <= cap ? 1 : 0;
  const int64_t used = fixed + (pl.a.slot_cache ? 2 * TK : 0);
  pl.a.page_cache = pl.a.slot_cache && pool.n_page_ids > 0 && used + pool.n_page_ids <= cap ? 1 : 0;
  const int64_t used2 = used + (pl.a.page_cache ? pool.n_page_ids : 0);
  // the placement's count table, when it fits beside them: per (chunk of nt
  // slots, wave, adapter), no barrier in the placement; else per (wave,
  // adapter), three barriers a chunk against one per wave of it
  const int64_t table = int64_t(nt / 64) * N;
  const int64_t table2 = (TK + nt - 1) / nt * table;
  if (pl.lds && pl.a.slot_cache && used2 + table2 <= cap) pl.a.place_table = 2;
  else if (pl.lds && pl.a.slot_cache && nt >= 256 && used2 + table <= cap) pl.a.place_table = 1;
  const int64_t tab = pl.a.place_table == 2 ? table2 : pl.a.place_table == 1 ? table : 0;
  pl.lds_bytes = size_t(used2 + tab) * sizeof(int);
  return pl;
}

hipError_t launch_plan(const int32_t *ids, const float *gates, int T, int K, const PoolView &pool,
                       int32_t *plan, hipStream_t s) {
  const int nt = plan_threads(int64_t(T) * K, pool.n_adapters);
  const PlanLaunch pl = plan_setup(ids, gates, T, K, pool, plan, nt, size_t(kPlanLdsInts) * sizeof(int));
  if (pl.lds) hipLaunchKernelGGL(plan_kernel<true>, dim3(1), dim3(nt), pl.lds_bytes, s, pl.a);
  else hipLaunchKernelGGL(plan_kernel<false>, dim3(1), dim3(nt), pl.lds_bytes, s, pl.a);
  return hipGetLastError();
}

}  // namespace lora
