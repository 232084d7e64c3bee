// extern "C" entry points of liblora: argument checks on the host (before any
// HIP call), workspace layout, and kernel dispatch on the caller's stream.
#include <string.h>

#include "lora_internal.h"

using namespace lora;

namespace {

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) & ~(kAlign - 1); }

bool dims_ok(int32_t d) { return d > 0 && d % 64 == 0; }

// Checks the descriptor fields every call needs; `need_pages` also asks for
// the factor pages and scales.
int32_t check_pool(const lora_pool_desc *p, bool need_pages) {
  if (!p) return LORA_ERR_INVALID_ARG;
  if (p->dtype != LORA_F32 && p->dtype != LORA_BF16) return LORA_ERR_INVALID_ARG;
  if (p->n_adapters < 1 || p->n_pages < 0 || p->n_page_ids < 0) return LORA_ERR_INVALID_ARG;
  if (!p->rank || !p->page_start || (p->n_page_ids > 0 && !p->page_ids)) return LORA_ERR_INVALID_ARG;
  if (need_pages) {
    if (!p->scale) return LORA_ERR_INVALID_ARG;
    if (p->n_pages > 0 && (!p->a_pages || !p->b_pages)) return LORA_ERR_INVALID_ARG;
    if (!dims_ok(p->d_in) || !dims_ok(p->d_out)) return LORA_ERR_UNSUPPORTED;
  }
  return LORA_OK;
}

int32_t check_batch(int32_t T, int32_t K) {
  if (T < 0 || K < 1 || K > LORA_MAX_K) return LORA_ERR_INVALID_ARG;
  if (int64_t(T) * K > kMaxPairs) return LORA_ERR_UNSUPPORTED;
  return LORA_OK;
}

int32_t dev(hipError_t e) { return e == hipSuccess ? LORA_OK : LORA_ERR_DEVICE; }

// Apply workspace: [split partials][U per slot, slot descriptors (decode
// shapes)][U].  The per-slot U (LORA_MAX_RANK floats per slot) and the slot
// descriptors are written by the per-slot shrink of lora_forward's decode
// launch.
struct ApplyWs {
  GemmConfig cfg;
  size_t partial_bytes;   // aligned
  float *partial;
  float *slot_u;          // decode shapes: [T*K][LORA_MAX_RANK]
  int4 *sdesc;            // decode shapes: [T*K]
  float *U;
  int64_t u_cap;
};

size_t slot_u_only_bytes(int32_t T, int32_t K) {
  return align_up(size_t(T) * size_t(K) * LORA_MAX_RANK * sizeof(float));
}

size_t slot_u_bytes(const GemmConfig &c, int32_t T, int32_t K) {
  return c.kind == 4 ? slot_u_only_bytes(T, K) + align_up(size_t(T) * size_t(K) * sizeof(int4)) : 0;
}

ApplyWs apply_layout(void *ws, size_t ws_bytes, int32_t T, int32_t K, int32_t d_in, int32_t d_out,
                     int32_t dtype) {
  ApplyWs w{};
  w.cfg = choose_gemm(T > 0 ? T : 1, d_in, d_out, dtype);
  w.partial_bytes = align_up(gemm_partial_bytes(w.cfg, T, d_out));
  const size_t head = w.partial_bytes + slot_u_bytes(w.cfg, T, K);
  w.partial = static_cast<float *>(ws);
  if (ws && ws_bytes >= head) {
    w.slot_u = w.cfg.kind == 4
                   ? reinterpret_cast<float *>(static_cast<char *>(ws) + w.partial_bytes) : nullptr;
    w.sdesc = w.cfg.kind == 4
                  ? reinterpret_cast<int4 *>(static_cast<char *>(ws) + w.partial_bytes +
                                             slot_u_only_bytes(T, K)) : nullptr;
    w.U = reinterpret_cast<float *>(static_cast<char *>(ws) + head);
    w.u_cap = int64_t((ws_bytes - head) / sizeof(float));
  } else {
    w.U = nullptr;
    w.u_cap = -1;
  }
  return w;
}

}  // namespace

extern "C" {

int32_t lora_abi_version(void) { return LORA_ABI_VERSION; }

const char *lora_status_string(int32_t status) {
  switch (status) {
    case LORA_OK: return "ok";
    case LORA_ERR_INVALID_ARG: return "invalid argument";
    case LORA_ERR_UNSUPPORTED: return "unsupported shape or dtype";
    case LORA_ERR_CAPACITY: return "buffer too small";
    case LORA_ERR_DEVICE: return "HIP call failed";
    default: return "unknown status";
  }
}

size_t lora_plan_bytes(int32_t T, int32_t K, int32_t n_adapters) {
  if (check_batch(T, K) != LORA_OK || n_adapters < 1) return 0;
  return size_t(plan_layout(int64_t(T) * K, n_adapters).total) * sizeof(int32_t);
}

int32_t lora_plan_layout(int32_t T, int32_t K, int32_t n_adapters, int64_t offsets_out[9]) {
  if (!offsets_out || n_adapters < 1) return LORA_ERR_INVALID_ARG;
  const int32_t st = check_batch(T, K);
  if (st != LORA_OK) return st;
  const PlanLayout L = plan_layout(int64_t(T) * K, n_adapters);
  const int64_t o[9] = {L.hdr, L.pair_tk, L.seg_adapter, L.seg_off, L.seg_row_off,
                        L.bucket_seg_off, L.u_off, L.slot_pos, L.pair_adapter};
  for (int i = 0; i < 9; ++i) offsets_out[i] = o[i] * int64_t(sizeof(int32_t));
  return LORA_OK;
}

int32_t lora_plan(const int32_t *ids, const float *gates, int32_t T, int32_t K,
                  const lora_pool_desc *pool, void *plan, size_t plan_bytes, void *stream) {
  int32_t st = check_batch(T, K);
  if (st != LORA_OK) return st;
  if ((st = check_pool(pool, false)) != LORA_OK) return st;
  if (!plan) return LORA_ERR_INVALID_ARG;
  if (int64_t(T) * K > 0 && (!ids || !gates)) return LORA_ERR_INVALID_ARG;
  if (plan_bytes < lora_plan_bytes(T, K, pool->n_adapters)) return LORA_ERR_CAPACITY;
  return dev(launch_plan(ids, gates, T, K, pool_view(pool), static_cast<int32_t *>(plan),
                         static_cast<hipStream_t>(stream)));
}

int32_t lora_plan_header(const void *plan, int32_t *out, void *stream) {
  if (!plan || !out) return LORA_ERR_INVALID_ARG;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  // the header is the plan buffer's first LORA_PLAN_HEADER_INTS words
  if (hipMemcpyAsync(out, plan, LORA_PLAN_HEADER_INTS * sizeof(int32_t), hipMemcpyDeviceToHost,
                     s) != hipSuccess)
    return LORA_ERR_DEVICE;
  return dev(hipStreamSynchronize(s));
}

size_t lora_apply_workspace_bytes(int32_t T, int32_t K, int32_t d_in, int32_t d_out,
                                  int32_t max_rank, int32_t dtype) {
  if (check_batch(T, K) != LORA_OK || !dims_ok(d_in) || !dims_ok(d_out)) return 0;
  if (max_rank < 0 || max_rank > LORA_MAX_RANK) return 0;
  if (dtype != LORA_F32 && dtype != LORA_BF16) return 0;
  const GemmConfig c = choose_gemm(T > 0 ? T : 1, d_in, d_out, dtype);
  const size_t u = size_t(T) * size_t(K) * size_t(max_rank) * sizeof(float);
  return align_up(gemm_partial_bytes(c, T, d_out)) + slot_u_bytes(c, T, K) + align_up(u > 0 ? u : 1);
}

size_t lora_apply_u_offset(int32_t T, int32_t K, int32_t d_in, int32_t d_out, int32_t dtype) {
  if (check_batch(T, K) != LORA_OK || !dims_ok(d_in) || !dims_ok(d_out)) return 0;
  if (dtype != LORA_F32 && dtype != LORA_BF16) return 0;
  const GemmConfig c = choose_gemm(T > 0 ? T : 1, d_in, d_out, dtype);
  return align_up(gemm_partial_bytes(c, T, d_out)) + slot_u_bytes(c, T, K);
}

namespace {

ShrinkArgs apply_shrink_args(const void *X, const uint8_t *keep_mask, float keep_scale,
                             int32_t T, int32_t K, const float *gates,
                             const lora_pool_desc *pool, const PlanView &pv, const ApplyWs &w) {
  ShrinkArgs a{};
  a.Z = X;
  a.mask = keep_mask;
  a.extra_scale = keep_mask ? keep_scale : 1.0f;
  a.T = T; a.K = K; a.d = pool->d_in;
  a.pages = pool->a_pages;
  a.rank = pool->rank; a.page_start = pool->page_start; a.page_ids = pool->page_ids;
  a.scale = pool->scale;
  a.gates = gates;
  a.plan = pv;
  a.err_word = const_cast<int32_t *>(pv.hdr) + LORA_PH_ERR;
  a.out = w.U;
  a.out_cap = w.u_cap;
  a.big_segments = shrink_tile_enabled(pool->dtype, int64_t(T) * K, pool->d_in, pool->d_out) ? 1 : 0;
  return a;
}

}  // namespace

int32_t lora_shrink(const void *X, const uint8_t *keep_mask, float keep_scale, int32_t T,
                    int32_t K, const float *gates, const lora_pool_desc *pool, const void *plan,
                    void *ws, size_t ws_bytes, void *stream) {
  int32_t st = check_batch(T, K);
  if (st != LORA_OK) return st;
  if ((st = check_pool(pool, true)) != LORA_OK) return st;
  if (!plan) return LORA_ERR_INVALID_ARG;
  if (T == 0) return LORA_OK;
  if (!X || !gates || !ws) return LORA_ERR_INVALID_ARG;
  const ApplyWs w = apply_layout(ws, ws_bytes, T, K, pool->d_in, pool->d_out, pool->dtype);
  if (w.u_cap < 0) return LORA_ERR_CAPACITY;
  const int64_t TK = int64_t(T) * K;
  const PlanView pv = plan_view(plan, TK, pool->n_adapters);
  const ShrinkArgs a = apply_shrink_args(X, keep_mask, keep_scale, T, K, gates, pool, pv, w);
  return dev(launch_shrink(a, pool->dtype, TK, pool->n_adapters, pool->d_in, pool->d_out,
                           static_cast<hipStream_t>(stream)));
}

namespace {

// Shared argument checks and GemmArgs for the two halves of the base stage.
int32_t base_args(const void *X, const void *W_t, void *Y, int32_t T, int32_t K,
                  const lora_pool_desc *pool, const void *plan, void *ws,
                  size_t ws_bytes, GemmConfig &cfg, GemmArgs &g) {
  int32_t st = check_batch(T, K);
  if (st != LORA_OK) return st;
  if ((st = check_pool(pool, true)) != LORA_OK) return st;
  if (!plan) return LORA_ERR_INVALID_ARG;
  if (T == 0) return LORA_OK;
  if (!X || !W_t || !Y || !ws) return LORA_ERR_INVALID_ARG;
  if (Y == X || Y == W_t) return LORA_ERR_INVALID_ARG;
  const ApplyWs w = apply_layout(ws, ws_bytes, T, K, pool->d_in, pool->d_out, pool->dtype);
  if (w.u_cap < 0) return LORA_ERR_CAPACITY;
  const int64_t TK = int64_t(T) * K;
  const PlanView pv = plan_view(plan, TK, pool->n_adapters);
  cfg = w.cfg;
  g = GemmArgs{};
  g.X = X; g.W = W_t; g.M = T; g.N = pool->d_out; g.Kd = pool->d_in;
  g.k_split = w.cfg.k_split;
  g.sk_g = w.cfg.sk;
  g.partial = w.partial;
  g.Y = Y;
  g.ex.K = K;
  g.ex.slot_desc = pv.slot_desc; g.ex.pair_tk = pv.pair_tk; g.ex.page_ids = pool->page_ids;
  g.ex.b_pages = pool->b_pages; g.ex.d_out = pool->d_out;
  g.ex.U = w.U; g.ex.hdr = pv.hdr; g.ex.u_cap = w.u_cap;
  return LORA_OK;
}

}  // namespace

int32_t lora_base_gemm(const void *X, const void *W_t, void *Y, int32_t T, int32_t K,
                       const lora_pool_desc *pool, const void *plan, void *ws,
                       size_t ws_bytes, void *stream) {
  GemmConfig cfg;
  GemmArgs g;
  const int32_t st = base_args(X, W_t, Y, T, K, pool, plan, ws, ws_bytes, cfg, g);
  if (st != LORA_OK || T == 0) return st;
  return dev(launch_base_gemm(cfg, g, static_cast<hipStream_t>(stream)));
}

int32_t lora_expand_epilogue(const void *X, const void *W_t, void *Y, int32_t T, int32_t K,
                             const lora_pool_desc *pool, const void *plan,
                             void *ws, size_t ws_bytes, void *stream) {
  GemmConfig cfg;
  GemmArgs g;
  const int32_t st = base_args(X, W_t, Y, T, K, pool, plan, ws, ws_bytes, cfg, g);
  if (st != LORA_OK || T == 0) return st;
  return dev(launch_epilogue(cfg, g, pool->dtype, static_cast<hipStream_t>(stream)));
}

int32_t lora_base_expand(const void *X, const void *W_t, void *Y, int32_t T, int32_t K,
                         const lora_pool_desc *pool, const void *plan,
                         void *ws, size_t ws_bytes, void *stream) {
  const int32_t st = lora_base_gemm(X, W_t, Y, T, K, pool, plan, ws, ws_bytes, stream);
  if (st != LORA_OK) return st;
  return lora_expand_epilogue(X, W_t, Y, T, K, pool, plan, ws, ws_bytes, stream);
}

int32_t lora_shrink_gemm(const void *X, const void *W_t, void *Y, int32_t T, int32_t K,
                         const float *gates, const uint8_t *keep_mask, float keep_scale,
                         const lora_pool_desc *pool, const void *plan, void *ws,
                         size_t ws_bytes, void *stream) {
  GemmConfig cfg;
  GemmArgs g;
  int32_t st = base_args(X, W_t, Y, T, K, pool, plan, ws, ws_bytes, cfg, g);
  if (st != LORA_OK || T == 0) return st;
  if (!gates) return LORA_ERR_INVALID_ARG;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const ApplyWs w = apply_layout(ws, ws_bytes, T, K, pool->d_in, pool->d_out, pool->dtype);
  const int64_t TK = int64_t(T) * K;
  const PlanView pv = plan_view(plan, TK, pool->n_adapters);
  const ShrinkArgs a = apply_shrink_args(X, keep_mask, keep_scale, T, K, gates, pool, pv, w);
  if (decode_shrink_fusable(cfg, pool->d_in)) {
    hipError_t e = launch_shrink_big(a, pool->dtype, TK, pool->n_adapters, pool->d_in,
                                     pool->d_out, s);
    if (e == hipSuccess) e = launch_decode_gemm_shrink(cfg, g, a, s);
    return dev(e);
  }
  hipError_t e = launch_shrink(a, pool->dtype, TK, pool->n_adapters, pool->d_in, pool->d_out, s);
  if (e == hipSuccess) e = launch_base_gemm(cfg, g, s);
  return dev(e);
}

int32_t lora_apply(const void *X, const void *W_t, void *Y, int32_t T, int32_t K,
                   const float *gates, const uint8_t *keep_mask,
                   float keep_scale, const lora_pool_desc *pool, const void *plan, void *ws,
                   size_t ws_bytes, void *stream) {
  int32_t st = check_batch(T, K);
  if (st != LORA_OK) return st;
  if ((st = check_pool(pool, true)) != LORA_OK) return st;
  if (T > 0 && (!X || !W_t || !Y || !gates || !ws || !plan)) return LORA_ERR_INVALID_ARG;
  st = lora_shrink_gemm(X, W_t, Y, T, K, gates, keep_mask, keep_scale, pool, plan, ws, ws_bytes,
                        stream);
  if (st != LORA_OK) return st;
  return lora_expand_epilogue(X, W_t, Y, T, K, pool, plan, ws, ws_bytes, stream);
}

}  // extern "C"

namespace {

// lora_forward's two halves.  Split GEMM shapes only (gemm_plan_fusable):
//   decode:   first = the plan (built by workgroup 0), GEMM partials and the
//             per-slot shrink (U per slot and slot descriptors), one launch;
//             finish = epilogue from the partials, per-slot U and
//             descriptors, which also stores U in the plan's u_off layout.
//   stream-K: first = GEMM partials with the plan built in the same launch;
//             finish = shrink, then epilogue.
// Other shapes: first = lora_plan, finish = lora_apply.
struct Fwd {
  GemmConfig cfg;
  GemmArgs g;
  bool split;
};

int32_t forward_args(const int32_t *ids, const float *gates, int32_t T, int32_t K, const void *X,
                     const void *W_t, void *Y, const lora_pool_desc *pool, void *plan,
                     size_t plan_bytes, void *ws, size_t ws_bytes, Fwd &f) {
  int32_t st = check_batch(T, K);
  if (st != LORA_OK) return st;
  if ((st = check_pool(pool, true)) != LORA_OK) return st;
  if (!plan) return LORA_ERR_INVALID_ARG;
  if (plan_bytes < lora_plan_bytes(T, K, pool->n_adapters)) return LORA_ERR_CAPACITY;
  f.split = false;
  if (T == 0) return LORA_OK;
  if (!ids || !gates || !X || !W_t || !Y || !ws) return LORA_ERR_INVALID_ARG;
  if ((st = base_args(X, W_t, Y, T, K, pool, plan, ws, ws_bytes, f.cfg, f.g)) != LORA_OK) return st;
  f.split = gemm_plan_fusable(f.cfg);
  return LORA_OK;
}

PlanLaunch forward_plan(const int32_t *ids, const float *gates, int32_t T, int32_t K,
                        const lora_pool_desc *pool, void *plan, const Fwd &f, const ApplyWs &w) {
  PlanLaunch pl = plan_setup(ids, gates, T, K, pool_view(pool), static_cast<int32_t *>(plan), 256,
                             plan_lds_cap(f.cfg));
  // decode: the per-slot shrink runs beside the plan, whose U the epilogue
  // later moves to the u_off layout; the decode-shrink wave records are skipped
  if (w.slot_u) pl.a.no_sched = 1;
  return pl;
}

}  // namespace

extern "C" {

int32_t lora_forward_gemm(const int32_t *ids, const float *gates, int32_t T, int32_t K,
                          const void *X, const void *W_t, void *Y, const uint8_t *keep_mask,
                          float keep_scale, const lora_pool_desc *pool, void *plan,
                          size_t plan_bytes, void *ws, size_t ws_bytes, void *stream) {
  Fwd f;
  int32_t st = forward_args(ids, gates, T, K, X, W_t, Y, pool, plan, plan_bytes, ws, ws_bytes, f);
  if (st != LORA_OK) return st;
  if (!f.split) return lora_plan(ids, gates, T, K, pool, plan, plan_bytes, stream);
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const ApplyWs w = apply_layout(ws, ws_bytes, T, K, pool->d_in, pool->d_out, pool->dtype);
  if (w.slot_u) {
    SlotShrinkArgs ss{};
    ss.ids = ids; ss.gates = gates; ss.K = K; ss.N = pool->n_adapters;
    ss.Z = X; ss.mask = keep_mask; ss.extra_scale = keep_mask ? keep_scale : 1.0f;
    ss.d = pool->d_in; ss.pages = pool->a_pages;
    ss.rank = pool->rank; ss.page_start = pool->page_start; ss.page_ids = pool->page_ids;
    ss.scale = pool->scale; ss.n_pages = pool->n_pages; ss.n_page_ids = pool->n_page_ids;
    ss.out = w.slot_u; ss.stride = LORA_MAX_RANK; ss.n_slots = T * K; ss.sdesc = w.sdesc;
    return dev(launch_decode_slot_plan(f.cfg, f.g, ss,
                                       forward_plan(ids, gates, T, K, pool, plan, f, w), s));
  }
  return dev(launch_gemm_plan(f.cfg, f.g, forward_plan(ids, gates, T, K, pool, plan, f, w), s));
}

int32_t lora_forward_finish(const int32_t *ids, const float *gates, int32_t T, int32_t K,
                            const void *X, const void *W_t, void *Y, const uint8_t *keep_mask,
                            float keep_scale, const lora_pool_desc *pool, void *plan,
                            size_t plan_bytes, void *ws, size_t ws_bytes, void *stream) {
  Fwd f;
  int32_t st = forward_args(ids, gates, T, K, X, W_t, Y, pool, plan, plan_bytes, ws, ws_bytes, f);
  if (st != LORA_OK || T == 0) return st;
  if (!f.split)
    return lora_apply(X, W_t, Y, T, K, gates, keep_mask, keep_scale, pool, plan, ws, ws_bytes,
                      stream);
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const ApplyWs w = apply_layout(ws, ws_bytes, T, K, pool->d_in, pool->d_out, pool->dtype);
  if (w.slot_u)
    return dev(launch_epilogue_ucopy(f.cfg, f.g, pool->dtype, w.slot_u, w.sdesc, w.U, w.u_cap, s));
  st = lora_shrink(X, keep_mask, keep_scale, T, K, gates, pool, plan, ws, ws_bytes, stream);
  if (st != LORA_OK) return st;
  return lora_expand_epilogue(X, W_t, Y, T, K, pool, plan, ws, ws_bytes, stream);
}

int32_t lora_forward(const int32_t *ids, const float *gates, int32_t T, int32_t K,
                     const void *X, const void *W_t, void *Y, const uint8_t *keep_mask,
                     float keep_scale, const lora_pool_desc *pool, void *plan, size_t plan_bytes,
                     void *ws, size_t ws_bytes, void *stream) {
  int32_t st = lora_forward_gemm(ids, gates, T, K, X, W_t, Y, keep_mask, keep_scale, pool, plan,
                                 plan_bytes, ws, ws_bytes, stream);
  if (st != LORA_OK || T == 0) return st;
  return lora_forward_finish(ids, gates, T, K, X, W_t, Y, keep_mask, keep_scale, pool, plan,
                             plan_bytes, ws, ws_bytes, stream);
}

}  // extern "C"

namespace {

MergeArgs merge_args(void *W_t, const lora_pool_desc *pool, const int32_t *merge_ids,
                     const float *coeffs, int32_t m) {
  MergeArgs a{};
  a.W = W_t; a.d_in = pool->d_in; a.d_out = pool->d_out;
  a.a_pages = pool->a_pages; a.b_pages = pool->b_pages;
  a.rank = pool->rank; a.page_start = pool->page_start; a.page_ids = pool->page_ids;
  a.scale = pool->scale;
  a.n_pages = pool->n_pages; a.n_page_ids = pool->n_page_ids; a.n_adapters = pool->n_adapters;
  a.ids = merge_ids; a.coeffs = coeffs; a.m = m;
  return a;
}

}  // namespace

extern "C" {

int32_t lora_merge_delta(void *W_t, const lora_pool_desc *pool, const int32_t *merge_ids,
                         const float *coeffs, int32_t m, void *stream) {
  int32_t st = check_pool(pool, true);
  if (st != LORA_OK) return st;
  if (m < 0 || !W_t) return LORA_ERR_INVALID_ARG;
  if (m == 0) return LORA_OK;
  if (!merge_ids || !coeffs) return LORA_ERR_INVALID_ARG;
  return dev(launch_merge(merge_args(W_t, pool, merge_ids, coeffs, m), pool->dtype,
                          static_cast<hipStream_t>(stream)));
}

int32_t lora_merge_delta_layers(const lora_layer_desc *layers, int32_t n_layers,
                                const int32_t *merge_ids, const float *coeffs, int32_t m,
                                void *stream) {
  if (n_layers < 0 || m < 0 || (n_layers > 0 && !layers)) return LORA_ERR_INVALID_ARG;
  for (int32_t l = 0; l < n_layers; ++l) {
    const int32_t st = check_pool(&layers[l].pool, true);
    if (st != LORA_OK) return st;
    if (!layers[l].W_t || layers[l].pool.dtype != layers[0].pool.dtype) return LORA_ERR_INVALID_ARG;
    for (int32_t q = 0; q < l; ++q)
      if (layers[q].W_t == layers[l].W_t) return LORA_ERR_INVALID_ARG;   // in place, once each
  }
  if (n_layers == 0 || m == 0) return LORA_OK;
  if (!merge_ids || !coeffs) return LORA_ERR_INVALID_ARG;
  constexpr int32_t kChunk = LORA_MERGE_MAX_LAYERS;
  MergeArgs a[kChunk];
  const hipStream_t s = static_cast<hipStream_t>(stream);
  for (int32_t l0 = 0; l0 < n_layers; l0 += kChunk) {
    const int32_t nl = n_layers - l0 < kChunk ? n_layers - l0 : kChunk;
    for (int32_t l = 0; l < nl; ++l)
      a[l] = merge_args(layers[l0 + l].W_t, &layers[l0 + l].pool, merge_ids, coeffs, m);
    const int32_t st = dev(launch_merge_layers(a, nl, layers[0].pool.dtype, s));
    if (st != LORA_OK) return st;
  }
  return LORA_OK;
}

size_t lora_grad_workspace_bytes(int32_t T, int32_t K, int32_t n_adapters, int32_t d_in,
                                 int32_t d_out, int32_t max_rank, int32_t dtype) {
  if (check_batch(T, K) != LORA_OK || !dims_ok(d_in) || !dims_ok(d_out) || n_adapters < 1) return 0;
  if (max_rank < 1 || max_rank > LORA_MAX_RANK) return 0;
  if (dtype != LORA_F32 && dtype != LORA_BF16) return 0;
  const int64_t TK = int64_t(T) * K;
  const size_t g = align_up(size_t(TK) * size_t(max_rank) * sizeof(float) + 4);
  const size_t pieces = size_t(grad_pieces(TK, n_adapters));
  const size_t pa = align_up(pieces * size_t(max_rank) * size_t(d_in) * sizeof(float));
  const size_t pb = align_up(pieces * size_t(max_rank) * size_t(d_out) * sizeof(float));
  // MFMA form: the per-tile dY.B^T partials
  const size_t gp = grad_mfma_form(dtype, TK, d_out)
                        ? align_up(size_t(grad_gpart_tiles(d_out)) * size_t(TK) * size_t(max_rank) *
                                   sizeof(float))
                        : 0;
  return g + pa + pb + gp;
}

int32_t lora_grad(const void *X, const uint8_t *keep_mask, float keep_scale, const void *dY,
                  int32_t T, int32_t K, const float *gates,
                  const lora_pool_desc *pool, const void *plan, const void *apply_ws,
                  size_t apply_ws_bytes, float *dA_pages, float *dB_pages, int32_t max_rank,
                  void *ws, size_t ws_bytes, void *stream) {
  int32_t st = check_batch(T, K);
  if (st != LORA_OK) return st;
  if ((st = check_pool(pool, true)) != LORA_OK) return st;
  if (!plan || max_rank < 1 || max_rank > LORA_MAX_RANK) return LORA_ERR_INVALID_ARG;
  if (T == 0) return LORA_OK;
  if (!X || !dY || !gates || !apply_ws || !dA_pages || !dB_pages || !ws)
    return LORA_ERR_INVALID_ARG;
  const int64_t TK = int64_t(T) * K;
  const size_t need = lora_grad_workspace_bytes(T, K, pool->n_adapters, pool->d_in, pool->d_out,
                                                max_rank, pool->dtype);
  if (ws_bytes < need) return LORA_ERR_CAPACITY;
  const ApplyWs aw = apply_layout(const_cast<void *>(apply_ws), apply_ws_bytes, T, K, pool->d_in,
                              pool->d_out, pool->dtype);
  if (aw.u_cap < 0) return LORA_ERR_CAPACITY;
  const PlanView pv = plan_view(plan, TK, pool->n_adapters);
  int32_t *err_word = const_cast<int32_t *>(pv.hdr) + LORA_PH_ERR;
  const hipStream_t s = static_cast<hipStream_t>(stream);

  char *base = static_cast<char *>(ws);
  const size_t g_bytes = align_up(size_t(TK) * size_t(max_rank) * sizeof(float) + 4);
  const size_t pieces = size_t(grad_pieces(TK, pool->n_adapters));
  const size_t pa = align_up(pieces * size_t(max_rank) * size_t(pool->d_in) * sizeof(float));
  float *G = reinterpret_cast<float *>(base);
  float *partA = reinterpret_cast<float *>(base + g_bytes);
  float *partB = reinterpret_cast<float *>(base + g_bytes + pa);
  const size_t pbytes = align_up(pieces * size_t(max_rank) * size_t(pool->d_out) * sizeof(float));
  const bool fused_g = grad_mfma_form(pool->dtype, TK, pool->d_out);
  float *gpart = fused_g ? reinterpret_cast<float *>(base + g_bytes + pa + pbytes) : nullptr;

  if (fused_g) {
    // prefill-size bf16 batches: dB and the per-tile dY.B^T partials in one
    // pass over dY, then G from the partials, then dA
    SegOuterArgs ob{};
    ob.Z = dY; ob.mask = nullptr; ob.T = T; ob.K = K; ob.d = pool->d_out;
    ob.coef = aw.U; ob.coef_cap = aw.u_cap; ob.plan = pv;
    ob.rank = pool->rank; ob.page_start = pool->page_start; ob.page_ids = pool->page_ids;
    ob.part = partB; ob.max_rank = max_rank; ob.out_pages = dB_pages; ob.err_word = err_word;
    ob.gpart = gpart; ob.b_pages = pool->b_pages;
    GReduceArgs gr{};
    gr.gpart = gpart; gr.n_tiles = grad_gpart_tiles(pool->d_out); gr.TK = TK;
    gr.max_rank = max_rank; gr.plan = pv; gr.rank = pool->rank; gr.scale = pool->scale;
    gr.extra_scale = keep_mask ? keep_scale : 1.0f;
    gr.G = G; gr.g_cap = int64_t(TK) * max_rank;
    // dB with the per-tile partials; its reduction launch also forms G
    hipError_t e = launch_seg_outer(ob, pool->dtype, TK, pool->n_adapters, s, &gr);
    if (e != hipSuccess) return LORA_ERR_DEVICE;
    SegOuterArgs oa = ob;
    oa.Z = X; oa.mask = keep_mask; oa.d = pool->d_in; oa.coef = G; oa.coef_cap = gr.g_cap;
    oa.part = partA; oa.out_pages = dA_pages;
    oa.gpart = nullptr; oa.b_pages = nullptr;
    return dev(launch_seg_outer(oa, pool->dtype, TK, pool->n_adapters, s));
  }

  // G = kappa . g . s . (dY . B_j): the shrink kernel on (dY, B pages)
  ShrinkArgs sa{};
  sa.Z = dY; sa.mask = nullptr; sa.extra_scale = keep_mask ? keep_scale : 1.0f;
  sa.T = T; sa.K = K; sa.d = pool->d_out;
  sa.pages = pool->b_pages;
  sa.rank = pool->rank; sa.page_start = pool->page_start; sa.page_ids = pool->page_ids;
  sa.scale = pool->scale; sa.gates = gates; sa.plan = pv; sa.err_word = err_word;
  sa.out = G; sa.out_cap = int64_t(TK) * max_rank;
  hipError_t e = launch_shrink(sa, pool->dtype, TK, pool->n_adapters, pool->d_in, pool->d_out, s);
  if (e != hipSuccess) return LORA_ERR_DEVICE;

  SegOuterArgs ob{};
  ob.Z = dY; ob.mask = nullptr; ob.T = T; ob.K = K; ob.d = pool->d_out;
  ob.coef = aw.U; ob.coef_cap = aw.u_cap; ob.plan = pv;
  ob.rank = pool->rank; ob.page_start = pool->page_start; ob.page_ids = pool->page_ids;
  ob.part = partB; ob.max_rank = max_rank; ob.out_pages = dB_pages; ob.err_word = err_word;
  e = launch_seg_outer(ob, pool->dtype, TK, pool->n_adapters, s);
  if (e != hipSuccess) return LORA_ERR_DEVICE;

  SegOuterArgs oa = ob;
  oa.Z = X; oa.mask = keep_mask; oa.d = pool->d_in; oa.coef = G; oa.coef_cap = sa.out_cap;
  oa.part = partA;
  oa.out_pages = dA_pages;
  e = launch_seg_outer(oa, pool->dtype, TK, pool->n_adapters, s);
  return dev(e);
}

}  // extern "C"

namespace {

// dX GEMM: dY [T][d_out] times W [d_in][d_out] along d_out, into fp32 partials
// (the epilogue adds the masked LoRA term before the one rounding).
GemmConfig grad_x_config(int32_t T, int32_t d_in, int32_t d_out, int32_t dtype) {
  // the forward's choice: with 256 x 256 tiles the LoRA term and the keep
  // mask go into the GEMM's own epilogue, otherwise split partials and the
  // epilogue launch
  return choose_gemm(T > 0 ? T : 1, d_out, d_in, dtype);
}

}  // namespace

extern "C" {

int32_t lora_transpose(const void *src, void *dst, int32_t rows, int32_t cols, int32_t dtype,
                       void *stream) {
  if (!src || !dst || src == dst || rows < 0 || cols < 0) return LORA_ERR_INVALID_ARG;
  if (dtype != LORA_F32 && dtype != LORA_BF16) return LORA_ERR_INVALID_ARG;
  if (rows == 0 || cols == 0) return LORA_OK;
  return dev(launch_transpose(src, dst, rows, cols, dtype, static_cast<hipStream_t>(stream)));
}

size_t lora_grad_x_workspace_bytes(int32_t T, int32_t d_in, int32_t d_out, int32_t dtype) {
  if (T < 0 || !dims_ok(d_in) || !dims_ok(d_out)) return 0;
  if (dtype != LORA_F32 && dtype != LORA_BF16) return 0;
  const GemmConfig c = grad_x_config(T, d_in, d_out, dtype);
  const size_t b = gemm_partial_bytes(c, T, d_in);
  return align_up(b > 0 ? b : 1);
}

int32_t lora_grad_x(const void *dY, const void *W, const uint8_t *keep_mask, int32_t T, int32_t K,
                    const lora_pool_desc *pool, const void *plan, const void *grad_ws,
                    size_t grad_ws_bytes, int32_t max_rank, void *dX, void *ws, size_t ws_bytes,
                    void *stream) {
  int32_t st = check_batch(T, K);
  if (st != LORA_OK) return st;
  if ((st = check_pool(pool, true)) != LORA_OK) return st;
  if (!plan || max_rank < 1 || max_rank > LORA_MAX_RANK) return LORA_ERR_INVALID_ARG;
  if (T == 0) return LORA_OK;
  if (!dY || !W || !grad_ws || !dX || !ws) return LORA_ERR_INVALID_ARG;
  if (dX == dY || dX == W) return LORA_ERR_INVALID_ARG;
  if (grad_ws_bytes < lora_grad_workspace_bytes(T, K, pool->n_adapters, pool->d_in, pool->d_out,
                                                max_rank, pool->dtype))
    return LORA_ERR_CAPACITY;
  if (ws_bytes < lora_grad_x_workspace_bytes(T, pool->d_in, pool->d_out, pool->dtype))
    return LORA_ERR_CAPACITY;
  const int64_t TK = int64_t(T) * K;
  const PlanView pv = plan_view(plan, TK, pool->n_adapters);
  const GemmConfig c = grad_x_config(T, pool->d_in, pool->d_out, pool->dtype);
  GemmArgs g{};
  g.X = dY; g.W = W; g.M = T; g.N = pool->d_in; g.Kd = pool->d_out;
  g.k_split = c.k_split;
  g.sk_g = c.sk;
  g.partial = static_cast<float *>(ws);
  g.Y = dX;
  // the expand of the epilogue, on G (lora_grad's workspace starts with it,
  // packed like U) and the A pages, rows of d_in
  g.ex.K = K;
  g.ex.slot_desc = pv.slot_desc; g.ex.pair_tk = pv.pair_tk; g.ex.page_ids = pool->page_ids;
  g.ex.b_pages = pool->a_pages; g.ex.d_out = pool->d_in;
  g.ex.U = static_cast<const float *>(grad_ws); g.ex.hdr = pv.hdr;
  g.ex.u_cap = TK * max_rank;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (c.fused) {
    g.mask = keep_mask;
    return dev(launch_base_gemm(c, g, s));
  }
  hipError_t e = launch_base_gemm(c, g, s);
  if (e == hipSuccess) e = launch_grad_x_epilogue(c, g, pool->dtype, keep_mask, s);
  return dev(e);
}

}  // extern "C"

extern "C" {

size_t lora_tsqr_workspace_bytes(int32_t M, int32_t m, int32_t n) {
  if (!tsqr_shape_ok(M, m, n) || m > (1 << 24)) return 0;
  return align_up(tsqr_workspace_bytes(M, m, n));
}

int32_t lora_tsqr(const void *src, int32_t dtype, const int32_t *cols, int32_t M, int32_t m,
                  int32_t n, float *Qt, float *R, void *ws, size_t ws_bytes, void *stream) {
  if (dtype != LORA_F32 && dtype != LORA_BF16) return LORA_ERR_INVALID_ARG;
  if (M < 0 || m < 1 || n < 1) return LORA_ERR_INVALID_ARG;
  if (M == 0) return LORA_OK;
  if (!tsqr_shape_ok(M, m, n) || m > (1 << 24)) return LORA_ERR_UNSUPPORTED;
  if (!src || !cols || !R || !ws) return LORA_ERR_INVALID_ARG;
  if (ws_bytes < lora_tsqr_workspace_bytes(M, m, n)) return LORA_ERR_CAPACITY;
  return dev(launch_tsqr(src, dtype, cols, M, m, n, Qt, R, ws, static_cast<hipStream_t>(stream)));
}

}  // extern "C"

extern "C" {

size_t lora_compress_workspace_bytes(int32_t M, int32_t d_in, int32_t d_out, int32_t n) {
  if (M < 1 || n < 1 || n > 64 || !dims_ok(d_in) || !dims_ok(d_out) || n > d_in || n > d_out)
    return 0;
  return align_up(compress_workspace_bytes(M, d_in, d_out, n));
}

int32_t lora_compress(const lora_pool_desc *pool, const int32_t *adapters, int32_t M, int32_t n,
                      int32_t policy, float ratio, float energy, int32_t floor_rank, void *out_a,
                      void *out_b, int32_t *out_rank, float *out_sigma, void *ws, size_t ws_bytes,
                      void *stream) {
  int32_t st = check_pool(pool, true);
  if (st != LORA_OK) return st;
  if (M < 0 || n < 1 || (policy != 0 && policy != 1)) return LORA_ERR_INVALID_ARG;
  if (!(ratio > 0.f && ratio <= 1.f) || !(energy > 0.f && energy <= 1.f) || floor_rank < 0)
    return LORA_ERR_INVALID_ARG;
  if (M == 0) return LORA_OK;
  if (n > 64 || n > pool->d_in || n > pool->d_out) return LORA_ERR_UNSUPPORTED;
  if (!adapters || !out_a || !out_b || !out_rank || !out_sigma || !ws || pool->n_pages < 1 ||
      !pool->page_ids)
    return LORA_ERR_INVALID_ARG;
  if (ws_bytes < lora_compress_workspace_bytes(M, pool->d_in, pool->d_out, n)) return LORA_ERR_CAPACITY;
  return dev(launch_compress(pool_view(pool), adapters, M, n, policy, ratio, energy, floor_rank,
                             out_a, out_b, out_rank, out_sigma, ws, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
