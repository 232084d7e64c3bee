/*
 * lora.h - C ABI of the batched multi-adapter LoRA layer on AMD Instinct
 * MI355X (gfx950).
 *
 *   Y = X.W + sum over a token's active slots k of  g[t][k] . s_a . (x~_t . A_a) . B_a
 *
 * where a = ids[t][k], x~_t is the token row (times a dropout keep mask and
 * its scale when one is given), A_a is d_in x r_a and B_a is r_a x d_out.
 * Pages cited (by title and section):
 *   [LoRAFusion] "LoRAFusion：消除冗余内存访问的多 LoRA 高效微调系统",
 *                section 解决什么真问题: A in R^{d x r}, B in R^{r x k};
 *                forward Y = X.W + X.(A.B), dropout among the small ops.
 *   [S-LoRA]     "S-LoRA：一个GPU运行数千大模型成为可能", section 批处理:
 *                batched base GEMM, every request's xAB added by custom
 *                kernels without padding; merging one adapter into W;
 *                section Unified Paging: one page per rank row.
 *   [AdaFuse]    "AdaFuse: Accelerating Dynamic Adapter Inference via
 *                Token-Level Pre-Gating and Fused Kernel Optimization",
 *                section 关键设计: item 1 gate-weighted experts (top-2),
 *                item 2 fused switch with negated previous adapters,
 *                item 3 segmented gather (rows grouped by adapter).
 *   [LoRAForge]  "LoRAForge：压缩与执行协同，让多LoRA服务更高效",
 *                section LoRAForge的核心设计: explicit retained ranks,
 *                rank-specialised kernels.
 *
 * Conventions for every entry point
 *   - All tensor pointers are DEVICE pointers owned by the caller; the
 *     library never allocates or frees, keeps no state, and never
 *     synchronises (lora_plan_header, a host-side reader, is the exception).
 *   - `stream` is a hipStream_t (NULL = the null stream).  Work is enqueued
 *     asynchronously on it; buffers must outlive the enqueued work.
 *   - Host-visible argument errors return a status BEFORE any HIP call.
 *     A failed kernel launch returns LORA_ERR_DEVICE.  Data-dependent errors
 *     (bad adapter ids, ranks or page tables, too-small U capacity) cannot be
 *     seen on the host without a sync: kernels OR LORA_DEVERR_* bits into
 *     word 2 of the plan header and skip the offending slots.
 *   - dtype LORA_F32: X, W_t, pages, Y are float32.  LORA_BF16: they are
 *     bfloat16 (raw 16-bit patterns); accumulation is always float32 and
 *     each output element is rounded once (nearest-even).
 *   - Row-major everywhere; d_in and d_out must be multiples of 64.
 */
#ifndef LORA_H
#define LORA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define LORA_ABI_VERSION 1
#define LORA_MAX_RANK 1024         /* largest rank a pool may hold            */
#define LORA_MAX_K 8               /* largest number of slots per token       */
#define LORA_N_BUCKETS 9           /* rank buckets <=1,2,4,...,128, >128      */
#define LORA_PLAN_HEADER_INTS 16

typedef enum {
  LORA_OK = 0,
  LORA_ERR_INVALID_ARG = 1,   /* null pointer, bad size, bad dtype          */
  LORA_ERR_UNSUPPORTED = 2,   /* shape the kernels do not handle            */
  LORA_ERR_CAPACITY = 3,      /* plan or workspace buffer too small         */
  LORA_ERR_DEVICE = 4         /* a HIP call failed                          */
} lora_status;

typedef enum { LORA_F32 = 0, LORA_BF16 = 1 } lora_dtype;

/* Bits of plan header word 2 (written on the device). */
#define LORA_DEVERR_BAD_ID 1       /* id < -1 or id >= n_adapters           */
#define LORA_DEVERR_BAD_RANK 2     /* referenced adapter rank <0 or >MAX    */
#define LORA_DEVERR_BAD_POOL 4     /* used adapter's page table inconsistent */
#define LORA_DEVERR_CAPACITY 8     /* U does not fit in the apply workspace  */

/* Plan header words (int32). */
#define LORA_PH_PAIRS 0      /* P: active (token, slot) pairs                 */
#define LORA_PH_SEGS 1       /* S: segments = distinct used adapters          */
#define LORA_PH_ERR 2        /* LORA_DEVERR_* bits                            */
#define LORA_PH_RPAIRS 3     /* sum of ranks over pairs = length of U         */
#define LORA_PH_RUSED 4      /* sum of ranks over used adapters               */
#define LORA_PH_T 5
#define LORA_PH_K 6
#define LORA_PH_N 7

/*
 * One projection's adapter pool ([S-LoRA] Unified Paging: a rank-R adapter
 * occupies R pages, pages interleaved and non-contiguous; [LoRAForge]:
 * each adapter keeps its exact retained rank, nothing is padded).
 * Rank row j of adapter a (column j of A_a, row j of B_a) is page
 * page_ids[page_start[a] + j] of a_pages and of b_pages.
 * The struct itself is host memory; every pointer in it is device memory.
 */
typedef struct {
  int32_t dtype;              /* lora_dtype of a_pages and b_pages           */
  int32_t d_in;               /* length of an A page                         */
  int32_t d_out;              /* length of a B page                          */
  int32_t n_adapters;         /* N                                           */
  int64_t n_pages;            /* rows of a_pages and b_pages                 */
  int64_t n_page_ids;         /* length of page_ids                          */
  const void *a_pages;        /* [n_pages][d_in]                             */
  const void *b_pages;        /* [n_pages][d_out]                            */
  const int32_t *rank;        /* [N], 0..LORA_MAX_RANK                       */
  const int32_t *page_start;  /* [N+1], page_start[a+1]-page_start[a]==rank[a] */
  const int32_t *page_ids;    /* [n_page_ids], values in [0, n_pages)        */
  const float *scale;         /* [N], per-adapter output scale s_a           */
} lora_pool_desc;

int32_t lora_abi_version(void);
const char *lora_status_string(int32_t status);

/* ------------------------------------------------------------------ plan
 * Groups a batch's active (token, slot) pairs by adapter ([AdaFuse] 关键设计
 * item 3, segmented gather; [LoRAForge] rank-specialised execution).  A slot
 * is active when 0 <= ids[t][k] < N, rank > 0 and gates[t][k] != 0.
 * Pairs are sorted stably by (rank bucket, adapter, token, slot), bucket(r) =
 * smallest b in 0..7 with r <= 2^b, else 8.  The plan holds, as int32 arrays
 * at the byte offsets lora_plan_layout() returns:
 *   header[16]             words LORA_PH_*
 *   pair_tk[T*K]           first P: t*K+k of each sorted pair
 *   seg_adapter[T*K]       first S: adapter of each segment
 *   seg_off[T*K+1]         first S+1: pair offsets of segments
 *   seg_row_off[T*K+1]     first S+1: prefix sum of segment ranks
 *   bucket_seg_off[16]     first 10: first segment with bucket >= b
 *   u_off[T*K+1]           first P+1: prefix sum of pair ranks (U offsets)
 *   slot_pos[T*K]          sorted position of slot t*K+k, or -1
 *   pair_adapter[T*K]      first P: adapter of each sorted pair
 *   internal               the gate of each sorted pair, packed segment and
 *                          slot descriptors, the decode-shrink schedule,
 *                          the segments left to the MFMA shrink, and scratch
 *                          used while building
 * Header words 0..7 are the LORA_PH_* values; words 8..10 hold internal
 * scheduling counts; word 11 is 1 when the decode-shrink wave records were
 * built (lora_plan builds them; lora_forward's decode path does not, and a
 * later shrink over its plan finds its starts by search); the rest are 0.
 * Everything is integer and bit-exact.  Built once per batch and shared by
 * every layer that uses the same routing.
 *   ids   [T][K] int32 device; -1 marks an empty slot.
 *   gates [T][K] float32 device.
 *   pool  rank/page_start/page_ids/n_* are read; dtype, d_in and d_out
 *         decide which segments the later MFMA shrink takes.
 *   plan  device buffer of at least lora_plan_bytes(T, K, N) bytes.
 * Errors: INVALID_ARG (null, T<0, K outside 1..LORA_MAX_K, N<1),
 * CAPACITY (plan_bytes too small), DEVICE (launch failed). */
size_t lora_plan_bytes(int32_t T, int32_t K, int32_t n_adapters);
int32_t lora_plan_layout(int32_t T, int32_t K, int32_t n_adapters, int64_t offsets_out[9]);
int32_t lora_plan(const int32_t *ids, const float *gates, int32_t T, int32_t K,
                  const lora_pool_desc *pool, void *plan, size_t plan_bytes, void *stream);
/* Copies the plan header (LORA_PLAN_HEADER_INTS int32 words: P, S, error
 * bits, R_pairs, R_used, T, K, N, internal words) to host memory `out` once
 * the work queued on `stream` before this call has finished.  The one entry
 * point that waits: it enqueues a device-to-host copy on `stream` and
 * synchronises that stream, so a host can size later buffers by R_pairs or
 * read the device error bits.  `plan` is a device pointer to a plan buffer,
 * `out` host memory of 16 int32 owned by the caller.
 * Errors: INVALID_ARG (null plan or out), DEVICE (copy or sync failed). */
int32_t lora_plan_header(const void *plan, int32_t *out, void *stream);

/* ----------------------------------------------------------------- apply
 * Y = X.W + the LoRA term above ([S-LoRA] 批处理, [LoRAFusion]
 * 解决什么真问题, [AdaFuse] 关键设计 item 1).  Two stages:
 *   lora_shrink:      U[u_off[p] + j] = g.s_a.kappa . sum_i X[t][i].m[t][i].A_a[i][j]
 *                     for every planned pair p = (t, k), j < r_a  (float32)
 *   lora_base_expand: Y[t][n] = round( sum_i X[t][i].W_t[n][i]
 *                                 + sum_{p of t} sum_j U[u_off[p]+j].B_a[j][n] )
 *                     the expand runs in the epilogue of the base GEMM, on
 *                     its float32 accumulators, before the single rounding.
 * lora_apply = lora_shrink then lora_base_expand on the same stream.
 *   X      [T][d_in]   dtype,  W_t [d_out][d_in] dtype (nn.Linear layout),
 *   Y      [T][d_out]  dtype, must not alias X or W_t,
 *   K, gates as given to lora_plan (same T, K) and the plan built from them;
 *     later kernels read adapters and gates from the plan only (the plan
 *     records each pair's gate), so gates must not change in between,
 *   keep_mask [T][d_in] uint8 0/1 or NULL, keep_scale its scale (1/keep_p),
 *     applied to the LoRA branch input only,
 *   ws     workspace of >= lora_apply_workspace_bytes(T, K, d_in, d_out,
 *          max_rank, dtype) bytes (split-K partials; for decode shapes U per
 *          slot, LORA_MAX_RANK floats each, and a 16-byte descriptor per
 *          slot; U); U stays in it for lora_grad.
 * Rows whose slots are all inactive equal the base-only result bit for bit.
 * Errors: INVALID_ARG, UNSUPPORTED (d_in or d_out not a multiple of 64,
 * dtype mismatch), CAPACITY (ws_bytes too small for the base GEMM stage),
 * DEVICE.  If U needs more than the workspace holds, the LoRA term is
 * skipped and LORA_DEVERR_CAPACITY is set in the plan header. */
size_t lora_apply_workspace_bytes(int32_t T, int32_t K, int32_t d_in, int32_t d_out,
                                  int32_t max_rank, int32_t dtype);
/* Byte offset of U (float32, packed by u_off) inside the apply workspace. */
size_t lora_apply_u_offset(int32_t T, int32_t K, int32_t d_in, int32_t d_out, int32_t dtype);
int32_t lora_shrink(const void *X, const uint8_t *keep_mask, float keep_scale, int32_t T,
                    int32_t K, const float *gates, const lora_pool_desc *pool, const void *plan,
                    void *ws, size_t ws_bytes, void *stream);
int32_t lora_base_expand(const void *X, const void *W_t, void *Y, int32_t T, int32_t K,
                         const lora_pool_desc *pool, const void *plan,
                         void *ws, size_t ws_bytes, void *stream);
/* lora_base_expand in its two launches, same arguments, so that each can be
 * timed on the caller's stream: the MFMA GEMM (which also runs the expand and
 * stores Y when the shape uses the fused epilogue; otherwise it writes fp32
 * split-K partials into ws), then the epilogue kernel (sums the partials,
 * adds the expand, rounds, stores Y; a no-op for the fused epilogue). */
int32_t lora_base_gemm(const void *X, const void *W_t, void *Y, int32_t T, int32_t K,
                       const lora_pool_desc *pool, const void *plan,
                       void *ws, size_t ws_bytes, void *stream);
int32_t lora_expand_epilogue(const void *X, const void *W_t, void *Y, int32_t T, int32_t K,
                             const lora_pool_desc *pool, const void *plan,
                             void *ws, size_t ws_bytes, void *stream);
/* lora_shrink followed by lora_base_gemm, with lora_apply's arguments.  For
 * decode shapes (T <= 128, bf16) both run in one launch: the GEMM's
 * workgroups and the shrink's waves side by side.  lora_apply =
 * lora_shrink_gemm then lora_expand_epilogue. */
int32_t lora_shrink_gemm(const void *X, const void *W_t, void *Y, int32_t T, int32_t K,
                         const float *gates, const uint8_t *keep_mask, float keep_scale,
                         const lora_pool_desc *pool, const void *plan, void *ws,
                         size_t ws_bytes, void *stream);
int32_t lora_apply(const void *X, const void *W_t, void *Y, int32_t T, int32_t K,
                   const float *gates, const uint8_t *keep_mask,
                   float keep_scale, const lora_pool_desc *pool, const void *plan, void *ws,
                   size_t ws_bytes, void *stream);

/* lora_plan then lora_apply for one batch, as one call, in two launches
 * for the shapes whose base GEMM writes split-K partials (the GEMM does not
 * depend on the routing, so the plan is built beside other work):
 *   decode (T <= 128, bf16):
 *     lora_forward_gemm:   the GEMM's partials, the shrink per slot (each
 *       active slot gathers its own adapter's A pages, which needs no plan:
 *       Punica-style gather for few tokens per adapter) into a per-slot part
 *       of the workspace, with a descriptor per slot, and the plan, built by
 *       the launch's first workgroup;
 *     lora_forward_finish: the epilogue (partials + expand from the per-slot
 *       U and descriptors, one rounding), which also stores U in the plan's
 *       u_off layout.
 *   stream-K shapes and float32:
 *     lora_forward_gemm:   the GEMM's partials with the plan built by one
 *       more workgroup of the launch;
 *     lora_forward_finish: lora_shrink, then lora_expand_epilogue.
 *   other shapes: lora_forward_gemm = lora_plan, lora_forward_finish =
 *     lora_apply.
 * lora_forward = lora_forward_gemm then lora_forward_finish (same
 * arguments, same stream).  A slot is active under the plan's rule (id in
 * range, gate not 0, rank 1..LORA_MAX_RANK, consistent page_start, page ids
 * in range).  The per-slot shrink adds the same products in the same order
 * as the plan-driven shrink, so plan, U and Y equal those of lora_plan then
 * lora_apply bit for bit.  When U does not fit the workspace both paths
 * behave alike: the LoRA term is skipped (Y is the base product), U is not
 * stored and LORA_DEVERR_CAPACITY is set.
 *   Arguments as for lora_plan and lora_apply, on one stream.
 * Errors: those of lora_plan and lora_apply. */
int32_t lora_forward_gemm(const int32_t *ids, const float *gates, int32_t T, int32_t K,
                          const void *X, const void *W_t, void *Y, const uint8_t *keep_mask,
                          float keep_scale, const lora_pool_desc *pool, void *plan,
                          size_t plan_bytes, void *ws, size_t ws_bytes, void *stream);
int32_t lora_forward_finish(const int32_t *ids, const float *gates, int32_t T, int32_t K,
                            const void *X, const void *W_t, void *Y, const uint8_t *keep_mask,
                            float keep_scale, const lora_pool_desc *pool, void *plan,
                            size_t plan_bytes, void *ws, size_t ws_bytes, void *stream);
int32_t lora_forward(const int32_t *ids, const float *gates, int32_t T, int32_t K,
                     const void *X, const void *W_t, void *Y, const uint8_t *keep_mask,
                     float keep_scale, const lora_pool_desc *pool, void *plan, size_t plan_bytes,
                     void *ws, size_t ws_bytes, void *stream);

/* ---------------------------------------------------- forward, no allocation
 * For callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.
 * lora_forward (same arguments, same kernels, same results bit for bit) with
 * its plan and workspace in a device array the library owns:
 * LORA_NOALLOC_SCRATCH_BYTES per GPU, taken on the first call on that GPU and
 * held until the process ends.  Nothing is allocated or freed by the call.
 *   The caller passes inputs and outputs only; max_rank bounds the rank of
 *   every adapter the batch uses (it sizes U, as in
 *   lora_apply_workspace_bytes).  The stream must belong to the current
 *   device.  Every call on one GPU shares that GPU's array, which keeps the
 *   last call's plan and U: calls that overlap on one GPU (on different
 *   streams, or from different host threads) race, and must be ordered by
 *   the caller.  Each call rebuilds everything it reads from the array.
 *   lora_forward_noalloc_bytes gives the array bytes a batch needs (0 for
 *   invalid sizes).
 * Errors: INVALID_ARG (as lora_forward, or max_rank outside 0..LORA_MAX_RANK),
 * CAPACITY (the batch needs more than LORA_NOALLOC_SCRATCH_BYTES: use
 * lora_forward with caller-owned buffers), UNSUPPORTED, DEVICE. */
#define LORA_NOALLOC_SCRATCH_BYTES (64u << 20)
size_t lora_forward_noalloc_bytes(int32_t T, int32_t K, int32_t n_adapters, int32_t d_in,
                                  int32_t d_out, int32_t max_rank, int32_t dtype);
int32_t lora_forward_noalloc(const int32_t *ids, const float *gates, int32_t T, int32_t K,
                             const void *X, const void *W_t, void *Y, const uint8_t *keep_mask,
                             float keep_scale, const lora_pool_desc *pool, int32_t max_rank,
                             void *stream);

/* ----------------------------------------------------------------- merge
 * In place: W_t <- round( W_t + sum_i coeffs[i] . s_{a_i} . (A_{a_i} . B_{a_i})^T )
 * with the delta summed in float32 and one rounding per element.  One adapter
 * with coefficient +1 merges it ([S-LoRA] 批处理); -1 un-merges it; a list
 * with the previous adapters at -1 and the new ones at +1 is the fused switch
 * of [AdaFuse] 关键设计 item 2, done in one launch.  Duplicates add.
 *   W_t [d_out][d_in] dtype; merge_ids [m] int32 device; coeffs [m] float32
 *   device.  Ids outside [0, N) or with an inconsistent page table are
 *   skipped.  W_t must not be read or written by other work meanwhile.
 * Errors: INVALID_ARG, UNSUPPORTED, DEVICE. */
int32_t lora_merge_delta(void *W_t, const lora_pool_desc *pool, const int32_t *merge_ids,
                         const float *coeffs, int32_t m, void *stream);

/* ----------------------------------------------------- merge, many layers
 * The same signed merge applied to several layers' weights at once
 * ([AdaFuse] 关键设计 item 3: the merges of every layer packed into one
 * batched launch, blocked across layers, added in place; its three-step
 * inference flow switches the chosen adapters in all layers together):
 *   for every layer l:  W_t^l <- round( W_t^l + sum_i coeffs[i] . s^l_{a_i} . (A^l_{a_i} . B^l_{a_i})^T )
 * with each layer's own pool (its pages, ranks, page table and scales; ids
 * index every pool alike).  One launch covers up to LORA_MERGE_MAX_LAYERS
 * layers when every layer is bf16 with d_in and d_out multiples of 128 (the
 * MFMA merge form); otherwise each layer takes its own launch.  Per layer the
 * result is the same, bit for bit, as lora_merge_delta on that layer.
 *   layers   host array [n_layers]; W_t and every pool pointer are device
 *            memory; all layers share one dtype; no two layers share a W_t.
 *   merge_ids, coeffs, m   as for lora_merge_delta (device arrays).
 * Errors: INVALID_ARG (null, n_layers < 0, mixed dtypes, a W_t given twice),
 * UNSUPPORTED (a layer's width not a multiple of 64), DEVICE. */
#define LORA_MERGE_MAX_LAYERS 16
typedef struct {
  void *W_t;                  /* [d_out][d_in] of this layer                 */
  lora_pool_desc pool;        /* this layer's adapter pool                    */
} lora_layer_desc;
int32_t lora_merge_delta_layers(const lora_layer_desc *layers, int32_t n_layers,
                                const int32_t *merge_ids, const float *coeffs, int32_t m,
                                void *stream);

/* ------------------------------------------------------------------ grad
 * Gradients of <dY, Y> with respect to the factors of every used adapter
 * (only A and B train, W frozen: [LoRAFusion] 解决什么真问题; the pages give
 * no backward formula, this is the derivative of the forward above):
 *   dB_a[j][n] = sum_{p of a} U[u_off[p]+j] . dY[t][n]
 *   dA_a[i][j] = sum_{p of a} kappa.m[t][i].X[t][i] . g.s_a . (dY_t . B_a[j])
 * written as float32 pages: dA_pages[page][i], dB_pages[page][n] for every
 * page of every used adapter (overwritten); other pages are not touched.
 *   apply_ws is the workspace of the lora_apply that produced U for this
 *   plan, X, mask and gates.  max_rank bounds every used adapter's rank
 *   (LORA_DEVERR_CAPACITY if not).  ws >= lora_grad_workspace_bytes(...).
 * Reductions over tokens run in a fixed order: results are deterministic.
 * Errors: INVALID_ARG, UNSUPPORTED, CAPACITY, DEVICE. */
size_t lora_grad_workspace_bytes(int32_t T, int32_t K, int32_t n_adapters, int32_t d_in,
                                 int32_t d_out, int32_t max_rank, int32_t dtype);
int32_t lora_grad(const void *X, const uint8_t *keep_mask, float keep_scale, const void *dY,
                  int32_t T, int32_t K, const float *gates, const lora_pool_desc *pool,
                  const void *plan, const void *apply_ws, size_t apply_ws_bytes,
                  float *dA_pages, float *dB_pages, int32_t max_rank, void *ws,
                  size_t ws_bytes, void *stream);

/* ---------------------------------------------------------- pool residency
 * Which adapters occupy the GPU pool, and the copy of a batch's missing
 * adapters into it ([S-LoRA] 批处理, last paragraph: all adapters are held in
 * host memory and only the running batch's adapters are loaded to the GPU;
 * 内存管理 and Unified Paging: one shared pool of pages, one page per rank
 * row, non-contiguous).  The victim policy (the pages leave it open):
 *   - a batch needs its valid ids (0 <= a < N, rank > 0), once each, in
 *     ascending order; its protected set is those plus the previous admitted
 *     batch's adapters; if their ranks add up to more than the pool's pages
 *     the batch is refused (LORA_ERR_CAPACITY) and nothing changes;
 *   - needed adapters are stamped with the batch index (last use);
 *   - each needed adapter not resident, in ascending id order, takes rank
 *     pages: while too few are free, the resident adapter outside the
 *     protected set with the smallest (last use, id) is evicted; then the
 *     lowest-numbered free pages are taken, rank row j on the j-th;
 *   - its rows are copied in maximal runs of consecutive pages.
 * The tables a batch runs with give each resident adapter its rank and pages
 * (page_start the prefix sums, page_ids in adapter order); adapters that are
 * not resident have rank 0, so a plan over them sees no active slot. */
typedef struct lora_page_table lora_page_table;      /* host object */
typedef struct {
  int32_t adapter, row, page, count;  /* rank rows row..row+count-1 -> pages page..page+count-1 */
} lora_page_copy;
/* The policy alone, in host memory (no HIP call).  rank: host [N]. */
int32_t lora_page_table_create(const int32_t *rank, int32_t n_adapters, int64_t n_pages,
                               lora_page_table **out);
void lora_page_table_destroy(lora_page_table *pt);
/* Admits one batch (host ids [n], -1 and out-of-range ids ignored): writes the
 * copies to make (host array, max_copies >= n_pages) and the evicted
 * adapters (host array, max_evicted >= N).  Errors: INVALID_ARG, CAPACITY. */
int32_t lora_page_table_admit(lora_page_table *pt, const int32_t *ids, int64_t n,
                              lora_page_copy *copies, int64_t max_copies, int64_t *n_copies,
                              int32_t *evicted, int64_t max_evicted, int64_t *n_evicted);
/* The current tables into host arrays rank [N], page_start [N+1],
 * page_ids [n_pages] (the first *n_page_ids are set). */
int32_t lora_page_table_tables(const lora_page_table *pt, int32_t *rank, int32_t *page_start,
                               int32_t *page_ids, int64_t *n_page_ids);

/* The GPU side.  The store holds every adapter's rank rows in pinned host
 * memory (hipHostMalloc; pageable memory makes the copies synchronous):
 * adapter a's row j is row store_row[a] + j of store_a [rows][d_in] (column j
 * of A_a) and of store_b [rows][d_out] (row j of B_a).  All buffers are the
 * caller's and must outlive the object. */
typedef struct {
  int32_t dtype, d_in, d_out, n_adapters;
  int64_t n_pages;              /* pages of the device pool                    */
  const int32_t *rank;          /* host [N]: every adapter's rank              */
  const int64_t *store_row;     /* host [N]: first store row of each adapter   */
  const void *store_a;          /* pinned host [rows][d_in]                    */
  const void *store_b;          /* pinned host [rows][d_out]                   */
  void *a_pages;                /* device [n_pages][d_in]                      */
  void *b_pages;                /* device [n_pages][d_out]                     */
  const float *scale;           /* device [N]                                  */
  int32_t *tables;              /* device, lora_residency_table_ints() int32   */
  int32_t *staging;             /* pinned host, the same number of int32       */
} lora_residency_config;
typedef struct lora_residency lora_residency;        /* host object */
size_t lora_residency_table_ints(int32_t n_adapters, int64_t n_pages);
int32_t lora_residency_create(const lora_residency_config *cfg, lora_residency **out);
void lora_residency_destroy(lora_residency *r);
/* Admits a batch (host ids [n]) and, on copy_stream, copies its missing
 * adapters' rows into their pages and uploads its tables (one of two table
 * sets, alternating); compute_stream then waits for those copies.  When the
 * store is mapped into the device's address space (hipHostMalloc memory,
 * every base 16-byte aligned) the rows are copied by one gather kernel that
 * reads the store over the host link; otherwise by one copy call per run of
 * consecutive pages.  Pages and
 * the table set that batch i - 2 used are overwritten only after batch i - 2's
 * finish point, so the copies of batch i + 1 may run while batch i computes.
 * pool_out: the descriptor the batch's calls must use.  Every prepare is
 * followed by lora_residency_finish once the batch's work is queued; the
 * compute work of all batches goes to one stream.  The host waits only when a
 * table staging set is still being copied from (two batches back).
 * Errors: INVALID_ARG (no finish for the previous batch), CAPACITY, DEVICE. */
int32_t lora_residency_prepare(lora_residency *r, const int32_t *ids, int64_t n,
                               void *copy_stream, void *compute_stream, lora_pool_desc *pool_out);
/* Marks the end of the prepared batch's work on compute_stream. */
int32_t lora_residency_finish(lora_residency *r, void *compute_stream);
/* out = {batches prepared, rank rows copied, adapters evicted, bytes copied}. */
int32_t lora_residency_stats(const lora_residency *r, int64_t out[4]);
/* The object's page table (read it with lora_page_table_tables). */
const lora_page_table *lora_residency_page_table(const lora_residency *r);

/* ------------------------------------------------------- tall-skinny QR
 * Batched thin QR of M tall, skinny matrices ([LoRAForge] section
 * FlashTSQR：批量因子构造的加速器 and its TSQR note: QR factorisations of
 * thousands of adapter modules for post-hoc compression, computed as local
 * QRs of row blocks merged afterwards, parallel over modules and row blocks):
 *   A_i = Q_i . R_i,  Q_i m x n with orthonormal columns, R_i n x n upper
 *   triangular with a non-negative diagonal (unique for full column rank).
 * Matrix i is given by its n columns: column j is row cols[i * n + j] of src
 * ([rows][m], dtype), so an adapter's A (its pages of a_pages, m = d_in) or
 * B^T (its pages of b_pages, m = d_out) is factored where it lies.
 *   cols  device int32 [M * n];  1 <= n <= 64, n <= m <= 2^24.
 *   Qt    device float32 [M][n][m] (Q's columns, the page layout) or NULL.
 *   R     device float32 [M][n][n] row-major.
 *   ws    >= lora_tsqr_workspace_bytes(M, m, n) bytes.
 * Float32 Householder reflections; a zero column below the diagonal takes
 * none (its R diagonal entry is then the column's own entry, sign-fixed).
 * Errors: INVALID_ARG, UNSUPPORTED (shape), CAPACITY (ws), DEVICE. */
size_t lora_tsqr_workspace_bytes(int32_t M, int32_t m, int32_t n);
int32_t lora_tsqr(const void *src, int32_t dtype, const int32_t *cols, int32_t M, int32_t m,
                  int32_t n, float *Qt, float *R, void *ws, size_t ws_bytes, void *stream);

/* Retained-rank recompression of M adapters of rank n ([LoRAForge]
 * LoRAForge的核心设计: explicit retained ranks, LoRAForge-U a uniform fraction
 * of each module's rank, LoRAForge-S by each module's spectral energy; the
 * factors come from batched QRs, section FlashTSQR：批量因子构造的加速器).
 * For adapter adapters[i] with factors A (d_in x n) and B (n x d_out) in the
 * pool: A = Q_A.R_A and B^T = Q_B.R_B (lora_tsqr on its pages), the n x n core
 * R_A.R_B^T = U.S.V^T (one-sided Jacobi, float64), retained rank
 *   policy 0 (uniform):  k = ceil(ratio * n), product in float32;
 *   policy 1 (spectral): the smallest k whose leading squared singular values
 *                        reach the fraction `energy` of their sum;
 *   then k = min(n, max(k, floor_rank, 1)),
 * and the best rank-k factors A' = Q_A.U_k.sqrt(S_k), B' = sqrt(S_k).V_k^T.Q_B^T
 * (A'.B' is the best rank-k approximation of A.B) are written, in the pool's
 * dtype, as pages: column j of A' is row i * n + j of out_a [M * n][d_in], row
 * j of B' row i * n + j of out_b [M * n][d_out], for j < k (other rows are not
 * written).  out_rank [M] int32 (0 for an adapter whose rank is not n or
 * whose page table is bad), out_sigma [M][n] float32 (descending).  All
 * device memory; 1 <= n <= 64, n <= d_in, d_out; the adapter scale is not
 * folded in (it stays the adapter's).
 * Errors: INVALID_ARG, UNSUPPORTED, CAPACITY (ws below
 * lora_compress_workspace_bytes), DEVICE. */
size_t lora_compress_workspace_bytes(int32_t M, int32_t d_in, int32_t d_out, int32_t n);
int32_t lora_compress(const lora_pool_desc *pool, const int32_t *adapters, int32_t M, int32_t n,
                      int32_t policy, float ratio, float energy, int32_t floor_rank, void *out_a,
                      void *out_b, int32_t *out_rank, float *out_sigma, void *ws, size_t ws_bytes,
                      void *stream);

/* ------------------------------------------------------------ grad of X
 * Input gradient of the fine-tune backward, handed to the layer below
 * ([LoRAFusion] 解决什么真问题: W frozen, A and B trained, dropout on the LoRA
 * branch; the pages give no backward formula, this is the derivative of
 * <dY, Y> for the forward above):
 *   dX[t][i] = round( sum_n dY[t][n] . W[i][n]
 *                     + m[t][i] . sum_{p of t} sum_j G[u_off[p]+j] . A_a[i][j] )
 * with G[u_off[p]+j] = g . s_a . kappa . (dY_t . B_a[j]), which lora_grad
 * leaves at the start of its workspace (call lora_grad on the same batch
 * first; dX reads G from grad_ws).
 *   dY [T][d_out] dtype; W [d_in][d_out] dtype: the frozen weight in its
 *   mathematical orientation, i.e. W_t transposed once by lora_transpose (the
 *   product runs along d_out, and the GEMM reads both operands along it);
 *   keep_mask [T][d_in] uint8 0/1 or NULL (the mask the forward used; its
 *   scale is already in G); plan as for the forward; max_rank as given to
 *   lora_grad; dX [T][d_in] dtype, must not alias dY or W;
 *   ws >= lora_grad_x_workspace_bytes(T, d_in, d_out, dtype) (fp32 partial
 *   products of dY . W^T; a few bytes, unused, when the batch fills the GPU
 *   with 256 x 256 output tiles, whose epilogue adds the masked LoRA term).
 * Rows whose slots are all inactive equal dY . W^T (rounded once) exactly.
 * Errors: INVALID_ARG, UNSUPPORTED, CAPACITY (grad_ws smaller than
 * lora_grad_workspace_bytes for these sizes, or ws too small), DEVICE. */
size_t lora_grad_x_workspace_bytes(int32_t T, int32_t d_in, int32_t d_out, int32_t dtype);
int32_t lora_grad_x(const void *dY, const void *W, const uint8_t *keep_mask, int32_t T, int32_t K,
                    const lora_pool_desc *pool, const void *plan, const void *grad_ws,
                    size_t grad_ws_bytes, int32_t max_rank, void *dX, void *ws, size_t ws_bytes,
                    void *stream);
/* dst[c][r] = src[r][c] for a rows x cols row-major matrix of dtype (device
 * pointers, dst of cols x rows, not overlapping src).  Used once per frozen
 * weight to give lora_grad_x its W from W_t (rows = d_out, cols = d_in).
 * Errors: INVALID_ARG (null, aliasing, negative sizes, bad dtype), DEVICE. */
int32_t lora_transpose(const void *src, void *dst, int32_t rows, int32_t cols, int32_t dtype,
                       void *stream);

#ifdef __cplusplus
}
#endif

#endif /* LORA_H */
