// Adapter pool residency: which adapters occupy the GPU pool's pages, and the
// asynchronous copy of a batch's missing adapters into it.
//
// S-LoRA keeps every adapter in host memory and loads only the adapters of
// the running batch to the GPU (page "S-LoRA：一个GPU运行数千大模型成为可能",
// section 批处理, last paragraph); adapters of different ranks share one pool
// of pages, one page per rank row, non-contiguous (sections 内存管理 and
// Unified Paging).  The pages leave the victim policy open; this one:
//   * a batch needs its valid ids (0 <= a < N, rank > 0), each once, in
//     ascending order; the protected set is those plus the previous admitted
//     batch's (whose kernels may still run while this batch is copied in);
//     if the protected set's ranks exceed the pool, the batch is refused and
//     nothing changes;
//   * needed adapters are stamped with the batch index (last use);
//   * each needed adapter that is not resident, in ascending id order, gets
//     rank pages: while too few are free, the resident adapter outside the
//     protected set with the smallest (last use, id) is evicted; then the
//     lowest-numbered free pages are taken, rank row j on the j-th;
//   * its rows are copied in maximal runs of consecutive pages.
//
// lora_page_table is that policy alone (host memory, no HIP call).
// lora_residency adds the GPU side: the runs are copied from a pinned host
// store into the pool's pages on a copy stream, the tables the kernels read
// (rank, page_start, page_ids, with rank 0 for adapters that are not
// resident) are uploaded into one of two device table sets, and the compute
// stream waits for both.  Batch i overwrites pages and the table set last
// used by batch i - 2 only after that batch's kernels have finished (its
// finish event), so with one compute stream the next batch's copies overlap
// the current batch's kernels.  When the store is mapped into the device's
// address space (pinned memory from hipHostMalloc is), the copies are one
// gather kernel that reads every copied row over the host link: one launch
// per batch instead of one copy call per run of pages, whose fixed cost
// dominated batches of many short runs.
#include <algorithm>
#include <set>
#include <vector>

#include "lora_internal.h"

struct lora_page_table {
  std::vector<int32_t> rank;
  int64_t n_pages = 0;
  std::vector<std::vector<int32_t>> pages;   // per adapter, empty when not resident
  std::vector<int64_t> last_use;
  std::vector<char> resident;
  std::set<int32_t> free_pages;
  int64_t batch = 0;
  std::vector<int32_t> prev;                  // adapters of the previous admitted batch
};

struct lora_residency {
  lora_page_table pt;
  lora_residency_config cfg;
  size_t esize = 0;
  int64_t set_ints = 0;                       // ints per table set
  hipEvent_t finish[2] = {nullptr, nullptr};  // batch i's kernels queued before this point
  hipEvent_t upload[2] = {nullptr, nullptr};  // staging set s has been copied out
  hipEvent_t ready = nullptr;
  bool finish_rec[2] = {false, false};
  bool upload_rec[2] = {false, false};
  int64_t prepared = 0;                       // batches prepared
  int64_t finished = 0;                       // batches finished
  int64_t rows_copied = 0, evictions = 0, bytes_copied = 0;
  std::vector<lora_page_copy> copies;
  std::vector<int32_t> evicted;
  bool gather = false;                        // copies by the gather kernel
  const char *dev_a = nullptr, *dev_b = nullptr;   // device addresses of the store
};

namespace {

int64_t align64(int64_t x) { return (x + 63) & ~int64_t(63); }

// One table set: rank [N], page_start [N+1], page_ids [n_pages], then the
// batch's copied rows as (store row, page) pairs [n_pages] (a page is written
// at most once per batch).
int64_t table_set_ints(int32_t N, int64_t n_pages) {
  const int64_t np = n_pages > 0 ? n_pages : 1;
  return align64(N) + align64(int64_t(N) + 1) + align64(np) + align64(2 * np);
}

// Copies rows [n_rows] of the store (mapped host memory) into the pool's
// pages: workgroups stride over the rows, 16 bytes per thread per step.
__global__ __launch_bounds__(256) void gather_rows_kernel(const int2 *rows, int n_rows, const char *sa,
                                                          const char *sb, char *ap, char *bp, int64_t ra,
                                                          int64_t rb) {
  for (int i = blockIdx.x; i < n_rows; i += gridDim.x) {
    const int2 e = rows[i];
    const uint4 *src_a = reinterpret_cast<const uint4 *>(sa + int64_t(e.x) * ra);
    const uint4 *src_b = reinterpret_cast<const uint4 *>(sb + int64_t(e.x) * rb);
    uint4 *dst_a = reinterpret_cast<uint4 *>(ap + int64_t(e.y) * ra);
    uint4 *dst_b = reinterpret_cast<uint4 *>(bp + int64_t(e.y) * rb);
    for (int64_t k = threadIdx.x; k < ra / 16; k += 256) dst_a[k] = src_a[k];
    for (int64_t k = threadIdx.x; k < rb / 16; k += 256) dst_b[k] = src_b[k];
  }
}

// The policy above.  On refusal nothing changes.
int32_t admit(lora_page_table &pt, const int32_t *ids, int64_t n,
              std::vector<lora_page_copy> &copies, std::vector<int32_t> &evicted) {
  const int32_t N = int32_t(pt.rank.size());
  std::vector<int32_t> need;
  for (int64_t i = 0; i < n; ++i) {
    const int32_t a = ids[i];
    if (a >= 0 && a < N && pt.rank[a] > 0) need.push_back(a);
  }
  std::sort(need.begin(), need.end());
  need.erase(std::unique(need.begin(), need.end()), need.end());
  std::vector<char> prot(size_t(N), 0);
  for (int32_t a : need) prot[a] = 1;
  for (int32_t a : pt.prev) prot[a] = 1;
  int64_t prot_pages = 0;
  for (int32_t a = 0; a < N; ++a)
    if (prot[a]) prot_pages += pt.rank[a];
  if (prot_pages > pt.n_pages) return LORA_ERR_CAPACITY;
  copies.clear();
  evicted.clear();
  for (int32_t a : need) pt.last_use[a] = pt.batch;
  for (int32_t a : need) {
    if (pt.resident[a]) continue;
    const int32_t r = pt.rank[a];
    while (int64_t(pt.free_pages.size()) < r) {
      int32_t victim = -1;
      for (int32_t v = 0; v < N; ++v) {
        if (!pt.resident[v] || prot[v]) continue;
        if (victim < 0 || pt.last_use[v] < pt.last_use[victim]) victim = v;
      }
      if (victim < 0) return LORA_ERR_CAPACITY;   // not reached: the protected set fits
      for (int32_t p : pt.pages[victim]) pt.free_pages.insert(p);
      pt.pages[victim].clear();
      pt.resident[victim] = 0;
      evicted.push_back(victim);
    }
    std::vector<int32_t> &pg = pt.pages[a];
    pg.clear();
    for (int32_t q = 0; q < r; ++q) {
      pg.push_back(*pt.free_pages.begin());
      pt.free_pages.erase(pt.free_pages.begin());
    }
    pt.resident[a] = 1;
    for (int32_t j = 0; j < r;) {
      int32_t k = j;
      while (k + 1 < r && pg[k + 1] == pg[k] + 1) ++k;
      copies.push_back(lora_page_copy{a, j, pg[j], k - j + 1});
      j = k + 1;
    }
  }
  pt.prev = need;
  ++pt.batch;
  return LORA_OK;
}

int64_t write_tables(const lora_page_table &pt, int32_t *rank, int32_t *page_start,
                     int32_t *page_ids) {
  const int32_t N = int32_t(pt.rank.size());
  int64_t o = 0;
  if (page_start) page_start[0] = 0;
  for (int32_t a = 0; a < N; ++a) {
    const int32_t r = pt.resident[a] ? pt.rank[a] : 0;
    if (rank) rank[a] = r;
    if (page_ids)
      for (int32_t q = 0; q < r; ++q) page_ids[o + q] = pt.pages[a][q];
    o += r;
    if (page_start) page_start[a + 1] = int32_t(o);
  }
  return o;
}

int32_t init_table(lora_page_table &pt, const int32_t *rank, int32_t N, int64_t n_pages) {
  if (!rank || N < 1 || n_pages < 0 || n_pages > (int64_t(1) << 31) - 1) return LORA_ERR_INVALID_ARG;
  pt.rank.assign(rank, rank + N);
  for (int32_t a = 0; a < N; ++a)
    if (pt.rank[a] < 0 || pt.rank[a] > LORA_MAX_RANK) return LORA_ERR_INVALID_ARG;
  pt.n_pages = n_pages;
  pt.pages.assign(size_t(N), {});
  pt.last_use.assign(size_t(N), -1);
  pt.resident.assign(size_t(N), 0);
  pt.free_pages.clear();
  for (int64_t p = 0; p < n_pages; ++p) pt.free_pages.insert(int32_t(p));
  pt.batch = 0;
  pt.prev.clear();
  return LORA_OK;
}

}  // namespace

extern "C" {

int32_t lora_page_table_create(const int32_t *rank, int32_t n_adapters, int64_t n_pages,
                               lora_page_table **out) {
  if (!out) return LORA_ERR_INVALID_ARG;
  *out = nullptr;
  lora_page_table *pt = new lora_page_table();
  const int32_t st = init_table(*pt, rank, n_adapters, n_pages);
  if (st != LORA_OK) {
    delete pt;
    return st;
  }
  *out = pt;
  return LORA_OK;
}

void lora_page_table_destroy(lora_page_table *pt) { delete pt; }

int32_t lora_page_table_admit(lora_page_table *pt, const int32_t *ids, int64_t n,
                              lora_page_copy *copies, int64_t max_copies, int64_t *n_copies,
                              int32_t *evicted, int64_t max_evicted, int64_t *n_evicted) {
  if (!pt || n < 0 || (n > 0 && !ids) || !n_copies || !n_evicted) return LORA_ERR_INVALID_ARG;
  // room for the worst case: every page its own run, every adapter evicted
  if (max_copies < pt->n_pages || max_evicted < int64_t(pt->rank.size())) return LORA_ERR_INVALID_ARG;
  if ((max_copies > 0 && !copies) || (max_evicted > 0 && !evicted)) return LORA_ERR_INVALID_ARG;
  std::vector<lora_page_copy> cp;
  std::vector<int32_t> ev;
  const int32_t st = admit(*pt, ids, n, cp, ev);
  if (st != LORA_OK) return st;
  std::copy(cp.begin(), cp.end(), copies);
  std::copy(ev.begin(), ev.end(), evicted);
  *n_copies = int64_t(cp.size());
  *n_evicted = int64_t(ev.size());
  return LORA_OK;
}

int32_t lora_page_table_tables(const lora_page_table *pt, int32_t *rank, int32_t *page_start,
                               int32_t *page_ids, int64_t *n_page_ids) {
  if (!pt || !rank || !page_start || !page_ids || !n_page_ids) return LORA_ERR_INVALID_ARG;
  *n_page_ids = write_tables(*pt, rank, page_start, page_ids);
  return LORA_OK;
}

size_t lora_residency_table_ints(int32_t n_adapters, int64_t n_pages) {
  if (n_adapters < 1 || n_pages < 0) return 0;
  return size_t(2 * table_set_ints(n_adapters, n_pages));
}

int32_t lora_residency_create(const lora_residency_config *cfg, lora_residency **out) {
  if (!out || !cfg) return LORA_ERR_INVALID_ARG;
  *out = nullptr;
  if (cfg->dtype != LORA_F32 && cfg->dtype != LORA_BF16) return LORA_ERR_INVALID_ARG;
  if (cfg->d_in <= 0 || cfg->d_out <= 0 || cfg->d_in % 64 || cfg->d_out % 64) return LORA_ERR_UNSUPPORTED;
  if (!cfg->rank || !cfg->store_row || !cfg->store_a || !cfg->store_b || !cfg->a_pages ||
      !cfg->b_pages || !cfg->scale || !cfg->tables || !cfg->staging)
    return LORA_ERR_INVALID_ARG;
  for (int32_t a = 0; a < cfg->n_adapters; ++a)
    if (cfg->store_row[a] < 0) return LORA_ERR_INVALID_ARG;
  lora_residency *r = new lora_residency();
  int32_t st = init_table(r->pt, cfg->rank, cfg->n_adapters, cfg->n_pages);
  if (st != LORA_OK) {
    delete r;
    return st;
  }
  r->cfg = *cfg;
  r->esize = cfg->dtype == LORA_BF16 ? 2 : 4;
  r->set_ints = table_set_ints(cfg->n_adapters, cfg->n_pages);
  bool ok = true;
  for (int s = 0; s < 2; ++s) {
    ok = ok && hipEventCreateWithFlags(&r->finish[s], hipEventDisableTiming) == hipSuccess;
    ok = ok && hipEventCreateWithFlags(&r->upload[s], hipEventDisableTiming) == hipSuccess;
  }
  ok = ok && hipEventCreateWithFlags(&r->ready, hipEventDisableTiming) == hipSuccess;
  if (!ok) {
    lora_residency_destroy(r);
    return LORA_ERR_DEVICE;
  }
  // the gather kernel when the store is device-mapped and every base is
  // 16-byte aligned (row sizes are multiples of 128 bytes); else one copy
  // call per run of pages
  void *da = nullptr, *db = nullptr;
  const bool aligned = ((reinterpret_cast<uintptr_t>(cfg->store_a) | reinterpret_cast<uintptr_t>(cfg->store_b) |
                         reinterpret_cast<uintptr_t>(cfg->a_pages) | reinterpret_cast<uintptr_t>(cfg->b_pages)) %
                        16) == 0;
  if (aligned && hipHostGetDevicePointer(&da, const_cast<void *>(cfg->store_a), 0) == hipSuccess &&
      hipHostGetDevicePointer(&db, const_cast<void *>(cfg->store_b), 0) == hipSuccess && da && db) {
    r->gather = true;
    r->dev_a = static_cast<const char *>(da);
    r->dev_b = static_cast<const char *>(db);
  } else {
    (void)hipGetLastError();   // not mapped: the copy-call path, no error left behind
  }
  *out = r;
  return LORA_OK;
}

void lora_residency_destroy(lora_residency *r) {
  if (!r) return;
  for (int s = 0; s < 2; ++s) {
    if (r->finish[s]) hipEventDestroy(r->finish[s]);
    if (r->upload[s]) hipEventDestroy(r->upload[s]);
  }
  if (r->ready) hipEventDestroy(r->ready);
  delete r;
}

int32_t lora_residency_prepare(lora_residency *r, const int32_t *ids, int64_t n,
                               void *copy_stream, void *compute_stream, lora_pool_desc *pool_out) {
  if (!r || !pool_out || n < 0 || (n > 0 && !ids)) return LORA_ERR_INVALID_ARG;
  if (r->prepared != r->finished) return LORA_ERR_INVALID_ARG;   // the previous batch has no finish
  const int32_t st = admit(r->pt, ids, n, r->copies, r->evicted);
  if (st != LORA_OK) return st;
  const hipStream_t cs = static_cast<hipStream_t>(copy_stream);
  const hipStream_t ks = static_cast<hipStream_t>(compute_stream);
  const lora_residency_config &c = r->cfg;
  const int s = int(r->prepared & 1);
  // staging set s was last copied out two batches ago: wait until that is done
  if (r->upload_rec[s] && hipEventSynchronize(r->upload[s]) != hipSuccess) return LORA_ERR_DEVICE;
  int32_t *stg = c.staging + s * r->set_ints;
  const int32_t N = c.n_adapters;
  int32_t *rk = stg, *ps = stg + align64(N), *pid = ps + align64(int64_t(N) + 1);
  const int64_t npid = write_tables(r->pt, rk, ps, pid);
  // pages and table set s were last read by batch prepared - 2, which ended
  // before its finish event (one compute stream: earlier batches too)
  if (r->finish_rec[s] && hipStreamWaitEvent(cs, r->finish[s], 0) != hipSuccess) return LORA_ERR_DEVICE;
  char *ap = static_cast<char *>(c.a_pages);
  char *bp = static_cast<char *>(c.b_pages);
  const char *sa = static_cast<const char *>(c.store_a);
  const char *sb = static_cast<const char *>(c.store_b);
  const size_t ra = size_t(c.d_in) * r->esize, rb = size_t(c.d_out) * r->esize;
  const int64_t np = c.n_pages > 0 ? c.n_pages : 1;
  const int64_t list_off = align64(N) + align64(int64_t(N) + 1) + align64(np);
  int32_t *list = stg + list_off;             // (store row, page) of every copied row
  int64_t n_rows = 0;
  for (const lora_page_copy &q : r->copies) {
    const int64_t row = c.store_row[q.adapter] + q.row;
    if (r->gather) {
      for (int32_t i = 0; i < q.count; ++i) {
        list[2 * n_rows] = int32_t(row + i);
        list[2 * n_rows + 1] = q.page + i;
        ++n_rows;
      }
    } else if (hipMemcpyAsync(ap + size_t(q.page) * ra, sa + size_t(row) * ra, size_t(q.count) * ra,
                              hipMemcpyHostToDevice, cs) != hipSuccess ||
               hipMemcpyAsync(bp + size_t(q.page) * rb, sb + size_t(row) * rb, size_t(q.count) * rb,
                              hipMemcpyHostToDevice, cs) != hipSuccess) {
      return LORA_ERR_DEVICE;
    }
    r->rows_copied += q.count;
    r->bytes_copied += int64_t(q.count) * int64_t(ra + rb);
  }
  r->evictions += int64_t(r->evicted.size());
  int32_t *dev = c.tables + s * r->set_ints;
  // the tables, and the row list when the gather kernel copies
  const int64_t up = r->gather ? list_off + 2 * n_rows : list_off;
  if (hipMemcpyAsync(dev, stg, size_t(up) * sizeof(int32_t), hipMemcpyHostToDevice, cs) != hipSuccess)
    return LORA_ERR_DEVICE;
  if (r->gather && n_rows > 0) {
    const unsigned grid = unsigned(n_rows < 1024 ? n_rows : 1024);
    hipLaunchKernelGGL(gather_rows_kernel, dim3(grid), dim3(256), 0, cs,
                       reinterpret_cast<const int2 *>(dev + list_off), int(n_rows), r->dev_a, r->dev_b, ap, bp,
                       int64_t(ra), int64_t(rb));
    if (hipGetLastError() != hipSuccess) return LORA_ERR_DEVICE;
  }
  if (hipEventRecord(r->upload[s], cs) != hipSuccess || hipEventRecord(r->ready, cs) != hipSuccess ||
      hipStreamWaitEvent(ks, r->ready, 0) != hipSuccess)
    return LORA_ERR_DEVICE;
  r->upload_rec[s] = true;
  pool_out->dtype = c.dtype;
  pool_out->d_in = c.d_in;
  pool_out->d_out = c.d_out;
  pool_out->n_adapters = N;
  pool_out->n_pages = c.n_pages;
  pool_out->n_page_ids = npid;
  pool_out->a_pages = c.a_pages;
  pool_out->b_pages = c.b_pages;
  pool_out->rank = dev;
  pool_out->page_start = dev + align64(N);
  pool_out->page_ids = dev + align64(N) + align64(int64_t(N) + 1);
  pool_out->scale = c.scale;
  ++r->prepared;
  return LORA_OK;
}

int32_t lora_residency_finish(lora_residency *r, void *compute_stream) {
  if (!r || r->finished + 1 != r->prepared) return LORA_ERR_INVALID_ARG;
  const int s = int(r->finished & 1);
  if (hipEventRecord(r->finish[s], static_cast<hipStream_t>(compute_stream)) != hipSuccess)
    return LORA_ERR_DEVICE;
  r->finish_rec[s] = true;
  ++r->finished;
  return LORA_OK;
}

int32_t lora_residency_stats(const lora_residency *r, int64_t out[4]) {
  if (!r || !out) return LORA_ERR_INVALID_ARG;
  out[0] = r->prepared;
  out[1] = r->rows_copied;
  out[2] = r->evictions;
  out[3] = r->bytes_copied;
  return LORA_OK;
}

const lora_page_table *lora_residency_page_table(const lora_residency *r) {
  return r ? &r->pt : nullptr;
}

}  // extern "C"
