// lora_forward_noalloc: lora_forward with its plan and workspace in a
// library-owned device array, for callers that cannot allocate device memory
// (code under HIP graph capture, tight serving loops, harnesses that forbid
// hipMalloc).  The caller still passes inputs and outputs.
//
// The array is a file-scope __device__ object: every GPU the library runs on
// holds its own copy, at its own address, until the process ends.  Its name
// in host code is a host-side stand-in, not a device address, so the device
// address is taken once per device with hipGetSymbolAddress (with that device
// current) and only that address is handed to the kernels.
#include <mutex>

#include "lora_internal.h"

using namespace lora;

namespace {

constexpr size_t kScratchBytes = size_t(64) << 20;   // LORA_NOALLOC_SCRATCH_BYTES
static_assert(kScratchBytes == LORA_NOALLOC_SCRATCH_BYTES, "header and library agree");
constexpr int kMaxDevices = 64;
constexpr size_t kAlign = 256;

__device__ __align__(256) char scratch[kScratchBytes];

std::mutex g_mu;
char *g_scratch[kMaxDevices];   // device address of `scratch` on each device, once known

// The current device's address of `scratch`, looked up on the first call on
// that device (with it current) and kept.
int32_t scratch_on_current_device(char **out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return LORA_ERR_DEVICE;
  if (dev < 0 || dev >= kMaxDevices) return LORA_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_scratch[dev] == nullptr) {
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
      return LORA_ERR_DEVICE;
    g_scratch[dev] = static_cast<char *>(p);
  }
  *out = g_scratch[dev];
  return LORA_OK;
}

size_t align_up(size_t x) { return (x + kAlign - 1) & ~(kAlign - 1); }

}  // namespace

extern "C" {

size_t lora_forward_noalloc_bytes(int32_t T, int32_t K, int32_t n_adapters, int32_t d_in,
                                  int32_t d_out, int32_t max_rank, int32_t dtype) {
  const size_t plan = lora_plan_bytes(T, K, n_adapters);
  const size_t ws = lora_apply_workspace_bytes(T, K, d_in, d_out, max_rank, dtype);
  if (plan == 0 || ws == 0) return 0;
  return align_up(plan) + ws;
}

int32_t lora_forward_noalloc(const int32_t *ids, const float *gates, int32_t T, int32_t K,
                             const void *X, const void *W_t, void *Y, const uint8_t *keep_mask,
                             float keep_scale, const lora_pool_desc *pool, int32_t max_rank,
                             void *stream) {
  // host-visible checks first, before any HIP call
  if (!pool) return LORA_ERR_INVALID_ARG;
  if (T < 0 || K < 1 || K > LORA_MAX_K) return LORA_ERR_INVALID_ARG;
  if (max_rank < 0 || max_rank > LORA_MAX_RANK) return LORA_ERR_INVALID_ARG;
  const size_t need = lora_forward_noalloc_bytes(T, K, pool->n_adapters, pool->d_in, pool->d_out,
                                                 max_rank, pool->dtype);
  if (need == 0) return LORA_ERR_INVALID_ARG;
  if (need > kScratchBytes) return LORA_ERR_CAPACITY;
  if (T > 0 && (!ids || !gates || !X || !W_t || !Y)) return LORA_ERR_INVALID_ARG;
  char *base = nullptr;
  const int32_t st = scratch_on_current_device(&base);
  if (st != LORA_OK) return st;
  const size_t plan_bytes = align_up(lora_plan_bytes(T, K, pool->n_adapters));
  return lora_forward(ids, gates, T, K, X, W_t, Y, keep_mask, keep_scale, pool, base, plan_bytes,
                      base + plan_bytes, need - plan_bytes, stream);
}

}  // extern "C"
