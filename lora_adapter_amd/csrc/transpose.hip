// Transpose of a row-major matrix: dst[c][r] = src[r][c].
//
// The fine-tune backward needs the input gradient dX = dY . W^T, with W the
// frozen base weight (LoRAFusion explainer, section 解决什么真问题: only A and
// B train).  The base GEMM reads both operands along K; for dX the
// contraction runs over d_out, so its weight operand is W itself, [d_in][d_out]
// row-major, while the forward keeps W_t [d_out][d_in].  The frozen weight is
// transposed once (at load) and both layouts stay resident.
//
// 64 x 64 tiles through LDS: every global read and write is a run of 64
// consecutive elements (coalesced), the LDS tile padded by one element per
// row so that the column reads of the transposed store hit distinct banks.
#include "lora_internal.h"

namespace lora {
namespace {

template <typename E>
__global__ __launch_bounds__(256) void transpose_kernel(const E *src, E *dst, int rows, int cols) {
  __shared__ E tile[64][65];
  const int r0 = blockIdx.y * 64, c0 = blockIdx.x * 64;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;   // 4 waves, 64 lanes
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int r = r0 + ty + 4 * i, c = c0 + tx;
    if (r < rows && c < cols) tile[ty + 4 * i][tx] = src[int64_t(r) * cols + c];
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int c = c0 + ty + 4 * i, r = r0 + tx;
    if (c < cols && r < rows) dst[int64_t(c) * rows + r] = tile[tx][ty + 4 * i];
  }
}

}  // namespace

hipError_t launch_transpose(const void *src, void *dst, int rows, int cols, int dtype,
                            hipStream_t s) {
  const dim3 grid(unsigned((cols + 63) / 64), unsigned((rows + 63) / 64)), block(256);
  if (dtype == LORA_BF16)
    hipLaunchKernelGGL(transpose_kernel<uint16_t>, grid, block, 0, s,
                       static_cast<const uint16_t *>(src), static_cast<uint16_t *>(dst), rows, cols);
  else
    hipLaunchKernelGGL(transpose_kernel<float>, grid, block, 0, s, static_cast<const float *>(src),
                       static_cast<float *>(dst), rows, cols);
  return hipGetLastError();
}

}  // namespace lora
