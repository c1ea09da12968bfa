// Combine: y[t] = sum over j ascending of g[t, j] * y_perm[row_pos[t*k + j]],
// accumulated in float32 and rounded to bf16 once.
#include "common.cuh"
#include "internal.h"

namespace bqmoe {
namespace {

__global__ void __launch_bounds__(256) combine_kernel(const uint16_t *__restrict__ y_perm,
                                                      const int32_t *__restrict__ row_pos,
                                                      const float *__restrict__ gates, int T, int k, int H,
                                                      uint16_t *__restrict__ y) {
  const int t = blockIdx.y;
  const int h = (blockIdx.x * blockDim.x + threadIdx.x) * 8;
  if (h >= H) return;
  float acc[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) acc[q] = 0.f;
  for (int j = 0; j < k; ++j) {
    const int p = row_pos[(size_t)t * k + j];
    if (p < 0 || p >= T * k) continue;
    const float g = gates[(size_t)t * k + j];
    const u32x4 v = *(const u32x4 *)(y_perm + (size_t)p * H + h);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      acc[2 * q] = __builtin_fmaf(g, bf16lo(v[q]), acc[2 * q]);
      acc[2 * q + 1] = __builtin_fmaf(g, bf16hi(v[q]), acc[2 * q + 1]);
    }
  }
  u32x4 o;
#pragma unroll
  for (int q = 0; q < 4; ++q) o[q] = pack_bf16x2(acc[2 * q], acc[2 * q + 1]);
  *(u32x4 *)(y + (size_t)t * H + h) = o;
}

}  // namespace

hipError_t launch_combine(const uint16_t *y_perm, const int32_t *row_pos, const float *gates, int T, int k,
                          int H, uint16_t *y, hipStream_t st) {
  const int threads = 256;
  dim3 grid((H / 8 + threads - 1) / threads, T);
  combine_kernel<<<grid, threads, 0, st>>>(y_perm, row_pos, gates, T, k, H, y);
  return hipGetLastError();
}

}  // namespace bqmoe
