// Combine: y[t] = sum over j ascending of g[t, j] * y_perm[row_pos[t*k + j]],
// accumulated in float32 and rounded to bf16 once.
#include "common.cuh"
#include "internal.h"

namespace bqmoe {
namespace {

// The row positions and gates of kJ consecutive j are read first and then
// their y_perm vectors, all loads of a batch in flight together; the fma
// chain then runs over them in j order (rows with an invalid position add
// nothing), so a call costs one round trip per batch rather than two per j.
constexpr int kJ = 8;
__global__ void __launch_bounds__(256) combine_kernel(const uint16_t *__restrict__ y_perm,
                                                      const int32_t *__restrict__ row_pos,
                                                      const float *__restrict__ gates, int T, int k, int H,
                                                      uint16_t *__restrict__ y) {
  const int t = blockIdx.y;
  const int h = (blockIdx.x * blockDim.x + threadIdx.x) * 8;
  if (h >= H) return;
  const int n = T * k;
  float acc[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) acc[q] = 0.f;
  for (int j0 = 0; j0 < k; j0 += kJ) {
    int p[kJ];
    float g[kJ];
#pragma unroll
    for (int b = 0; b < kJ; ++b) {
      const int j = min(j0 + b, k - 1);  // past k: re-read the last (not used)
      p[b] = row_pos[(size_t)t * k + j];
      g[b] = gates[(size_t)t * k + j];
    }
    u32x4 v[kJ];
#pragma unroll
    for (int b = 0; b < kJ; ++b) {
      const int pc = (p[b] >= 0 && p[b] < n) ? p[b] : 0;
      v[b] = *(const u32x4 *)(y_perm + (size_t)pc * H + h);
    }
#pragma unroll
    for (int b = 0; b < kJ; ++b) {
      if (j0 + b >= k || p[b] < 0 || p[b] >= n) continue;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        acc[2 * q] = __builtin_fmaf(g[b], bf16lo(v[b][q]), acc[2 * q]);
        acc[2 * q + 1] = __builtin_fmaf(g[b], bf16hi(v[b][q]), acc[2 * q + 1]);
      }
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
