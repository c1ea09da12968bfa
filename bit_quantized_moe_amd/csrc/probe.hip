// Measurement probes: the device's achievable HBM read rate and bf16 MFMA
// rate, against which the layer's kernels are also rated (the spec sheet's
// 8 TB/s and 2.5 PFLOP/s are the other yardstick).
//
//  * stream_read_kernel: every thread reads eight 16-byte vectors, all in
//    flight at once, and folds them with xor, so no load can be dropped; one
//    word per block is written.  Loads of one wave cover 1 KiB contiguously.
//  * mfma_loop_kernel: every wave runs v_mfma_f32_16x16x32_bf16 back to back on
//    register operands, eight independent accumulators so that no MFMA waits
//    for the previous one's result; the accumulators are folded and written.
#include "common.cuh"
#include "internal.h"

namespace bqmoe {
namespace {

// Each thread reads kStreamU 16-byte vectors 4 KiB apart (a wave covers
// 1 KiB contiguously per load), all issued before any is used; a block covers
// 256 * kStreamU vectors.  Indexes past the end read the last vector again and
// are not folded, so every load is in bounds and none sits behind a branch.
constexpr int kStreamU = 8;
__global__ void __launch_bounds__(256) stream_read_kernel(const u32x4 *src, size_t n16, uint32_t *out) {
  const size_t base = (size_t)blockIdx.x * 256 * kStreamU + threadIdx.x;
  u32x4 v[kStreamU];
#pragma unroll
  for (int u = 0; u < kStreamU; ++u) v[u] = src[min(base + (size_t)u * 256, n16 - 1)];
  u32x4 acc = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int u = 0; u < kStreamU; ++u)
    if (base + (size_t)u * 256 < n16) acc ^= v[u];
  uint32_t w = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
  for (int d = 32; d >= 1; d >>= 1) w ^= __shfl_xor(w, d, 64);
  __shared__ uint32_t red[4];
  if (threadIdx.x % 64 == 0) red[threadIdx.x / 64] = w;
  __syncthreads();
  if (threadIdx.x == 0) out[blockIdx.x] = red[0] ^ red[1] ^ red[2] ^ red[3];
}

__global__ void __launch_bounds__(256) mfma_loop_kernel(int iters, float seed, float *out) {
  const float s = seed + (float)(threadIdx.x % 64) * 1e-3f;
  const bf16x8 a = {(__bf16)s, (__bf16)(s * 0.5f), (__bf16)1.f, (__bf16)-1.f, (__bf16)0.25f, (__bf16)s,
                    (__bf16)0.5f, (__bf16)-0.5f};
  const bf16x8 b = {(__bf16)0.5f, (__bf16)-0.25f, (__bf16)s, (__bf16)1.f, (__bf16)(s * 0.25f), (__bf16)-1.f,
                    (__bf16)0.125f, (__bf16)s};
  f32x4 c[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) c[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 8; ++j) c[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(j & 1 ? a : b, j & 2 ? a : b, c[j], 0, 0, 0);
  }
  f32x4 t = c[0];
#pragma unroll
  for (int j = 1; j < 8; ++j) t += c[j];
  if (threadIdx.x % 64 == 0) out[blockIdx.x * 4 + threadIdx.x / 64] = t[0] + t[1] + t[2] + t[3];
}

}  // namespace

size_t probe_stream_blocks(size_t bytes) { return (bytes / 16 + 256 * kStreamU - 1) / (256 * kStreamU); }

hipError_t launch_probe_stream(const void *buf, size_t bytes, uint32_t *out, hipStream_t st) {
  const size_t n16 = bytes / 16;
  if (n16 == 0) return hipSuccess;
  stream_read_kernel<<<(unsigned)probe_stream_blocks(bytes), 256, 0, st>>>((const u32x4 *)buf, n16, out);
  return hipGetLastError();
}

hipError_t launch_probe_mfma(int blocks, int iters, float *out, hipStream_t st) {
  mfma_loop_kernel<<<blocks, 256, 0, st>>>(iters, 1.0f, out);
  return hipGetLastError();
}

}  // namespace bqmoe
