// NVFP4 activation quantiser (page "Qwen3.8-Flash-Next NVFP4", "Format": W4A4
// E2M1 in groups of 16; the group scale is FP8 E4M3 and one float32 scale
// covers the tensor, as NVFP4 defines them).  One thread per group of 16:
//   amax = max |x|,  s = E4M3(amax / (6 G)),  q = E2M1(x / (s G))  (0 if s = 0)
// and the output is q * s as bf16 (exact: 2 x 4 significant bits); the
// tensor scale G is applied after the products.  Each step is one float32
// operation in that order, so the codes are those of any IEEE implementation
// of the same steps.
#include "common.cuh"
#include "internal.h"

namespace bqmoe {
namespace {

__global__ void __launch_bounds__(256) quant_nvfp4_kernel(const uint16_t *__restrict__ x, int64_t n_groups, float G,
                                                          uint16_t *__restrict__ vals, uint8_t *__restrict__ scales) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n_groups) return;
  const u32x4 *src = (const u32x4 *)(x + i * 16);
  const u32x4 a = src[0], b = src[1];
  float v[16];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    v[2 * j] = bf16lo(a[j]);
    v[2 * j + 1] = bf16hi(a[j]);
    v[8 + 2 * j] = bf16lo(b[j]);
    v[8 + 2 * j + 1] = bf16hi(b[j]);
  }
  float amax = 0.f;
#pragma unroll
  for (int j = 0; j < 16; ++j) amax = fmaxf(amax, fabsf(v[j]));
  const float s = round_e4m3(amax / (6.f * G));
  const float sg = s * G;
  uint32_t o[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const float q0 = sg > 0.f ? round_e2m1(v[2 * j] / sg) : 0.f;
    const float q1 = sg > 0.f ? round_e2m1(v[2 * j + 1] / sg) : 0.f;
    o[j] = pack_bf16x2(q0 * s, q1 * s);
  }
  u32x4 *dst = (u32x4 *)(vals + i * 16);
  dst[0] = u32x4{o[0], o[1], o[2], o[3]};
  dst[1] = u32x4{o[4], o[5], o[6], o[7]};
  if (scales) scales[i] = (uint8_t)f32_to_e4m3_code(s);
}

}  // namespace

hipError_t launch_quant_nvfp4(const uint16_t *x, int64_t n, float G, uint16_t *vals, uint8_t *scales, hipStream_t st) {
  const int64_t groups = n / 16;
  const unsigned blocks = (unsigned)((groups + 255) / 256);
  quant_nvfp4_kernel<<<blocks, 256, 0, st>>>(x, groups, G, vals, scales);
  return hipGetLastError();
}

}  // namespace bqmoe
