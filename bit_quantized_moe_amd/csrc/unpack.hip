// Diagnostic kernels that expose the two device dequantisation routines:
//  - moe_unpack_codes: the bf16 unpack of the decode GEMV kernels (offset
//    form for INT4 and 2-bit, a float conversion for INT8, the FP6 e2m3
//    conversion), converted back to signed integer codes (FP6: 8 * value);
//  - moe_dequant_bf16 / _grouped: the bf16 (q - z) * s of the grouped-GEMM
//    kernels.
#include "common.cuh"
#include "internal.h"

namespace bqmoe {
namespace {

template <int BITS>
__global__ void unpack_kernel(const uint32_t *__restrict__ words, int64_t n_words, int8_t *__restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n_words) return;
  const uint32_t w = words[i];
  constexpr int P = 32 / BITS;
  int8_t q[P];
  // bf16 pairs (128 + u) in the field order of the unpack, back to field order
  if constexpr (BITS == 8) {
    const u32x4 pr = unpack8_bf16(w, 0u);
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      q[2 * p] = (int8_t)((int)bf16lo(pr[p]) - 128);
      q[2 * p + 1] = (int8_t)((int)bf16hi(pr[p]) - 128);
    }
  } else if constexpr (BITS == 4) {
    const u32x4 pr = unpack4_pairs(w, kMagic43);
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      q[kOrder4[2 * p]] = (int8_t)((int)bf16lo(pr[p]) - 136);
      q[kOrder4[2 * p + 1]] = (int8_t)((int)bf16hi(pr[p]) - 136);
    }
  } else {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const u32x4 pr = unpack2_pairs(w, h, kMagic43);
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        q[kOrder2[8 * h + 2 * p]] = (int8_t)((int)bf16lo(pr[p]) - 128);
        q[kOrder2[8 * h + 2 * p + 1]] = (int8_t)((int)bf16hi(pr[p]) - 128);
      }
    }
  }
#pragma unroll
  for (int p = 0; p < P; ++p) out[i * P + p] = q[p];
}

// FP6: thread i converts the 32 codes of words 6i .. 6i+5 (the decode routine)
// and stores 8 * value, an integer in [-60, 60].
__global__ void unpack6_kernel(const uint32_t *__restrict__ words, int64_t n_groups, int8_t *__restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n_groups) return;
  const uint32_t *w = words + i * 6;
  const u32x16 v = fp6x32_to_bf16(u32x6{w[0], w[1], w[2], w[3], w[4], w[5]});
#pragma unroll
  for (int p = 0; p < 16; ++p) {
    out[i * 32 + 2 * p] = (int8_t)(int)(bf16lo(v[p]) * 8.f);
    out[i * 32 + 2 * p + 1] = (int8_t)(int)(bf16hi(v[p]) * 8.f);
  }
}

// FP6 dequant: thread i takes 32 codes (6 words) of one row, the GEMM routine.
__global__ void dequant6_kernel(const uint32_t *__restrict__ words, const uint16_t *__restrict__ scales, int N, int K,
                                uint16_t *__restrict__ out) {
  const int gpr = K / 32;  // 32-code groups per row
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (int64_t)N * gpr) return;
  const int n = (int)(i / gpr), gi = (int)(i % gpr);
  const float s = fp16_to_f32(scales[(size_t)n * (K / kGroup) + gi * 32 / kGroup]);
  const uint32_t *w = words + i * 6;
  const u32x16 v = fp6x32_to_bf16(u32x6{w[0], w[1], w[2], w[3], w[4], w[5]});
  uint32_t *dst = (uint32_t *)(out + (size_t)n * K + (size_t)gi * 32);
#pragma unroll
  for (int p = 0; p < 16; ++p) dst[p] = pack_bf16x2(bf16lo(v[p]) * s, bf16hi(v[p]) * s);
}

template <int BITS, int GS>
__global__ void dequant_kernel(const uint32_t *__restrict__ words, const uint16_t *__restrict__ scales,
                               const uint8_t *__restrict__ zeros, int N, int K, uint16_t *__restrict__ out) {
  constexpr int P = 32 / BITS;
  const int wpr = K / P;  // words per row
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (int64_t)N * wpr) return;
  const int n = (int)(i / wpr);
  const int kw = (int)(i % wpr);
  const int g = kw * P / GS;
  const float s = bf16_to_f32(scales[(size_t)n * (K / GS) + g]);
  const float z = BITS == 4 ? 8.f : BITS == 8 ? 128.f : (float)zeros[(size_t)n * (K / GS) + g];
  const uint32_t w = words[i];
  uint32_t o[P / 2];
  if constexpr (BITS == 8)
    dequant4_int8(w, s, -z * s, o);
  else if constexpr (BITS == 4)
    dequant8_int4(w, s, -z * s, o);
  else
    dequant16_int2(w, s, -z * s, o);
  uint32_t *dst = (uint32_t *)(out + (size_t)n * K + (size_t)kw * P);
#pragma unroll
  for (int p = 0; p < P / 2; ++p) dst[p] = o[p];
}

}  // namespace

hipError_t launch_unpack(const uint32_t *words, int bits, int64_t n_words, int8_t *out, hipStream_t st) {
  const int threads = 256;
  const int64_t blocks = (n_words + threads - 1) / threads;
  if (bits == 6) {
    const int64_t groups = n_words / 6;
    unpack6_kernel<<<(unsigned)((groups + threads - 1) / threads), threads, 0, st>>>(words, groups, out);
  } else if (bits == 8)
    unpack_kernel<8><<<(unsigned)blocks, threads, 0, st>>>(words, n_words, out);
  else if (bits == 4)
    unpack_kernel<4><<<(unsigned)blocks, threads, 0, st>>>(words, n_words, out);
  else
    unpack_kernel<2><<<(unsigned)blocks, threads, 0, st>>>(words, n_words, out);
  return hipGetLastError();
}

hipError_t launch_dequant_bf16(const uint32_t *words, const uint16_t *scales, const uint8_t *zeros, int bits,
                               int group, int N, int K, uint16_t *out, hipStream_t st) {
  const int threads = 256;
  const int64_t n_words = (int64_t)N * K * bits / 32;
  const unsigned blocks = (unsigned)((n_words + threads - 1) / threads);
  if (bits == 6) {
    const int64_t groups = (int64_t)N * (K / 32);
    dequant6_kernel<<<(unsigned)((groups + threads - 1) / threads), threads, 0, st>>>(words, scales, N, K, out);
  } else if (bits == 8 && group == 32)
    dequant_kernel<8, 32><<<blocks, threads, 0, st>>>(words, scales, zeros, N, K, out);
  else if (bits == 8)
    dequant_kernel<8, 128><<<blocks, threads, 0, st>>>(words, scales, zeros, N, K, out);
  else if (bits == 4 && group == 32)
    dequant_kernel<4, 32><<<blocks, threads, 0, st>>>(words, scales, zeros, N, K, out);
  else if (bits == 4)
    dequant_kernel<4, 128><<<blocks, threads, 0, st>>>(words, scales, zeros, N, K, out);
  else
    dequant_kernel<2, 128><<<blocks, threads, 0, st>>>(words, scales, zeros, N, K, out);
  return hipGetLastError();
}

}  // namespace bqmoe
