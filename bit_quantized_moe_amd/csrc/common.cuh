// Device helpers shared by the MoE kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bqmoe {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;
constexpr int kGroup = 128;  // quantisation group along K

// Control block at the start of every workspace (int32 words).
//   [2]          sticky error flags (bit 0: a bounded wait timed out)
//   route workspace:
//   [32]         selector blocks finished (several selectors grouping rows)
//   expert-FFN workspace:
//   [64 ..]      per-active-expert counters, kCtrStride apart, then the fused
//                layer's "past routing" counters
constexpr int kCtlError = 2;
constexpr int kCtlRouteSel = 32;
constexpr int kCtlCounters = 64;
constexpr int kCtrStride = 32;   // ints between counters: one 128-byte line each
constexpr int kCtlWords = 1024;  // minimum control block: 4 KiB
constexpr size_t kCtlBytes = kCtlWords * 4;

__device__ __forceinline__ float bf16_to_f32(uint32_t b16) { return __uint_as_float(b16 << 16); }
__device__ __forceinline__ float bf16lo(uint32_t pair) { return __uint_as_float(pair << 16); }
__device__ __forceinline__ float bf16hi(uint32_t pair) { return __uint_as_float(pair & 0xffff0000u); }

// Two float32 -> packed bf16 pair (round to nearest even), lo in bits [0,16).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2 v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  __bf16 b = (__bf16)f;
  return __builtin_bit_cast(uint16_t, b);
}

// a.lo*b.lo + a.hi*b.hi + c for packed bf16 pairs, float32 accumulate.
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b), c,
                                         false);
}

// ---------------------------------------------------------------- decode-path unpack
// Offset form used by the GEMV kernels: a code field u (< 128) in the low byte
// of a bf16 whose high byte is 0x43 is exactly the value 128 + u.  The fields
// are isolated into bytes with one mask per shift, and v_perm_b32 pairs two
// of those bytes with the 0x43 bytes of `magic` (0x43434343, passed in a
// register).  The pairs come out in a fixed field order:
//   INT4 word          -> fields 0 2 4 6 1 3 5 7
//   INT2 word, half 0  -> fields 0 4 8 12 1 5 9 13
//   INT2 word, half 1  -> fields 2 6 10 14 3 7 11 15
// The activations are arranged in the same order, so that the dot product of
// a pair sequence with them, minus (128 + zero) * sum(x), is sum((u - zero) x).
constexpr int kOrder4[8] = {0, 2, 4, 6, 1, 3, 5, 7};
constexpr int kOrder2[16] = {0, 4, 8, 12, 1, 5, 9, 13, 2, 6, 10, 14, 3, 7, 11, 15};
constexpr uint32_t kMagic43 = 0x43434343u;
constexpr uint32_t kPermB01 = 0x04010400u;  // (byte 0, 0x43, byte 1, 0x43)
constexpr uint32_t kPermB23 = 0x04030402u;  // (byte 2, 0x43, byte 3, 0x43)

__device__ __forceinline__ u32x4 unpack4_pairs(uint32_t w, uint32_t magic) {
  const uint32_t lo = w & 0x0F0F0F0Fu, hi = (w >> 4) & 0x0F0F0F0Fu;
  return u32x4{__builtin_amdgcn_perm(magic, lo, kPermB01), __builtin_amdgcn_perm(magic, lo, kPermB23),
               __builtin_amdgcn_perm(magic, hi, kPermB01), __builtin_amdgcn_perm(magic, hi, kPermB23)};
}
__device__ __forceinline__ u32x4 unpack2_pairs(uint32_t w, int half, uint32_t magic) {
  const uint32_t a = (w >> (4 * half)) & 0x03030303u, b = (w >> (4 * half + 2)) & 0x03030303u;
  return u32x4{__builtin_amdgcn_perm(magic, a, kPermB01), __builtin_amdgcn_perm(magic, a, kPermB23),
               __builtin_amdgcn_perm(magic, b, kPermB01), __builtin_amdgcn_perm(magic, b, kPermB23)};
}

// INT8 fields are 8 bits wide, too many for the offset form: each byte u goes
// through a float conversion, exact for 0..255, whose upper 16 bits are the
// bf16 value u.  Two words (8 fields) -> four bf16 pairs in K order.
__device__ __forceinline__ u32x4 unpack8_bf16(uint32_t w0, uint32_t w1) {
  auto pr = [](uint32_t w, int b) {
    const float lo = (float)((w >> (8 * b)) & 0xFFu), hi = (float)((w >> (8 * b + 8)) & 0xFFu);
    return __builtin_amdgcn_perm(__float_as_uint(hi), __float_as_uint(lo), 0x07060302u);
  };
  return u32x4{pr(w0, 0), pr(w0, 2), pr(w1, 0), pr(w1, 2)};
}

// FP6 e2m3: 32 codes, a little-endian stream of 6-bit fields in six words ->
// 32 bf16 values in K order (16 pairs).  gfx950 converts the 32 codes in one
// instruction; with scale 1 every e2m3 value is exact in bf16.
//
// The conversion is written in inline asm, and the compiler's hazard
// recognizer does not look inside asm: it cannot count the wait states
// between this VALU write and a following MFMA that reads the result as its
// A or B operand (the ISA asks for two).  The s_nop after it, in the same
// statement, supplies five, so the result is safe to feed straight into an
// MFMA whatever the compiler schedules next.
typedef uint32_t u32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x6 __attribute__((ext_vector_type(6)));
__device__ __forceinline__ u32x16 fp6x32_to_bf16(u32x6 v) {
  u32x16 r;
  asm("v_cvt_scalef32_pk32_bf16_fp6 %0, %1, 1.0\n\ts_nop 4" : "=&v"(r) : "v"(v));
  return r;
}
__device__ __forceinline__ float fp16_to_f32(uint32_t h16) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)h16);
}

// ---------------------------------------------------------------- NVFP4
// E2M1 elements in groups of 16 with an FP8 E4M3 scale per group and a
// float32 tensor scale.  Rounding to either grid is to nearest, ties to even
// (rintf), with saturation; powers of two are applied with ldexp, so every
// step other than the rint is exact.
__device__ __forceinline__ int floor_log2_f32(float v) {  // v >= 0; zero and denormals give <= -127
  return (int)((__float_as_uint(v) >> 23) & 0xFFu) - 127;
}
// v >= 0 to the E4M3 grid (3 mantissa bits, smallest binade 2^-6, max 448)
__device__ __forceinline__ float round_e4m3(float v) {
  const int e = max(floor_log2_f32(v), -6);
  const float q = __builtin_ldexpf(1.f, e - 3);
  return fminf(__builtin_rintf(v / q) * q, 448.f);
}
// v to the E2M1 grid (1 mantissa bit, smallest binade 2^0, max 6), sign kept
__device__ __forceinline__ float round_e2m1(float v) {
  const float a = fabsf(v);
  const int e = max(floor_log2_f32(a), 0);
  const float q = __builtin_ldexpf(1.f, e - 1);
  return copysignf(fminf(__builtin_rintf(a / q) * q, 6.f), v);
}
// E4M3 code (sign ignored: scales are positive) -> its value
__device__ __forceinline__ float e4m3_to_f32(uint32_t c) {
  const uint32_t e = (c >> 3) & 15u, m = c & 7u;
  return e ? __uint_as_float(((e + 120u) << 23) | (m << 20)) : (float)m * 0.001953125f;
}
// an E4M3 grid value (>= 0) -> its code
__device__ __forceinline__ uint32_t f32_to_e4m3_code(float r) {
  if (r < 0.015625f) return (uint32_t)(r * 512.f);  // subnormal: m * 2^-9
  const uint32_t b = __float_as_uint(r);
  return ((((b >> 23) & 0xFFu) - 120u) << 3) | ((b >> 20) & 7u);
}
// NVFP4 quantisation of a group of 16 h values held by 16 consecutive lanes
// (one value each): the group maximum through xor shuffles inside the 16
// lanes, then the steps of the activation quantiser.  Returns q * s.
__device__ __forceinline__ float quant16_lanes(float hv, float G) {
  float amax = fabsf(hv);
#pragma unroll
  for (int d = 1; d < 16; d <<= 1) amax = fmaxf(amax, __shfl_xor(amax, d, 64));
  const float s = round_e4m3(amax / (6.f * G));
  const float sg = s * G;
  return (sg > 0.f ? round_e2m1(hv / sg) : 0.f) * s;
}

// Eight E2M1 codes of w (K order) times the group scale s -> four bf16 pairs,
// exact (2 x 4 significant bits).  gfx950 converts the two codes of a byte
// to bf16 in one instruction; its scale operand takes only a power of two,
// so it runs with scale 1 (exact values, low nibble first) and s is applied
// in float32.
__device__ __forceinline__ void dequant8_e2m1(uint32_t w, float s, uint32_t out[4]) {
  const bf16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 0);
  const bf16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 1);
  const bf16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 2);
  const bf16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 3);
  const uint32_t q[4] = {__builtin_bit_cast(uint32_t, p0), __builtin_bit_cast(uint32_t, p1),
                         __builtin_bit_cast(uint32_t, p2), __builtin_bit_cast(uint32_t, p3)};
#pragma unroll
  for (int b = 0; b < 4; ++b) out[b] = pack_bf16x2(bf16lo(q[b]) * s, bf16hi(q[b]) * s);
}

// Natural-order bf16 activations d (pairs (x0,x1), (x2,x3), ...) -> the pair
// order of the unpacked codes: o[i] = (x[ord[2i]], x[ord[2i+1]]).  N elements.
template <int N>
__device__ __forceinline__ void order_pairs(const uint32_t *d, uint32_t *o) {
#pragma unroll
  for (int i = 0; i < N / 2; ++i) {
    const int a = (N == 8) ? kOrder4[2 * i] : kOrder2[2 * i];
    const int b = (N == 8) ? kOrder4[2 * i + 1] : kOrder2[2 * i + 1];
    // a and b have the same parity in both orders
    o[i] = __builtin_amdgcn_perm(d[b / 2], d[a / 2], (a & 1) ? 0x07060302u : 0x05040100u);
  }
}

// ---------------------------------------------------------------- GEMM-path dequant
// The masked words below hold one field per byte.  Passed through an empty asm
// statement, their bits are opaque to the optimizer, which would otherwise
// fold the mask into every field's extraction (a bit-field extract, then a
// byte convert); this way each byte converts with one v_cvt_f32_ubyteN.  The
// asm emits no instruction.
__device__ __forceinline__ uint32_t field_bytes(uint32_t v) {
  asm("" : "+v"(v));
  return v;
}

// Eight 4-bit fields of w -> four packed bf16 pairs of (u - zoff) * s, in K order.
// (u - zoff) * s is exact in float32 (a small integer times a bf16 value); the
// conversion to bf16 rounds to nearest even.
__device__ __forceinline__ void dequant8_int4(uint32_t w, float s, float zs, uint32_t out[4]) {
  const uint32_t lo = field_bytes(w & 0x0F0F0F0Fu);          // fields 0, 2, 4, 6
  const uint32_t hi = field_bytes((w >> 4) & 0x0F0F0F0Fu);   // fields 1, 3, 5, 7
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const float f0 = (float)((lo >> (8 * b)) & 0xFFu);
    const float f1 = (float)((hi >> (8 * b)) & 0xFFu);
    out[b] = pack_bf16x2(__builtin_fmaf(f0, s, zs), __builtin_fmaf(f1, s, zs));
  }
}

// Four 8-bit fields of w (u = q + 128) -> two packed bf16 pairs of (u - 128) * s,
// in K order (zs = -128 * s).  (u - 128) * s has at most 16 significant bits, so
// the fma is exact in float32; the conversion to bf16 rounds to nearest even.
__device__ __forceinline__ void dequant4_int8(uint32_t w, float s, float zs, uint32_t out[2]) {
  const float f0 = (float)(w & 0xFFu), f1 = (float)((w >> 8) & 0xFFu);
  const float f2 = (float)((w >> 16) & 0xFFu), f3 = (float)(w >> 24);
  out[0] = pack_bf16x2(__builtin_fmaf(f0, s, zs), __builtin_fmaf(f1, s, zs));
  out[1] = pack_bf16x2(__builtin_fmaf(f2, s, zs), __builtin_fmaf(f3, s, zs));
}

// Sixteen 2-bit fields of w -> eight packed bf16 pairs of (u - z) * s, in K order.
// |u - z| <= 2 for z in {1, 2}, so the values are exact in bf16.
__device__ __forceinline__ void dequant16_int2(uint32_t w, float s, float zs, uint32_t out[8]) {
  const uint32_t f0 = field_bytes(w & 0x03030303u);          // fields 0, 4, 8, 12
  const uint32_t f1 = field_bytes((w >> 2) & 0x03030303u);   // fields 1, 5, 9, 13
  const uint32_t f2 = field_bytes((w >> 4) & 0x03030303u);   // fields 2, 6, 10, 14
  const uint32_t f3 = field_bytes((w >> 6) & 0x03030303u);   // fields 3, 7, 11, 15
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const float a0 = (float)((f0 >> (8 * b)) & 0xFFu);
    const float a1 = (float)((f1 >> (8 * b)) & 0xFFu);
    const float a2 = (float)((f2 >> (8 * b)) & 0xFFu);
    const float a3 = (float)((f3 >> (8 * b)) & 0xFFu);
    out[2 * b + 0] = pack_bf16x2(__builtin_fmaf(a0, s, zs), __builtin_fmaf(a1, s, zs));
    out[2 * b + 1] = pack_bf16x2(__builtin_fmaf(a2, s, zs), __builtin_fmaf(a3, s, zs));
  }
}

// ---------------------------------------------------------------- wave helpers
__device__ __forceinline__ int lane_id() { return __lane_id(); }

// Load through the scalar cache.  Only for data that no wave writes during
// the kernel, at a wave-uniform address.
template <typename T>
__device__ __forceinline__ T sload(const T *ptr) {
  return *(const __attribute__((address_space(4))) T *)ptr;
}

#define BQ_DPP_ADD(v, ctrl) \
  ((v) + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, (v)), (ctrl), 0xF, 0xF, false)))

// Sum of v over aligned groups of `width` lanes (1, 2, 4, ..., 64); every lane
// of a group receives the group sum.  Lane distances 1 and 2 use quad
// permutes, 4 and 8 the row (half-)mirror, 16 a ds_swizzle xor inside each
// half-wave, and the two halves are combined from v_readlane.  At every level
// a lane adds the sums of the two halves of its group (in either operand
// order, which float addition does not see), so the result is the balanced
// pairwise tree over the lanes in index order, bit for bit the same in every
// lane.
__device__ __forceinline__ uint32_t xor16_lanes(uint32_t x) {
  // bitmask swizzle: and 0x1f, or 0, xor 0x10 within each group of 32 lanes
  return (uint32_t)__builtin_amdgcn_ds_swizzle((int)x, 0x401F);
}
__device__ __forceinline__ float group_sum(float v, int width) {
  if (width >= 2) v = BQ_DPP_ADD(v, 0xB1);   // quad_perm [1,0,3,2]
  if (width >= 4) v = BQ_DPP_ADD(v, 0x4E);   // quad_perm [2,3,0,1]
  if (width >= 8) v = BQ_DPP_ADD(v, 0x141);  // row_half_mirror
  if (width >= 16) v = BQ_DPP_ADD(v, 0x140); // row_mirror
  if (width >= 32) v += __builtin_bit_cast(float, xor16_lanes(__builtin_bit_cast(uint32_t, v)));
  if (width >= 64) {
    const float lo = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 0));
    const float hi = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 32));
    v = lo + hi;
  }
  return v;
}

// Block barrier that orders LDS accesses only.  Unlike __syncthreads() it does
// not first wait for this wave's outstanding global loads, so weights already
// in flight stay in flight across it.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Wait until this wave's outstanding vector-memory operations (including
// stores) have completed: s_waitcnt vmcnt(0).
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

}  // namespace bqmoe
