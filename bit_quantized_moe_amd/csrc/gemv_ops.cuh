// Weight-operand building blocks shared by the expert-FFN kernels that read
// packed weights straight into MFMA registers (the decode kernel and the
// middle-batch kernel): the formats, the activation chunk order that matches
// the unpacked codes, a lane's weight slices, and the per-128-K-unit MFMA with
// its scale / zero-point correction.
#pragma once

#include <type_traits>

#include "common.cuh"
#include "internal.h"

namespace bqmoe {
namespace {

// ---------------------------------------------------------------- formats
// BITS: 4 (INT4, field q + 8), 2 (field u, integer zero-point), 8 (INT8,
// field q + 128), 6 (FP6 e2m3 codes, fp16 scales) or 5, which stands for
// NVFP4 (4-bit E2M1 codes with an E4M3 scale per 16 K, the scale applied to B
// exactly; the activations arrive quantised).  GS: quantisation group along
// K, 128 or 32 (128 for NVFP4: the kernels' unit).  The kernels walk K in
// units of 128 (kGroup); a unit holds 128 / GS scales per row.
template <int BITS>
constexpr int kCodeBits = BITS == 5 ? 4 : BITS;
template <int GS>
constexpr int kSPU = kGroup / GS;
// Units whose weight loads a wave keeps in flight together: 8 of INT4 or
// 2-bit, 4 of INT8 (the same bytes); half that with groups of 32, whose four
// scales per unit and transposed slices take registers.
template <int BITS, int GS>
constexpr int kCG = (BITS >= 5 ? 4 : 8) / (GS == 32 ? 2 : 1);
// A scale's 16 bits as a float: fp16 for FP6, bf16 otherwise.
template <int BITS>
__device__ __forceinline__ float scale_f32(uint32_t b16) {
  if constexpr (BITS == 6)
    return fp16_to_f32(b16);
  else
    return bf16_to_f32(b16);
}

// ---------------------------------------------------------------- operands
// One chunk of natural-order bf16 activations (d: pairs (x0,x1), (x2,x3), ...)
// in the field order of the unpacked codes: INT4 chunks of 8, INT2 chunks of
// 16; INT8 and FP6 codes unpack in K order, so their chunks (of 8) stay as
// they are.
template <int BITS>
__device__ __forceinline__ void permute_chunk(const uint32_t *d, uint32_t *o) {
  if constexpr (BITS >= 5) {
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = d[i];
  } else {
    order_pairs<BITS == 4 ? 8 : 16>(d, o);
  }
}

// Activation elements per chunk of the operand order (see permute_chunk).
template <int BITS>
constexpr int kChunkE = BITS == 2 ? 16 : 8;

template <int BITS>
__device__ __forceinline__ void load_act_chunk(const uint16_t *src, int q, uint32_t *d) {
  const uint32_t *s32 = (const uint32_t *)(src + q * kChunkE<BITS>);
#pragma unroll
  for (int t = 0; t < kChunkE<BITS> / 2; t += 4) {
    const u32x4 v = *(const u32x4 *)(s32 + t);
    d[t] = v[0];
    d[t + 1] = v[1];
    d[t + 2] = v[2];
    d[t + 3] = v[3];
  }
}

template <int BITS>
__device__ __forceinline__ void store_act_chunk(uint8_t *row, int q, const uint32_t *d) {
  uint32_t o[kChunkE<BITS> / 2];
  permute_chunk<BITS>(d, o);
  uint32_t *dst = (uint32_t *)(row + q * kChunkE<BITS> * 2);
#pragma unroll
  for (int t = 0; t < kChunkE<BITS> / 2; t += 4) *(u32x4 *)(dst + t) = u32x4{o[t], o[t + 1], o[t + 2], o[t + 3]};
}

// ---------------------------------------------------------------- weights
// A lane reads 32 consecutive K of one weight row per 128-K unit: a 16-byte
// (INT4), 8-byte (INT2), 32-byte (INT8) or 24-byte (FP6) slice at byte
// lsub * kGroupBytes / 4 of the unit.
typedef uint32_t u32x8 __attribute__((ext_vector_type(8)));
template <int BITS>
using Word = typename std::conditional<
    BITS == 4 || BITS == 5, u32x4,
    typename std::conditional<BITS == 2, u32x2, typename std::conditional<BITS == 8, u32x8, u32x6>::type>::type>::type;
// One lane slice (FP6: 16 + 8 bytes, so that no load reaches past the slice).
template <int BITS>
__device__ __forceinline__ Word<BITS> load_word(const uint8_t *p) {
  if constexpr (BITS == 6) {
    const u32x4 a = *(const u32x4 *)p;
    const u32x2 b = *(const u32x2 *)(p + 16);
    return u32x6{a[0], a[1], a[2], a[3], b[0], b[1]};
  } else {
    return *(const Word<BITS> *)p;
  }
}
template <int BITS>
constexpr int kGroupBytes = kGroup * kCodeBits<BITS> / 8;

// kCG consecutive units of one row (the lane's slices), their bf16 scales
// (kCG * 128 / GS of them, two per word) and, for INT2, their zero-points
// (8 bytes).
template <int BITS, int GS>
struct Chunk {
  Word<BITS> w[kCG<BITS, GS>];
  // NVFP4: per unit the lane's two E4M3 group scales (its 32 K)
  uint32_t s[BITS == 5 ? kCG<BITS, GS> : kCG<BITS, GS> * kSPU<GS> / 2];
  u32x2 z;
};

// Offsets (bytes) of a lane's first unit in the expert's code, scale and
// zero-point arrays (SPU scales per unit).
struct Off {
  uint32_t c, s, z;
};
template <int SPU>
__device__ __forceinline__ Off row_off(int row, int G, int g0, int gbytes, int lsub) {
  Off o;
  o.z = (uint32_t)row * G + g0;
  o.s = 2 * SPU * o.z;
  o.c = o.z * gbytes + lsub * (gbytes / 4);
  return o;
}
template <int SPU>
__device__ __forceinline__ Off add_groups(Off o, int dg, int gbytes) {
  return Off{o.c + dg * gbytes, o.s + 2 * SPU * dg, o.z + dg};
}

// Expert-local arrays (wave-uniform bases).
struct ExpertW {
  const uint8_t *codes, *scales, *zeros;
};
// Expert e's W13 (first = 0) or W2 (first = 3) blocks from the address table
// (wave-uniform entries, read through the scalar cache).  The table the
// pages describe lets experts live anywhere the GPU can read, e.g. pinned
// host memory read in place (page "Qwen3.8-Flash-Next on one 24 GB GPU",
// "What the patch does").
__device__ __forceinline__ ExpertW expert_from_table(const uint64_t *tab, int e, int first) {
  const uint64_t *t = tab + (size_t)e * kTabStride + first;
  return ExpertW{(const uint8_t *)sload(t), (const uint8_t *)sload(t + 1), (const uint8_t *)sload(t + 2)};
}

template <int BITS, int GS>
__device__ __forceinline__ void load_chunk(const ExpertW &x, Off o, Chunk<BITS, GS> &ch) {
  constexpr int CG = kCG<BITS, GS>;
  constexpr int NS = CG * kSPU<GS> / 2;  // scale words: 4 (16 bytes), 2 or 8
#pragma unroll
  for (int c = 0; c < CG; ++c) ch.w[c] = load_word<BITS>(x.codes + o.c + c * kGroupBytes<BITS>);
  if constexpr (BITS == 5) {  // 8 scale bytes per unit; o.s already points at the lane's two
#pragma unroll
    for (int c = 0; c < CG; ++c) ch.s[c] = *(const uint16_t *)(x.scales + o.s + 8 * c);
  } else if constexpr (NS == 2) {
    const u32x2 v = *(const u32x2 *)(x.scales + o.s);
    ch.s[0] = v[0];
    ch.s[1] = v[1];
  } else {
#pragma unroll
    for (int h = 0; h < NS / 4; ++h) {
      const u32x4 v = *(const u32x4 *)(x.scales + o.s + 16 * h);
#pragma unroll
      for (int i = 0; i < 4; ++i) ch.s[4 * h + i] = v[i];
    }
  }
  if constexpr (BITS == 2) ch.z = *(const u32x2 *)(x.zeros + o.z);
}

// B operand j (8 K per lane) from words of the lane's slice: INT4 word j, INT2
// half j & 1 of word j / 2, INT8 words 2j and 2j + 1.
template <int BITS>
__device__ __forceinline__ bf16x8 b_op(Word<BITS> w, int j, uint32_t magic) {
  if constexpr (BITS == 4)
    return __builtin_bit_cast(bf16x8, unpack4_pairs(w[j], magic));
  else if constexpr (BITS == 2)
    return __builtin_bit_cast(bf16x8, unpack2_pairs(w[j / 2], j & 1, magic));
  else
    return __builtin_bit_cast(bf16x8, unpack8_bf16(w[2 * j], w[2 * j + 1]));
}

// C (16 activation rows x 16 weight rows) over one 128-wide group, for NR row
// sets sharing the activations.  ap: the lane's activation bytes of the group
// (row, K offset 32 * lsub).
template <int BITS, int NR>
__device__ __forceinline__ void group_mfma(const Word<BITS> *w, const uint8_t *ap, uint32_t magic,
                                           f32x4 *cg) {
#pragma unroll
  for (int r = 0; r < NR; ++r) cg[r] = f32x4{0.f, 0.f, 0.f, 0.f};
  if constexpr (BITS == 6) {  // the slice's 32 codes converted at once, 8 per MFMA
    u32x16 v[NR];
#pragma unroll
    for (int r = 0; r < NR; ++r) v[r] = fp6x32_to_bf16(w[r]);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const bf16x8 a = *(const bf16x8 *)(ap + j * 16);
#pragma unroll
      for (int r = 0; r < NR; ++r) {
        const u32x4 b = u32x4{v[r][4 * j], v[r][4 * j + 1], v[r][4 * j + 2], v[r][4 * j + 3]};
        cg[r] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, __builtin_bit_cast(bf16x8, b), cg[r], 0, 0, 0);
      }
    }
    return;
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const bf16x8 a = *(const bf16x8 *)(ap + j * 16);
#pragma unroll
    for (int r = 0; r < NR; ++r)
      cg[r] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b_op<BITS>(w[r], j, magic), cg[r], 0, 0, 0);
  }
}

// acc += s * (C - (128 + zero) * sum(x)), xs: the group sums of the lane's C rows.
template <bool ONE>
__device__ __forceinline__ void group_acc(f32x4 cg, float s, float zo, const float *xs, f32x4 &acc) {
  if constexpr (ONE) {
    acc[0] = __builtin_fmaf(s, __builtin_fmaf(-zo, xs[0], cg[0]), acc[0]);
  } else {
    const f32x4 v = *(const f32x4 *)xs;
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i] = __builtin_fmaf(s, __builtin_fmaf(-zo, v[i], cg[i]), acc[i]);
  }
}

// The B value of code 0 offset: the unpacked value minus the signed code.
template <int BITS>
__device__ __forceinline__ float zero_off(uint32_t z) {
  if constexpr (BITS == 4)
    return 136.f;  // offset-binary code q + 8, plus the 128 of the unpack
  else if constexpr (BITS == 8)
    return 128.f;  // offset-binary code q + 128, unpacked as is
  else if constexpr (BITS == 6 || BITS == 5)
    return 0.f;    // e2m3 / e2m1 values are signed: no offset
  else
    return 128.f + (float)z;
}

// Groups of 32: a lane's slice of a unit is one whole group, but an MFMA sums
// over the slices of the four lanes 16 r + n.  A 4 x 4 transpose of words
// across those lanes (two swaps of 32-lane halves, two of 16-lane rows) gives
// lane 16 r + n, in v[j], the word lane 16 j + n held in v[r]: afterwards MFMA
// j reads group j only.
__device__ __forceinline__ void transpose4_rows(uint32_t &v0, uint32_t &v1, uint32_t &v2, uint32_t &v3) {
  const auto a = __builtin_amdgcn_permlane32_swap(v0, v2, false, false);
  const auto b = __builtin_amdgcn_permlane32_swap(v1, v3, false, false);
  const auto c = __builtin_amdgcn_permlane16_swap(a[0], b[0], false, false);
  const auto d = __builtin_amdgcn_permlane16_swap(a[1], b[1], false, false);
  v0 = c[0];
  v1 = c[1];
  v2 = d[0];
  v3 = d[1];
}
template <int BITS>
__device__ __forceinline__ void transpose_slices(Word<BITS> &w) {
  if constexpr (BITS == 4) {
    uint32_t v0 = w[0], v1 = w[1], v2 = w[2], v3 = w[3];
    transpose4_rows(v0, v1, v2, v3);
    w = u32x4{v0, v1, v2, v3};
  } else {  // INT8: word pairs, transposed as even and odd words
    uint32_t e0 = w[0], e1 = w[2], e2 = w[4], e3 = w[6], o0 = w[1], o1 = w[3], o2 = w[5], o3 = w[7];
    transpose4_rows(e0, e1, e2, e3);
    transpose4_rows(o0, o1, o2, o3);
    w = u32x8{e0, o0, e1, o1, e2, o2, e3, o3};
  }
}

// One 128-K unit with groups of 32, NR row sets: MFMA j covers group j (A from
// K 32 j + 8 lsub, ap: the unit's activation bytes of the row + 16 lsub), and
// each group's C is corrected with its own scale.  sc[r]: the unit's four bf16
// scales of row set r (two words); xs: Xs of the unit's first group.
template <int BITS, bool ONE, int NR>
__device__ __forceinline__ void unit32_acc(Word<BITS> *w, const uint8_t *ap, const uint32_t (*sc)[2], const float *xs,
                                           uint32_t magic, f32x4 *acc) {
#pragma unroll
  for (int r = 0; r < NR; ++r) transpose_slices<BITS>(w[r]);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const bf16x8 a = *(const bf16x8 *)(ap + j * 64);
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      const f32x4 cg = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b_op<BITS>(w[r], j, magic),
                                                               f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
      const float s = bf16_to_f32((sc[r][j / 2] >> (16 * (j & 1))) & 0xFFFFu);
      group_acc<ONE>(cg, s, zero_off<BITS>(0u), xs + j * 16, acc[r]);
    }
  }
}

// NVFP4: one unit of NR row sets, B = e2m1 * the lane's E4M3 group scale
// (exact in bf16), so acc += C with no correction.  sc[r]: the two scale
// bytes of row set r (K 32 lsub .. +16 and +16 .. +32).
template <int NR>
__device__ __forceinline__ void nv_unit_acc(const u32x4 *w, const uint32_t *sc, const uint8_t *ap, f32x4 *acc) {
  float s0[NR], s1[NR];
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    s0[r] = e4m3_to_f32(sc[r] & 0xFFu);
    s1[r] = e4m3_to_f32((sc[r] >> 8) & 0xFFu);
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const bf16x8 a = *(const bf16x8 *)(ap + j * 16);
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      uint32_t o[4];
      dequant8_e2m1(w[r][j], j < 2 ? s0[r] : s1[r], o);
      acc[r] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, __builtin_bit_cast(bf16x8, u32x4{o[0], o[1], o[2], o[3]}),
                                                       acc[r], 0, 0, 0);
    }
  }
}

// A full chunk (units G0 .. G0+kCG-1) of NR row sets.  ap: activation bytes of
// unit G0 for the lane; xs: Xs of unit G0's first group (+ 4 * lsub unless ONE).
template <int BITS, int GS, bool ONE, int NR>
__device__ __forceinline__ void chunk_gemv(Chunk<BITS, GS> *ch, const uint8_t *ap, const float *xs, uint32_t magic,
                                           f32x4 *acc) {
#pragma unroll
  for (int c = 0; c < kCG<BITS, GS>; ++c) {
    Word<BITS> w[NR];
#pragma unroll
    for (int r = 0; r < NR; ++r) w[r] = ch[r].w[c];
    if constexpr (BITS == 5) {
      uint32_t sc[NR];
#pragma unroll
      for (int r = 0; r < NR; ++r) sc[r] = ch[r].s[c];
      nv_unit_acc<NR>(w, sc, ap + c * (kGroup * 2), acc);
    } else if constexpr (GS == 32) {
      uint32_t sc[NR][2];
#pragma unroll
      for (int r = 0; r < NR; ++r) {
        sc[r][0] = ch[r].s[2 * c];
        sc[r][1] = ch[r].s[2 * c + 1];
      }
      unit32_acc<BITS, ONE, NR>(w, ap + c * (kGroup * 2), sc, xs + c * 64, magic, acc);
    } else {
      f32x4 cg[NR];
      group_mfma<BITS, NR>(w, ap + c * (kGroup * 2), magic, cg);
#pragma unroll
      for (int r = 0; r < NR; ++r) {
        const float s = scale_f32<BITS>((ch[r].s[c / 2] >> (16 * (c & 1))) & 0xFFFFu);
        const float zo = zero_off<BITS>((ch[r].z[c / 4] >> (8 * (c % 4))) & 0xFFu);
        group_acc<ONE>(cg[r], s, zo, xs + c * 16, acc[r]);
      }
    }
  }
}

// One unit at a time (shapes whose units do not split into full chunks),
// NR row sets at offsets o[r].
template <int BITS, int GS, bool ONE, int NR>
__device__ __forceinline__ void groups_gemv_slow(const ExpertW &x, const Off *o, int ng, const uint8_t *ap,
                                                 const float *xs, uint32_t magic, f32x4 *acc) {
  for (int c = 0; c < ng; ++c) {
    Word<BITS> w[NR];
#pragma unroll
    for (int r = 0; r < NR; ++r) w[r] = load_word<BITS>(x.codes + o[r].c + c * kGroupBytes<BITS>);
    if constexpr (BITS == 5) {
      uint32_t sc[NR];
#pragma unroll
      for (int r = 0; r < NR; ++r) sc[r] = *(const uint16_t *)(x.scales + o[r].s + 8 * c);
      nv_unit_acc<NR>(w, sc, ap + c * (kGroup * 2), acc);
    } else if constexpr (GS == 32) {
      uint32_t sc[NR][2];
#pragma unroll
      for (int r = 0; r < NR; ++r) {
        const u32x2 v = *(const u32x2 *)(x.scales + o[r].s + 8 * c);
        sc[r][0] = v[0];
        sc[r][1] = v[1];
      }
      unit32_acc<BITS, ONE, NR>(w, ap + c * (kGroup * 2), sc, xs + c * 64, magic, acc);
    } else {
      f32x4 cg[NR];
      group_mfma<BITS, NR>(w, ap + c * (kGroup * 2), magic, cg);
#pragma unroll
      for (int r = 0; r < NR; ++r) {
        const float s = scale_f32<BITS>(*(const uint16_t *)(x.scales + o[r].s + 2 * c));
        const float zo = zero_off<BITS>(BITS == 2 ? x.zeros[o[r].z + c] : 0u);
        group_acc<ONE>(cg[r], s, zo, xs + c * 16, acc[r]);
      }
    }
  }
}

__device__ __forceinline__ float silu_f(float v) { return v / (1.f + __expf(-v)); }

}  // namespace
}  // namespace bqmoe
