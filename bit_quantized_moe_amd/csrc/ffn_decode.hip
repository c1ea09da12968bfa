// Decode-path expert FFN (T <= 16 tokens): one fused kernel that streams each
// selected expert's packed weights from HBM exactly once.
//
// The pages locate the decode cost in the expert GEMV that reads each selected
// expert in place (page "Qwen3.8-Flash-Next on one 24 GB GPU", "What the
// patch does": an N-contiguous batch-1 GEMV measured at 320 GB/s in-kernel;
// page "Qwen3.8-Flash-Next FP6-INT8", "Step budget and hardware floors": the
// expert GEMV is about 6 ms of each added decode stream) and dispatch to a GEMV
// up to 16 rows (same page, "Quantization quality").  This kernel is a
// from-scratch gfx950 design on the canonical K-packed layout:
//
//  * Phase 1 (gate_up + SwiGLU): a wave owns a contiguous run of items; an
//    item is a (gate row i, up row I+i) pair of one expert.  Each lane reads
//    whole 16-byte chunks of packed codes (global_load_dwordx4), dots them
//    against bf16 activation pairs with v_dot2_f32_bf16, and a reduction over
//    the row's lanes gives the row result; h = silu(gate) * up goes to the
//    workspace as bf16.  The weights of the next item are in flight while the
//    current one is computed.
//  * Phase 2 (down): a wave owns a contiguous run of down rows.  Their weight
//    chunks are requested as soon as the wave's phase-1 loads are out; before
//    using h of an expert the wave waits until every phase-1 item of that
//    expert is published.
//
// Hand-off without cache flushes: h is written with device-coherent stores
// (sc1), the writer waits for them to complete (vmcnt(0)) and then bumps the
// expert's counter with a device-scope atomic; a reader polls the counter and
// reads h with device-coherent loads.  Counters sit on separate 128-byte lines.
// The grid never exceeds the co-resident block count and every wave finishes
// its phase-1 items before it waits, so every wait ends; the waits are bounded
// anyway and a timeout only raises an error flag.
//
// Unpack: OR-ing a code field u into the mantissa of bf16 128.0 gives exactly
// 128 + u.  With activations arranged in the same (field i, field i + P/2)
// pairs, sum((128 + u) x) - (128 + zero) * sum(x) = sum((u - zero) x), times
// the group scale (zero = 8 for INT4 offset-binary codes).
#include <mutex>

#include "common.cuh"
#include "internal.h"

namespace bqmoe {
namespace {

struct DecodeParams {
  const uint16_t *x;
  const int32_t *offsets;
  const int32_t *sorted_rows;
  const int32_t *active;
  int T, k, E, H, I, Amax;
  const uint32_t *w13c;
  const uint16_t *w13s;
  const uint8_t *w13z;
  const uint32_t *w2c;
  const uint16_t *w2s;
  const uint8_t *w2z;
  uint16_t *y_perm;
  uint16_t *hbuf;  // [T*k, I] bf16
  int *ctl;
  int lpr1, rpw1, items1;  // phase 1: lanes per row, rows per wave pass, items per expert
  int lpr2, rpw2, items2;  // phase 2
  int max_spins;
  uint32_t magic;          // bf16 pair (128.0, 128.0); an argument so it sits in an SGPR
};

__device__ __forceinline__ int *counter(int *ctl, int a) { return ctl + kCtlCounters + a * kCtrStride; }

// bf16 activations of one 16-byte weight chunk, arranged as the unpack pairs.
// INT4 chunk = 32 K (4 words); INT2 chunk = 64 K (4 words).
template <int BITS>
struct ActChunk {
  static constexpr int NP = (BITS == 4) ? 16 : 32;  // packed bf16 pairs
  uint32_t p[NP];
  float sum;
};

template <int BITS>
__device__ __forceinline__ void arrange_act(const uint32_t *d, ActChunk<BITS> &a) {
  constexpr int ND = ActChunk<BITS>::NP;
  if constexpr (BITS == 4) {
    // word j covers 8 K: dwords (x0,x1)(x2,x3)(x4,x5)(x6,x7) -> pairs (x_i, x_{i+4})
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      a.p[4 * j + 0] = __builtin_amdgcn_perm(d[4 * j + 2], d[4 * j + 0], 0x05040100u);
      a.p[4 * j + 1] = __builtin_amdgcn_perm(d[4 * j + 2], d[4 * j + 0], 0x07060302u);
      a.p[4 * j + 2] = __builtin_amdgcn_perm(d[4 * j + 3], d[4 * j + 1], 0x05040100u);
      a.p[4 * j + 3] = __builtin_amdgcn_perm(d[4 * j + 3], d[4 * j + 1], 0x07060302u);
    }
  } else {
    // word j covers 16 K: dwords d[8j..8j+7] -> pairs (x_i, x_{i+8})
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint32_t lo = d[8 * j + i / 2], hi = d[8 * j + 4 + i / 2];
        a.p[8 * j + i] = (i & 1) ? __builtin_amdgcn_perm(hi, lo, 0x07060302u)
                                 : __builtin_amdgcn_perm(hi, lo, 0x05040100u);
      }
  }
  float s = 0.f;
#pragma unroll
  for (int q = 0; q < ND; ++q) s = dot2_bf16(d[q], 0x3F803F80u, s);  // sum of the chunk's activations
  a.sum = s;
}

// activations from ordinary memory (x)
template <int BITS>
__device__ __forceinline__ void load_act(const uint16_t *src, ActChunk<BITS> &a) {
  constexpr int ND = ActChunk<BITS>::NP;
  uint32_t d[ND];
#pragma unroll
  for (int q = 0; q < ND / 4; ++q) {
    const u32x4 v = *(const u32x4 *)(src + 8 * q);
    d[4 * q + 0] = v[0];
    d[4 * q + 1] = v[1];
    d[4 * q + 2] = v[2];
    d[4 * q + 3] = v[3];
  }
  arrange_act<BITS>(d, a);
}

// activations written by other blocks during this kernel (h): device-coherent loads
template <int BITS>
__device__ __forceinline__ void load_act_coherent(const uint16_t *src, ActChunk<BITS> &a) {
  constexpr int ND = ActChunk<BITS>::NP;
  uint32_t d[ND];
  const uint32_t *s32 = (const uint32_t *)src;
#pragma unroll
  for (int q = 0; q < ND; ++q) d[q] = __hip_atomic_load(s32 + q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  arrange_act<BITS>(d, a);
}

// sum over one chunk of (128 + u) * act
template <int BITS>
__device__ __forceinline__ float chunk_dot(const u32x4 &w, const ActChunk<BITS> &a, uint32_t mask, uint32_t magic) {
  float acc = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t v = w[j];
    if constexpr (BITS == 4) {
      const uint32_t v4 = v >> 4;
      acc = dot2_bf16(and_or_b32(v, mask, magic), a.p[4 * j + 0], acc);
      acc = dot2_bf16(and_or_b32(v4, mask, magic), a.p[4 * j + 1], acc);
      acc = dot2_bf16(and_or_b32(v >> 8, mask, magic), a.p[4 * j + 2], acc);
      acc = dot2_bf16(and_or_b32(v4 >> 8, mask, magic), a.p[4 * j + 3], acc);
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) acc = dot2_bf16(and_or_b32(v >> (2 * i), mask, magic), a.p[8 * j + i], acc);
    }
  }
  return acc;
}

__device__ __forceinline__ float silu_f(float v) { return v / (1.f + __expf(-v)); }

// One row's packed chunks for one lane, with scale and (2-bit) zero-point.
template <int BITS, int MC>
struct RowChunks {
  u32x4 w[MC];
  float s[MC];
  float z[BITS == 2 ? MC : 1];  // 128 + zero-point (2-bit only; INT4 uses 136)
};

// lane-relative pointers of one weight row: codes at chunk lr (+c*lpr), scales at its groups
template <int BITS, int MC>
__device__ __forceinline__ void load_row(const uint32_t *codes_row, const uint16_t *scales_row,
                                         const uint8_t *zeros_row, int lr, int lpr, RowChunks<BITS, MC> &rc) {
  constexpr int KPC = 128 / BITS;  // K values per 16-byte chunk
#pragma unroll
  for (int c = 0; c < MC; ++c) {
    const int ch = lr + c * lpr;
    rc.w[c] = *(const u32x4 *)(codes_row + ch * 4);
    const int g = ch * KPC / kGroup;
    rc.s[c] = bf16_to_f32(scales_row[g]);
    if constexpr (BITS == 2) rc.z[c] = 128.f + (float)zeros_row[g];
  }
}

template <int BITS, int MC>
__device__ __forceinline__ float row_partial(const RowChunks<BITS, MC> &rc, const ActChunk<BITS> *act, uint32_t mask,
                                             uint32_t magic) {
  float tot = 0.f;
#pragma unroll
  for (int c = 0; c < MC; ++c) {
    const float raw = chunk_dot<BITS>(rc.w[c], act[c], mask, magic);
    const float z = (BITS == 4) ? 136.f : rc.z[BITS == 2 ? c : 0];
    tot += rc.s[c] * __builtin_fmaf(-z, act[c].sum, raw);
  }
  return tot;
}

// Per-expert metadata of active slot a, reloaded (through the scalar cache)
// only when the slot changes.
struct Meta {
  int a = -1, e = 0, o0 = 0, o1 = 0;
  __device__ __forceinline__ void get(const DecodeParams &p, int slot, int nrows) {
    if (slot == a) return;
    a = slot;
    e = min(max(sload(p.active + 1 + slot), 0), p.E - 1);
    o0 = min(max(sload(p.offsets + e), 0), nrows);
    o1 = min(max(sload(p.offsets + e + 1), o0), nrows);
  }
};

// Position (active slot, item within the expert) of a contiguous item run.
struct Cursor {
  int a, ib;
  __device__ __forceinline__ void advance(int items) {
    if (++ib == items) {
      ib = 0;
      ++a;
    }
  }
};

template <int BITS, int MC>
struct PairBuf {
  RowChunks<BITS, MC> g, u;
};

template <int BITS, int MC1, int MC2, bool ONE>
struct Depth {
  static constexpr int NTR = ONE ? 1 : 2;  // routed rows of one expert whose activations stay in registers
  static constexpr int NB2 = 4;            // phase-2 items per load batch (two batches in flight)
};

// ONE: T == 1 (each expert has exactly one routed row, token 0)
template <int BITS, int MC1, int MC2, bool ONE>
__global__ void __launch_bounds__(256, 2) ffn_decode_kernel(DecodeParams p) {
  constexpr int KPC = 128 / BITS;
  constexpr int NTR = Depth<BITS, MC1, MC2, ONE>::NTR;
  constexpr int NB2 = Depth<BITS, MC1, MC2, ONE>::NB2;
  const uint32_t magic = p.magic;
  const uint32_t mask = (BITS == 4) ? 0x000F000Fu : 0x00030003u;
  const int lane = lane_id();
  const int gw = blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int W = gridDim.x * 4;
  // With one token every active slot holds one of its k distinct experts, so
  // the partition can use the host-known Amax (= k) without first reading A.
  const int A = ONE ? p.Amax : min(max(sload(p.active), 0), p.Amax);
  const int nrows = p.T * p.k;

  const int rs1 = lane / p.lpr1, lr1 = lane % p.lpr1;
  const int rs2 = lane / p.lpr2, lr2 = lane % p.lpr2;
  const int wpr1 = p.H * BITS / 32, gpr1 = p.H / kGroup;
  const int wpr2 = p.I * BITS / 32, gpr2 = p.I / kGroup;
  const int total1 = A * p.items1, total2 = A * p.items2;
  const int per1 = (total1 + W - 1) / W, per2 = (total2 + W - 1) / W;
  const int it1_0 = min(total1, gw * per1), it1_1 = min(total1, it1_0 + per1);
  const int it2_0 = min(total2, gw * per2), it2_1 = min(total2, it2_0 + per2);

  // ---------------------------------------------------------------- phase-2 loads
  RowChunks<BITS, MC2> dwA[NB2], dwB[NB2];
  Cursor c2l{it2_0 / max(p.items2, 1), it2_0 % max(p.items2, 1)};
  Meta m2l;
  int it2_loaded = it2_0;
  auto load2 = [&](RowChunks<BITS, MC2>(&dw)[NB2]) {
#pragma unroll
    for (int j = 0; j < NB2; ++j) {
      if (it2_loaded < it2_1) {
        m2l.get(p, c2l.a, nrows);
        const size_t row = (size_t)m2l.e * p.H + c2l.ib * p.rpw2 + rs2;
        load_row<BITS, MC2>(p.w2c + row * wpr2, p.w2s + row * gpr2, BITS == 2 ? p.w2z + row * gpr2 : nullptr,
                            lr2, p.lpr2, dw[j]);
        c2l.advance(p.items2);
        ++it2_loaded;
      }
    }
  };

  // ---------------------------------------------------------------- phase 1
  // activations of the routed rows of the current expert (one token: loaded first)
  ActChunk<BITS> xa[NTR][MC1];
  Meta m1c;
  int x_for = -1;
  if constexpr (ONE) {
#pragma unroll
    for (int c = 0; c < MC1; ++c) load_act<BITS>(p.x + (lr1 + c * p.lpr1) * KPC, xa[0][c]);
  }

  Cursor c1l{it1_0 / max(p.items1, 1), it1_0 % max(p.items1, 1)};
  Cursor c1c = c1l;
  Meta m1l;
  auto load1 = [&](PairBuf<BITS, MC1> &b) {
    m1l.get(p, c1l.a, nrows);
    const size_t row = (size_t)m1l.e * 2 * p.I + c1l.ib * p.rpw1 + rs1;
    load_row<BITS, MC1>(p.w13c + row * wpr1, p.w13s + row * gpr1, BITS == 2 ? p.w13z + row * gpr1 : nullptr, lr1,
                        p.lpr1, b.g);
    const size_t rowu = row + p.I;
    load_row<BITS, MC1>(p.w13c + rowu * wpr1, p.w13s + rowu * gpr1, BITS == 2 ? p.w13z + rowu * gpr1 : nullptr,
                        lr1, p.lpr1, b.u);
    c1l.advance(p.items1);
  };

  int cur_a = -1, done_in_a = 0;
  auto publish = [&]() {
    if (done_in_a) {
      wait_vmem();
      if (lane == 0) atomicAdd(counter(p.ctl, cur_a), done_in_a);
    }
  };
  auto compute1 = [&](const PairBuf<BITS, MC1> &b) {
    const int a = c1c.a;
    const int i = c1c.ib * p.rpw1 + rs1;
    if (a != cur_a) {
      publish();
      cur_a = a;
      done_in_a = 0;
    }
    m1c.get(p, a, nrows);
    if constexpr (ONE) {
      const float gv = group_sum(row_partial<BITS, MC1>(b.g, xa[0], mask, magic), p.lpr1);
      const float uv = group_sum(row_partial<BITS, MC1>(b.u, xa[0], mask, magic), p.lpr1);
      if (lr1 == 0 && m1c.o1 > m1c.o0)
        __hip_atomic_store(p.hbuf + (size_t)m1c.o0 * p.I + i, f32_to_bf16(silu_f(gv) * uv), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    } else {
      if (x_for != a) {
        x_for = a;
#pragma unroll
        for (int r = 0; r < NTR; ++r)
          if (m1c.o0 + r < m1c.o1) {
            const int t = min(max(sload(p.sorted_rows + m1c.o0 + r), 0) / p.k, p.T - 1);
#pragma unroll
            for (int c = 0; c < MC1; ++c) load_act<BITS>(p.x + (size_t)t * p.H + (lr1 + c * p.lpr1) * KPC, xa[r][c]);
          }
      }
#pragma unroll
      for (int r = 0; r < NTR; ++r)
        if (m1c.o0 + r < m1c.o1) {
          const float gv = group_sum(row_partial<BITS, MC1>(b.g, xa[r], mask, magic), p.lpr1);
          const float uv = group_sum(row_partial<BITS, MC1>(b.u, xa[r], mask, magic), p.lpr1);
          if (lr1 == 0)
            __hip_atomic_store(p.hbuf + (size_t)(m1c.o0 + r) * p.I + i, f32_to_bf16(silu_f(gv) * uv),
                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
      for (int q = m1c.o0 + NTR; q < m1c.o1; ++q) {  // more routed rows than are cached
        const int t = min(max(sload(p.sorted_rows + q), 0) / p.k, p.T - 1);
        ActChunk<BITS> act[MC1];
#pragma unroll
        for (int c = 0; c < MC1; ++c) load_act<BITS>(p.x + (size_t)t * p.H + (lr1 + c * p.lpr1) * KPC, act[c]);
        const float gv = group_sum(row_partial<BITS, MC1>(b.g, act, mask, magic), p.lpr1);
        const float uv = group_sum(row_partial<BITS, MC1>(b.u, act, mask, magic), p.lpr1);
        if (lr1 == 0)
          __hip_atomic_store(p.hbuf + (size_t)q * p.I + i, f32_to_bf16(silu_f(gv) * uv), __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
      }
    }
    ++done_in_a;
    c1c.advance(p.items1);
  };

  // one item ahead: the loads of item j+1 are issued before item j is computed;
  // after the wave's last phase-1 load its first two phase-2 batches follow.
  PairBuf<BITS, MC1> bA, bB;
  bool p2_issued = false;
  auto issue_p2 = [&]() {
    if (!p2_issued) {
      load2(dwA);
      load2(dwB);
      p2_issued = true;
    }
  };
  if (it1_0 < it1_1) load1(bA);
  for (int it = it1_0; it < it1_1; it += 2) {
    if (it + 1 < it1_1) load1(bB); else issue_p2();
    compute1(bA);
    if (it + 1 < it1_1) {
      if (it + 2 < it1_1) load1(bA); else issue_p2();
      compute1(bB);
    }
  }
  issue_p2();
  publish();

  // ---------------------------------------------------------------- phase 2
  Cursor c2c{it2_0 / max(p.items2, 1), it2_0 % max(p.items2, 1)};
  Meta m2c;
  int ready_a = -1;
  ActChunk<BITS> hc[NTR][MC2];
  auto compute2 = [&](const RowChunks<BITS, MC2> &d) {
    const int a = c2c.a;
    const int n = c2c.ib * p.rpw2 + rs2;
    m2c.get(p, a, nrows);
    if (a != ready_a) {
      int ok = 1;
      if (lane == 0) ok = wait_counter_geq(counter(p.ctl, a), p.items1, p.max_spins) ? 1 : 0;
      ok = __shfl(ok, 0, kWave);
      if (!ok && lane == 0) atomicOr(&p.ctl[kCtlError], 1);
      ready_a = a;
#pragma unroll
      for (int r = 0; r < NTR; ++r)
        if (m2c.o0 + r < m2c.o1)
#pragma unroll
          for (int c = 0; c < MC2; ++c)
            load_act_coherent<BITS>(p.hbuf + (size_t)(m2c.o0 + r) * p.I + (lr2 + c * p.lpr2) * KPC, hc[r][c]);
    }
#pragma unroll
    for (int r = 0; r < NTR; ++r)
      if (m2c.o0 + r < m2c.o1) {
        const float yv = group_sum(row_partial<BITS, MC2>(d, hc[r], mask, magic), p.lpr2);
        if (lr2 == 0) p.y_perm[(size_t)(m2c.o0 + r) * p.H + n] = f32_to_bf16(yv);
      }
    if constexpr (!ONE) {
      for (int q = m2c.o0 + NTR; q < m2c.o1; ++q) {  // more routed rows than are cached
        ActChunk<BITS> act[MC2];
#pragma unroll
        for (int c = 0; c < MC2; ++c)
          load_act_coherent<BITS>(p.hbuf + (size_t)q * p.I + (lr2 + c * p.lpr2) * KPC, act[c]);
        const float yv = group_sum(row_partial<BITS, MC2>(d, act, mask, magic), p.lpr2);
        if (lr2 == 0) p.y_perm[(size_t)q * p.H + n] = f32_to_bf16(yv);
      }
    }
    c2c.advance(p.items2);
  };
  for (int base = it2_0; base < it2_1; base += 2 * NB2) {
#pragma unroll
    for (int j = 0; j < NB2; ++j)
      if (base + j < it2_1) compute2(dwA[j]);
    if (base + 2 * NB2 < it2_1) load2(dwA);
#pragma unroll
    for (int j = 0; j < NB2; ++j)
      if (base + NB2 + j < it2_1) compute2(dwB[j]);
    if (base + 3 * NB2 < it2_1) load2(dwB);
  }

  // ---------------------------------------------------------------- counters reset
  // The last block to finish re-zeroes the counters (no cache flush needed:
  // every block has finished polling before it is counted).
  __shared__ int s_last;
  __syncthreads();
  if (threadIdx.x == 0) {
    const int prev = atomicAdd(&p.ctl[kCtlFfnDone], 1);
    s_last = (prev == (int)gridDim.x - 1);
  }
  __syncthreads();
  if (s_last) {
    for (int a = threadIdx.x; a < p.Amax; a += blockDim.x)
      __hip_atomic_store(counter(p.ctl, a), 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (threadIdx.x == 0) __hip_atomic_store(&p.ctl[kCtlFfnDone], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

struct Layout {
  int lpr, cpl, rpw;
};

Layout row_layout(int K, int bits) {
  const int chunks = K * bits / 128;  // 16-byte chunks per row
  Layout l;
  l.lpr = chunks < kWave ? chunks : kWave;
  l.cpl = chunks / l.lpr;
  l.rpw = kWave / l.lpr;
  return l;
}

template <int BITS, bool ONE>
const void *decode_fn_mc(int mc1, int mc2) {
  if (mc2 == 1) {
    if (mc1 == 1) return (const void *)ffn_decode_kernel<BITS, 1, 1, ONE>;
    if (mc1 == 2) return (const void *)ffn_decode_kernel<BITS, 2, 1, ONE>;
    if (mc1 == 4) return (const void *)ffn_decode_kernel<BITS, 4, 1, ONE>;
  } else if (mc2 == 2) {
    if (mc1 == 1) return (const void *)ffn_decode_kernel<BITS, 1, 2, ONE>;
    if (mc1 == 2) return (const void *)ffn_decode_kernel<BITS, 2, 2, ONE>;
    if (mc1 == 4) return (const void *)ffn_decode_kernel<BITS, 4, 2, ONE>;
  }
  return nullptr;
}

const void *decode_kernel_fn(int bits, int mc1, int mc2, bool one) {
  if (bits == 4) return one ? decode_fn_mc<4, true>(mc1, mc2) : decode_fn_mc<4, false>(mc1, mc2);
  return one ? decode_fn_mc<2, true>(mc1, mc2) : decode_fn_mc<2, false>(mc1, mc2);
}

// Co-resident blocks per CU of one decode instantiation (cached per device and kernel).
int resident_blocks_per_cu(const void *fn, int device) {
  static std::mutex mu;
  static const void *c_fn[64];
  static int c_dev[64], c_nb[64], n_cached = 0;
  std::lock_guard<std::mutex> lk(mu);
  for (int i = 0; i < n_cached; ++i)
    if (c_fn[i] == fn && c_dev[i] == device) return c_nb[i];
  int nb = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, fn, 256, 0) != hipSuccess) return 0;
  if (n_cached < 64) {
    c_fn[n_cached] = fn;
    c_dev[n_cached] = device;
    c_nb[n_cached] = nb;
    ++n_cached;
  }
  return nb;
}

}  // namespace

bool decode_layout_ok(int H, int I, int bits) {
  const Layout a = row_layout(H, bits), b = row_layout(I, bits);
  const int ca = H * bits / 128, cb = I * bits / 128;
  auto pow2 = [](int v) { return v > 0 && (v & (v - 1)) == 0; };
  return (a.cpl == 1 || a.cpl == 2 || a.cpl == 4) && (b.cpl == 1 || b.cpl == 2) && ca % a.lpr == 0 &&
         cb % b.lpr == 0 && pow2(a.lpr) && pow2(b.lpr) && I % a.rpw == 0 && H % b.rpw == 0;
}

size_t ffn_ctl_bytes(int T, int k, int E) {
  const long amax = E < (long)T * k ? E : (long)T * k;
  size_t b = (size_t)(kCtlCounters + amax * kCtrStride) * 4;
  if (b < kCtlBytes) b = kCtlBytes;
  return (b + 255) / 256 * 256;
}

hipError_t launch_ffn_decode(const FfnArgs &a, const DeviceInfo &dev, hipStream_t st) {
  DecodeParams p;
  p.x = a.x;
  p.offsets = a.offsets;
  p.sorted_rows = a.sorted_rows;
  p.active = a.active;
  p.T = a.T;
  p.k = a.k;
  p.E = a.E;
  p.H = a.H;
  p.I = a.I;
  p.Amax = a.E < a.T * a.k ? a.E : a.T * a.k;
  p.w13c = a.w13_codes;
  p.w13s = a.w13_scales;
  p.w13z = a.w13_zeros;
  p.w2c = a.w2_codes;
  p.w2s = a.w2_scales;
  p.w2z = a.w2_zeros;
  p.y_perm = a.y_perm;
  p.ctl = (int *)a.ws;
  p.hbuf = (uint16_t *)((char *)a.ws + ffn_ctl_bytes(a.T, a.k, a.E));
  const Layout l1 = row_layout(a.H, a.bits), l2 = row_layout(a.I, a.bits);
  p.lpr1 = l1.lpr;
  p.rpw1 = l1.rpw;
  p.items1 = a.I / l1.rpw;
  p.lpr2 = l2.lpr;
  p.rpw2 = l2.rpw;
  p.items2 = a.H / l2.rpw;
  p.max_spins = 1 << 22;
  p.magic = 0x43004300u;
  const void *fn = decode_kernel_fn(a.bits, l1.cpl, l2.cpl, a.T == 1);
  if (!fn) return hipErrorInvalidConfiguration;
  const int per_cu = resident_blocks_per_cu(fn, dev.device);
  if (per_cu < 1) return hipErrorInvalidConfiguration;
  const long waves_needed = (long)p.Amax * (p.items1 > p.items2 ? p.items1 : p.items2);
  long blocks = (waves_needed + 3) / 4;
  const long resident = (long)dev.num_cus * per_cu;
  if (blocks > resident) blocks = resident;
  if (blocks < 1) blocks = 1;
  void *args[] = {&p};
  return hipLaunchKernel(fn, dim3((unsigned)blocks), dim3(256), args, 0, st);
}

}  // namespace bqmoe
