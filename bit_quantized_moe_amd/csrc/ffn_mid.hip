// Middle-batch expert FFN: a few to a few dozen routed rows per expert (about
// T = 256 to 768 tokens at E = 256, top-8), where the decode kernel would
// stream each expert's weights once per four rows and the grouped GEMMs spend
// more time dequantising a tile of weights than multiplying it.
//
// The pages route each token to its top-k experts and run every selected
// expert's gate_up -> SwiGLU -> down on its rows, reading only the selected
// experts (page "Qwen3.8-Flash-Next on one 24 GB GPU", "What the patch does";
// page "Qwen3.8-Flash-Next FP6-INT8", "Quantization quality": a GEMV for up to
// 16 rows, a GEMM above).  This is the same computation, the batch between
// those two regimes, as two launches:
//
//  * gate_up (mid_kernel<BITS, true>): block (active slot a, tile of 64 h
//    columns); wave w owns gate rows c, up rows I + c for its 16 columns c, so
//    SwiGLU needs no exchange between waves; h = silu(g) * u goes to the
//    workspace in bf16, rows in sorted order;
//  * down (mid_kernel<BITS, false>): block (a, tile of 128 output columns),
//    wave w owns 32 down rows, y_perm rows in sorted order.
//
// Per block, K advances in steps of two 128-K units.  Every step the block
// stages the expert's routed rows (up to 32 per pass) for those 256 K in LDS,
// in the K order the unpacked codes come out in, with their per-unit sums;
// each wave holds the step's packed weights of its two 16-row sets in
// registers (requested one step ahead) and runs v_mfma_f32_16x16x32_bf16 with
// one or two 16-row A tiles (by the pass's row count) against them.  Weights are read once per pass and
// unpacked once per step (the offset-bf16 codes 128 + u, exact), and each
// unit's C is corrected as s * (C - (128 + zero) * sum(x)) before it is
// added in float32.  An expert with more than 32 rows takes further passes.
#include "common.cuh"
#include "gemv_ops.cuh"
#include "internal.h"

namespace bqmoe {
namespace {

constexpr int kMidWaves = 4;
constexpr int kMidUnits = 2;                 // 128-K units per step (2 measured faster than 4: 3 blocks per CU)
constexpr int kMidStepK = kMidUnits * kGroup;
constexpr int kMidRows = 32;                 // routed rows per pass: two 16-row M tiles
constexpr int kMidPitch = kMidStepK * 2 + 16;  // LDS bytes per staged row (16 rows hit 16 distinct bank quads)

struct MidParams {
  const uint16_t *a;    // gate_up: x [T, H]; down: h [T*k, I] in sorted order
  const int32_t *offsets, *sorted_rows, *active;
  int T, k, E, I, H;
  int K;                // reduction length (H or I)
  int n_rows_w;         // weight rows per expert (2I or H)
  int n_tiles;          // column tiles per expert
  const uint8_t *codes, *scales, *zeros;  // stacked expert arrays
  const uint64_t *tab;  // per-expert address table or null; this GEMM's entries start at tab_off
  int tab_off;
  uint16_t *out;        // gate_up: h [T*k, I]; down: y_perm [T*k, H]
  int max_rows;         // experts with more rows are left to the grouped GEMMs (prefill hybrid)
  uint32_t magic;       // 0x43434343 (the bf16 high byte of 128)
};

// One step of a wave's weights: kMidUnits units of its two row sets.
template <int BITS>
struct MidW {
  Word<BITS> w[2][kMidUnits];
  uint32_t s[2][kMidUnits / 2];  // bf16 scales, two per word (unit u: word u / 2, half u & 1)
  uint32_t z[2];                 // 2-bit: the zero-point bytes of the step's units (low kMidUnits bytes)
};

template <int BITS>
__device__ __forceinline__ void mid_load(const ExpertW &x, const Off (&o)[2], int u0, MidW<BITS> &b) {
  constexpr int GB = kGroupBytes<BITS>;
#pragma unroll
  for (int r = 0; r < 2; ++r) {
#pragma unroll
    for (int u = 0; u < kMidUnits; ++u) b.w[r][u] = load_word<BITS>(x.codes + o[r].c + (u0 + u) * GB);
    b.s[r][0] = *(const uint32_t *)(x.scales + o[r].s + 2 * u0);
    if constexpr (BITS == 2) b.z[r] = *(const uint16_t *)(x.zeros + o[r].z + u0);
  }
}

// Activation chunks of one step a thread stages: the pass's rows x the
// step's K in chunks of kChunkE elements, chunk c = threadIdx.x + 256 i.
template <int BITS>
constexpr int kMidChunks = kMidRows * (kMidStepK / kChunkE<BITS>) / (kMidWaves * kWave);
template <int BITS>
struct MidA {
  uint32_t d[kMidChunks<BITS>][kChunkE<BITS> / 2];
};

// Element offsets (from p.a) of the source rows of a thread's chunks in the
// pass starting at sorted position q0: x of the row's token, or h in sorted
// order; rows past R keep offset 0 and are never loaded.
template <int BITS, bool G1>
__device__ __forceinline__ void mid_rows(const MidParams &p, int q0, int R, uint32_t (&off)[kMidChunks<BITS>]) {
  constexpr int CPR = kMidStepK / kChunkE<BITS>;  // chunks per staged row
#pragma unroll
  for (int i = 0; i < kMidChunks<BITS>; ++i) {
    const int r = (threadIdx.x + kMidWaves * kWave * i) / CPR;
    off[i] = 0;
    if (r < R) {
      if constexpr (G1)
        off[i] = (uint32_t)(min(max(p.sorted_rows[q0 + r], 0) / p.k, p.T - 1) * p.K);
      else
        off[i] = (uint32_t)((q0 + r) * p.K);
    }
  }
}

template <int BITS>
__device__ __forceinline__ void mid_fetch_a(const uint16_t *src, const uint32_t (&off)[kMidChunks<BITS>], int R,
                                            int k0, MidA<BITS> &a) {
  constexpr int CPR = kMidStepK / kChunkE<BITS>;
#pragma unroll
  for (int i = 0; i < kMidChunks<BITS>; ++i) {
    const int c = threadIdx.x + kMidWaves * kWave * i, r = c / CPR, q = c % CPR;
    if (r < R) load_act_chunk<BITS>(src + off[i] + k0, q, a.d[i]);
  }
}

// Stores a thread's chunks to LDS in operand order and the per-unit sums of
// the staged rows to Xs[u * 32 + r]: the lanes holding one unit of one row
// (128 / kChunkE consecutive lanes) add their chunks' sums.  Rows past R get
// sums of stale registers; their C rows are never stored.
template <int BITS>
__device__ __forceinline__ void mid_store_a(uint8_t *act, float *Xs, int R, const MidA<BITS> &a) {
  constexpr int CE = kChunkE<BITS>, CPR = kMidStepK / CE, CPU = kGroup / CE;
#pragma unroll
  for (int i = 0; i < kMidChunks<BITS>; ++i) {
    const int c = threadIdx.x + kMidWaves * kWave * i, r = c / CPR, q = c % CPR;
    if (r < R) store_act_chunk<BITS>(act + r * kMidPitch, q, a.d[i]);
    float sum = 0.f;
#pragma unroll
    for (int z = 0; z < CE / 2; ++z) sum = dot2_bf16(a.d[i][z], 0x3F803F80u, sum);
    sum = group_sum(sum, CPU);
    if (q % CPU == 0) Xs[(q / CPU) * kMidRows + r] = sum;
  }
}

// The step's MFMAs: unit u, operand j unpacked once for both row sets and
// used by each of the MT row tiles; every unit's C then corrected into acc.
template <int BITS, int MT>
__device__ __forceinline__ void mid_step(const MidW<BITS> &b, const uint8_t *act, const float *Xs, int R,
                                         uint32_t magic, f32x4 (&acc)[2][2]) {
  const int lane = lane_id(), m = lane % 16, lsub = lane / 16;
#pragma unroll
  for (int u = 0; u < kMidUnits; ++u) {
    f32x4 cg[2][MT];
#pragma unroll
    for (int r = 0; r < 2; ++r)
#pragma unroll
      for (int t = 0; t < MT; ++t) cg[r][t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const bf16x8 b0 = b_op<BITS>(b.w[0][u], j, magic), b1 = b_op<BITS>(b.w[1][u], j, magic);
#pragma unroll
      for (int t = 0; t < MT; ++t) {
        const int arow = min(t * 16 + m, R - 1);
        const bf16x8 av = *(const bf16x8 *)(act + arow * kMidPitch + u * (kGroup * 2) + lsub * 64 + j * 16);
        cg[0][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, b0, cg[0][t], 0, 0, 0);
        cg[1][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, b1, cg[1][t], 0, 0, 0);
      }
    }
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const float s = scale_f32<BITS>((b.s[r][u / 2] >> (16 * (u & 1))) & 0xFFFFu);
      const float zo = zero_off<BITS>((b.z[r] >> (8 * u)) & 0xFFu);
#pragma unroll
      for (int t = 0; t < MT; ++t) group_acc<false>(cg[r][t], s, zo, Xs + u * kMidRows + t * 16 + 4 * lsub, acc[r][t]);
    }
  }
}

// One pass over the expert's weights for the R <= 32 rows at sorted positions
// q0 .. q0 + R - 1, with MT 16-row tiles (MT = 1 while R <= 16).
template <int BITS, bool G1, int MT>
__device__ __forceinline__ void mid_pass(const MidParams &p, const ExpertW &xw, const Off (&o)[2], int c0, int q0,
                                         int R, int steps, uint8_t *act, float *Xs) {
  const int lane = lane_id(), m = lane % 16, lsub = lane / 16;
  uint32_t roff[kMidChunks<BITS>];
  mid_rows<BITS, G1>(p, q0, R, roff);
  MidW<BITS> wcur, wnext;
  MidA<BITS> an;
  mid_load<BITS>(xw, o, 0, wcur);
  mid_fetch_a<BITS>(p.a, roff, R, 0, an);
  f32x4 acc[2][2];
#pragma unroll
  for (int r = 0; r < 2; ++r)
#pragma unroll
    for (int t = 0; t < 2; ++t) acc[r][t] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int s = 0; s < steps; ++s) {
    // stage this step's rows (fetched during the previous step) and their sums
    __syncthreads();
    mid_store_a<BITS>(act, Xs, R, an);
    __syncthreads();
    // next step's weights and rows in flight during this step's MFMAs
    if (s + 1 < steps) {
      mid_load<BITS>(xw, o, (s + 1) * kMidUnits, wnext);
      mid_fetch_a<BITS>(p.a, roff, R, (s + 1) * kMidStepK, an);
    }
    mid_step<BITS, MT>(wcur, act, Xs, R, p.magic, acc);
    wcur = wnext;
  }
  // epilogue: C row 4 lsub + i of tile t is staged row 16 t + 4 lsub + i, column m
#pragma unroll
  for (int t = 0; t < MT; ++t)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int rr = t * 16 + 4 * lsub + i;
      if (rr >= R) continue;
      const size_t q = (size_t)(q0 + rr);
      if constexpr (G1) {
        const float g = acc[0][t][i], u = acc[1][t][i];
        p.out[q * p.I + c0 + m] = f32_to_bf16(silu_f(g) * u);
      } else {
        p.out[q * p.H + c0 + m] = f32_to_bf16(acc[0][t][i]);
        p.out[q * p.H + c0 + 16 + m] = f32_to_bf16(acc[1][t][i]);
      }
    }
}

template <int BITS, bool G1>
__global__ void __launch_bounds__(kMidWaves * kWave, 3) mid_kernel(MidParams p) {
  __shared__ __attribute__((aligned(16))) uint8_t act[kMidRows * kMidPitch];
  __shared__ __attribute__((aligned(16))) float Xs[kMidUnits * kMidRows];
  const int a = blockIdx.x / p.n_tiles, tile = blockIdx.x - a * p.n_tiles;
  if (a >= min(max(sload(p.active), 0), min(p.E, p.T * p.k))) return;  // block-uniform
  const int m = lane_id() % 16, lsub = lane_id() / 16;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int nrows = p.T * p.k;
  const int e = min(max(sload(p.active + 1 + a), 0), p.E - 1);
  const int o0 = min(max(sload(p.offsets + e), 0), nrows);
  const int o1 = min(max(sload(p.offsets + e + 1), o0), nrows);
  if (o1 - o0 > p.max_rows) return;  // block-uniform
  constexpr int GB = kGroupBytes<BITS>;
  const int G = p.K / kGroup, steps = G / kMidUnits;
  ExpertW xw;
  if (p.tab) {
    xw = expert_from_table(p.tab, e, p.tab_off);
  } else {
    const size_t erow = (size_t)e * p.n_rows_w;
    xw = ExpertW{p.codes + erow * (G * GB), p.scales + erow * (G * 2), p.zeros + erow * G};
  }
  // the wave's two row sets: gate and up rows of its 16 h columns, or 32 down rows
  const int c0 = G1 ? tile * 64 + wv * 16 : tile * 128 + wv * 32;
  const int rows0 = c0, rows1 = G1 ? p.I + c0 : c0 + 16;
  const Off o[2] = {row_off<1>(rows0 + m, G, 0, GB, lsub), row_off<1>(rows1 + m, G, 0, GB, lsub)};
  for (int q0 = o0; q0 < o1; q0 += kMidRows) {
    const int R = min(kMidRows, o1 - q0);
    if (R > 16)
      mid_pass<BITS, G1, 2>(p, xw, o, c0, q0, R, steps, act, Xs);
    else
      mid_pass<BITS, G1, 1>(p, xw, o, c0, q0, R, steps, act, Xs);
  }
}

}  // namespace

bool mid_layout_ok(int H, int I, int bits, int group) {
  return (bits == 4 || bits == 2) && group == 128 && H % kMidStepK == 0 && I % kMidStepK == 0;
}

// The two launches for the experts with at most max_rows rows (gate_up into
// hbuf, then down into y_perm); h is left for the caller to clear.
static MidParams mid_params(const FfnArgs &a, uint16_t *hbuf, int max_rows, bool g1) {
  MidParams m{};
  m.offsets = a.offsets;
  m.sorted_rows = a.sorted_rows;
  m.active = a.active;
  m.T = a.T;
  m.k = a.k;
  m.E = a.E;
  m.I = a.I;
  m.H = a.H;
  m.tab = a.tab;
  m.max_rows = max_rows;
  m.magic = 0x43434343u;
  if (g1) {
    m.a = a.x;
    m.K = a.H;
    m.n_rows_w = 2 * a.I;
    m.n_tiles = a.I / 64;
    m.codes = (const uint8_t *)a.w13_codes;
    m.scales = (const uint8_t *)a.w13_scales;
    m.zeros = a.w13_zeros;
    m.tab_off = 0;
    m.out = hbuf;
  } else {
    m.a = hbuf;
    m.K = a.I;
    m.n_rows_w = a.H;
    m.n_tiles = a.H / 128;
    m.codes = (const uint8_t *)a.w2_codes;
    m.scales = (const uint8_t *)a.w2_scales;
    m.zeros = a.w2_zeros;
    m.tab_off = 3;
    m.out = a.y_perm;
  }
  return m;
}

hipError_t launch_mid_gemm(const FfnArgs &a, uint16_t *hbuf, int max_rows, bool gate_up, hipStream_t st) {
  const int nrows = a.T * a.k;
  const int amax = a.E < nrows ? a.E : nrows;
  const MidParams m = mid_params(a, hbuf, max_rows, gate_up);
  const dim3 grid((unsigned)(amax * m.n_tiles));
  if (a.bits == 4)
    gate_up ? mid_kernel<4, true><<<grid, kMidWaves * kWave, 0, st>>>(m)
            : mid_kernel<4, false><<<grid, kMidWaves * kWave, 0, st>>>(m);
  else
    gate_up ? mid_kernel<2, true><<<grid, kMidWaves * kWave, 0, st>>>(m)
            : mid_kernel<2, false><<<grid, kMidWaves * kWave, 0, st>>>(m);
  return hipGetLastError();
}

hipError_t launch_ffn_mid(const FfnArgs &a, hipStream_t st) {
  uint16_t *hbuf = (uint16_t *)((char *)a.ws + ffn_ctl_bytes(a.T, a.k, a.E));
  hipError_t e = launch_mid_gemm(a, hbuf, a.T * a.k, true, st);
  if (e == hipSuccess) e = launch_mid_gemm(a, hbuf, a.T * a.k, false, st);
  if (e != hipSuccess) return e;
  return launch_zero16(hbuf, (size_t)a.T * a.k * a.I * sizeof(uint16_t), st);
}

}  // namespace bqmoe
