// Prefill-path expert FFN (T > 16 tokens): two grouped GEMMs on bf16 MFMA.
//
//   G1: h[p, i] = silu(x_t . W13[e, i]) * (x_t . W13[e, I + i])   -> bf16 workspace
//   G2: y_perm[p, n] = h[p] . W2[e, n]                            -> bf16
//
// for every active expert e and its sorted rows p (token t = sorted_rows[p]/k).
// The pages name the expert GEMM as the bound of a prefill chunk once the
// interconnect is fast (page "Qwen3.8-Flash-Next FP6-INT8", "Step budget and
// hardware floors") and run prefill through a grouped MoE kernel with the
// low-bit unpack inside it (page "Qwen3.8-Flash-Next on one 24 GB GPU", "What
// the patch does").  This is a from-scratch gfx950 design:
//
//  * a block computes a BM x BN tile of one expert; the tile list (expert,
//    M-tile) is derived on the device from the permutation offsets, so the
//    host launches an upper bound of M-tile slots and surplus blocks exit;
//  * A rows (gathered activations for G1, contiguous h rows for G2) and the B
//    tile, dequantised once per block to bf16 (q - z) * s, are staged in LDS
//    with an XOR swizzle of 16-byte chunks so the MFMA operand reads are
//    conflict-free;
//  * 4 waves in a 2 x 2 arrangement each own a 64 x 64 sub-tile computed with
//    v_mfma_f32_16x16x32_bf16 (float32 accumulation);
//  * global loads of the next K tile are issued before the MFMAs of the
//    current one (register staging).
#include "common.cuh"
#include "internal.h"

namespace bqmoe {
namespace {

constexpr int BM = 128, BN = 128, BK = 128;
constexpr int kRowBytes = BK * 2;  // one LDS row: 128 bf16 = 16 chunks of 16 B

struct GemmParams {
  const uint16_t *a_src;   // G1: x [T, H]; G2: h [T*k, I]
  const int32_t *offsets;
  const int32_t *sorted_rows;
  const int32_t *active;
  int T, k, E, H, I;
  int K;                   // reduction length: H (G1) or I (G2)
  const uint32_t *codes;   // G1: w13 codes; G2: w2 codes
  const uint16_t *scales;
  const uint8_t *zeros;
  uint16_t *out;           // G1: h; G2: y_perm
  int n_rows_w;            // rows of one expert's weight matrix: 2I (G1) or H (G2)
};

__device__ __forceinline__ int swz(int row, int chunk) { return row * kRowBytes + ((chunk ^ (row & 15)) << 4); }

// Find the (expert, M-tile) of M-tile slot `slot`; returns false past the end.
__device__ bool find_tile(const GemmParams &p, int slot, int *e_out, int *m0_out, int *n_e_out) {
  __shared__ int s_info[3];
  const int tid = threadIdx.x;
  const int nrows = p.T * p.k;
  if (tid < kWave) {
    const int lane = tid;
    const int A = min(max(p.active[0], 0), min(p.E, nrows));
    int base = 0;
    int found = 0;
    for (int a0 = 0; a0 < A && !found; a0 += kWave) {
      const int a = a0 + lane;
      int tiles = 0, e = 0, o0 = 0, o1 = 0;
      if (a < A) {
        e = min(max(p.active[1 + a], 0), p.E - 1);
        o0 = min(max(p.offsets[e], 0), nrows);
        o1 = min(max(p.offsets[e + 1], o0), nrows);
        tiles = (o1 - o0 + BM - 1) / BM;
      }
      int inc = tiles;
#pragma unroll
      for (int d = 1; d < kWave; d <<= 1) {
        const int v = __shfl_up(inc, d, kWave);
        if (lane >= d) inc += v;
      }
      const int excl = base + inc - tiles;
      const bool mine = (a < A) && slot >= excl && slot < excl + tiles;
      const uint64_t m = __ballot(mine);
      if (m) {
        found = 1;
        if (mine) {
          s_info[0] = e;
          s_info[1] = o0 + (slot - excl) * BM;
          s_info[2] = min(BM, o1 - (o0 + (slot - excl) * BM));
        }
      }
      base += __shfl(inc, kWave - 1, kWave);
    }
    if (lane == 0 && !found) s_info[0] = -1;
  }
  __syncthreads();
  *e_out = s_info[0];
  *m0_out = s_info[1];
  *n_e_out = s_info[2];
  return s_info[0] >= 0;
}

template <int BITS, bool GATEUP>
__global__ void __launch_bounds__(256, 2) ffn_gemm_kernel(GemmParams p) {
  __shared__ __attribute__((aligned(16))) uint8_t lds_a[BM * kRowBytes];
  __shared__ __attribute__((aligned(16))) uint8_t lds_b[BN * kRowBytes];
  int e, m0, rows;
  if (!find_tile(p, blockIdx.x, &e, &m0, &rows)) return;

  const int tid = threadIdx.x;
  const int lane = tid % kWave;
  const int wave = tid / kWave;
  const int wm = wave / 2, wn = wave % 2;
  const int nb = blockIdx.y;

  // ---- this thread's global sources
  // A: tile row ra = tid / 2, K half (tid % 2) * 64 .. +64 (8 chunks of 8 bf16)
  const int ra = tid / 2, ha = tid % 2;
  const uint16_t *a_row = nullptr;
  if (ra < rows) {
    const int q = m0 + ra;
    const size_t src_row = GATEUP ? (size_t)min(max(p.sorted_rows[q], 0) / p.k, p.T - 1) : (size_t)q;
    a_row = p.a_src + src_row * p.K + ha * 64;
  }
  // B: tile column cb = tid / 2 (a weight row), K half (tid % 2) * 64 .. +64
  const int cb = tid / 2, hb = tid % 2;
  int wrow;
  if (GATEUP) {
    const int wn_b = cb / 64, cc = cb % 64;
    const int i = nb * 64 + wn_b * 32 + (cc % 32);
    wrow = (cc < 32) ? i : p.I + i;
  } else {
    wrow = nb * BN + cb;
  }
  constexpr int WPH = 64 * BITS / 32;  // words per half row of the K tile: 8 (INT4) or 4 (INT2)
  const size_t wrow_g = (size_t)e * p.n_rows_w + wrow;
  const uint32_t *b_row = p.codes + wrow_g * (p.K * BITS / 32) + hb * WPH;
  const uint16_t *s_row = p.scales + wrow_g * (p.K / kGroup);
  const uint8_t *z_row = (BITS == 2) ? p.zeros + wrow_g * (p.K / kGroup) : nullptr;

  u32x4 a_reg[8];
  u32x4 b_reg[WPH / 4];
  float s_reg = 0.f, z_reg = 0.f;
  auto load_global = [&](int kt) {
    if (a_row) {
#pragma unroll
      for (int c = 0; c < 8; ++c) a_reg[c] = *(const u32x4 *)(a_row + kt * BK + c * 8);
    } else {
#pragma unroll
      for (int c = 0; c < 8; ++c) a_reg[c] = u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int c = 0; c < WPH / 4; ++c) b_reg[c] = *(const u32x4 *)(b_row + (size_t)kt * (BK * BITS / 32) + c * 4);
    s_reg = bf16_to_f32(s_row[kt]);
    z_reg = (BITS == 4) ? 8.f : (float)z_row[kt];
  };
  auto store_lds = [&]() {
#pragma unroll
    for (int c = 0; c < 8; ++c) *(u32x4 *)(lds_a + swz(ra, ha * 8 + c)) = a_reg[c];
    const float zs = -z_reg * s_reg;
    if constexpr (BITS == 4) {
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          uint32_t o[4];
          dequant8_int4(b_reg[c][j], s_reg, zs, o);
          *(u32x4 *)(lds_b + swz(cb, hb * 8 + c * 4 + j)) = u32x4{o[0], o[1], o[2], o[3]};
        }
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        uint32_t o[8];
        dequant16_int2(b_reg[0][j], s_reg, zs, o);
        *(u32x4 *)(lds_b + swz(cb, hb * 8 + 2 * j)) = u32x4{o[0], o[1], o[2], o[3]};
        *(u32x4 *)(lds_b + swz(cb, hb * 8 + 2 * j + 1)) = u32x4{o[4], o[5], o[6], o[7]};
      }
    }
  };

  f32x4 acc[4][4];
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
#pragma unroll
    for (int ni = 0; ni < 4; ++ni) acc[mi][ni] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nk = p.K / BK;
  load_global(0);
  for (int kt = 0; kt < nk; ++kt) {
    __syncthreads();
    store_lds();
    __syncthreads();
    if (kt + 1 < nk) load_global(kt + 1);
#pragma unroll
    for (int kk = 0; kk < BK / 32; ++kk) {
      const int ch = kk * 4 + lane / 16;
      bf16x8 af[4], bfr[4];
#pragma unroll
      for (int mi = 0; mi < 4; ++mi)
        af[mi] = *(const bf16x8 *)(lds_a + swz(wm * 64 + mi * 16 + lane % 16, ch));
#pragma unroll
      for (int ni = 0; ni < 4; ++ni)
        bfr[ni] = *(const bf16x8 *)(lds_b + swz(wn * 64 + ni * 16 + lane % 16, ch));
#pragma unroll
      for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int ni = 0; ni < 4; ++ni)
          acc[mi][ni] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[mi], bfr[ni], acc[mi][ni], 0, 0, 0);
    }
  }

  // ---- epilogue: C[m][n] of (mi, ni, r) is m = 4*(lane/16) + r, n = lane % 16
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int m = wm * 64 + mi * 16 + 4 * (lane / 16) + r;
      if (m >= rows) continue;
      const size_t orow = (size_t)(m0 + m);
      if (GATEUP) {
#pragma unroll
        for (int ni = 0; ni < 2; ++ni) {
          const float g = acc[mi][ni][r], u = acc[mi][ni + 2][r];
          const float hv = g / (1.f + __expf(-g)) * u;
          const int col = nb * 64 + wn * 32 + ni * 16 + lane % 16;
          p.out[orow * p.I + col] = f32_to_bf16(hv);
        }
      } else {
#pragma unroll
        for (int ni = 0; ni < 4; ++ni) {
          const int col = nb * BN + wn * 64 + ni * 16 + lane % 16;
          p.out[orow * p.H + col] = f32_to_bf16(acc[mi][ni][r]);
        }
      }
    }
}

}  // namespace

hipError_t launch_ffn_prefill(const FfnArgs &a, const DeviceInfo &, hipStream_t st) {
  const int nrows = a.T * a.k;
  const int Amax = a.E < nrows ? a.E : nrows;
  const long slots = ((long)nrows + (long)Amax * (BM - 1)) / BM;
  uint16_t *hbuf = (uint16_t *)((char *)a.ws + ffn_ctl_bytes(a.T, a.k, a.E));

  GemmParams g1;
  g1.a_src = a.x;
  g1.offsets = a.offsets;
  g1.sorted_rows = a.sorted_rows;
  g1.active = a.active;
  g1.T = a.T;
  g1.k = a.k;
  g1.E = a.E;
  g1.H = a.H;
  g1.I = a.I;
  g1.K = a.H;
  g1.codes = a.w13_codes;
  g1.scales = a.w13_scales;
  g1.zeros = a.w13_zeros;
  g1.out = hbuf;
  g1.n_rows_w = 2 * a.I;

  GemmParams g2 = g1;
  g2.a_src = hbuf;
  g2.K = a.I;
  g2.codes = a.w2_codes;
  g2.scales = a.w2_scales;
  g2.zeros = a.w2_zeros;
  g2.out = a.y_perm;
  g2.n_rows_w = a.H;

  dim3 grid1((unsigned)slots, a.I / 64), grid2((unsigned)slots, a.H / BN);
  if (a.bits == 4) {
    ffn_gemm_kernel<4, true><<<grid1, 256, 0, st>>>(g1);
    ffn_gemm_kernel<4, false><<<grid2, 256, 0, st>>>(g2);
  } else {
    ffn_gemm_kernel<2, true><<<grid1, 256, 0, st>>>(g1);
    ffn_gemm_kernel<2, false><<<grid2, 256, 0, st>>>(g2);
  }
  return hipGetLastError();
}

}  // namespace bqmoe
