// Grouped-GEMM expert FFN (many rows per expert, e.g. prefill): two grouped GEMMs on bf16 MFMA.
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
//    tile, dequantised once per block to bf16 (q - z) * s (INT4, 2-bit, INT8
//    or FP6 e2m3 codes; one scale per 128 or per 32 K; NVFP4: E2M1 codes with
//    an E4M3 scale per 16 K, exact in bf16), go through two LDS
//    buffers with an XOR swizzle of 16-byte chunks, so both the staging
//    writes and the MFMA operand reads are free of bank conflicts;
//  * 4 waves in a 2 x 2 arrangement each own a 64 x 64 sub-tile computed with
//    v_mfma_f32_16x16x32_bf16 (float32 accumulation);
//  * software pipeline with one barrier per K tile of 64: while the MFMAs
//    read one buffer, the next tile is dequantised into the other and global
//    loads run S tiles ahead in registers;
//  * INT4 and 2-bit g128: the experts with at most kHybridRows rows run the
//    middle-batch kernel instead (their M tile would dequantise a whole
//    expert's weights for a few rows), so the GEMMs skip them.
#include <type_traits>

#include "common.cuh"
#include "internal.h"

namespace bqmoe {
namespace {

constexpr int BM = 128, BN = 128;
constexpr int BK = 64;                       // K per tile: half a 128 group, two 32 groups
constexpr int kRowBytes = BK * 2;            // one LDS row: 64 bf16 = 8 chunks of 16 B
constexpr int kTileBytes = 128 * kRowBytes;  // 16 KiB per operand tile
constexpr int kBufWord3 = 0x00020000;        // buffer resource word 3: raw 32-bit access
constexpr int kMGroup = 1;  // consecutive M-tile slots per XCD, iterated fastest (2-8 measured: no gain)
constexpr int kHybridRows = 64;  // INT4 / 2-bit g128: experts with at most this many rows take the mid kernel (32-128 measured, 64 best)

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
  const uint64_t *tab;     // per-expert address table or null; this GEMM's entries start at tab_off
  int tab_off;
  int n_blocks;            // N tiles: I / 64 (G1) or H / BN (G2)
  int min_rows;            // experts with at most this many rows are left to the mid kernel
  // NVFP4: per-expert float32 tensor scales of the weights, the tensor scale
  // of this GEMM's (quantised) A operand, and G1's h quantiser scale
  const float *gscale;
  float act_g, out_g;
};



// LDS position of 16-byte chunk `chunk` of tile row `row`.  Eight lanes that
// read (or write) the same chunk of eight consecutive rows, or eight chunks
// of one row, touch eight distinct 16-byte bank groups.
__device__ __forceinline__ int swz(int row, int chunk) { return row * kRowBytes + ((chunk ^ (row & 7)) << 4); }

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
        tiles = o1 - o0 > p.min_rows ? (o1 - o0 + BM - 1) / BM : 0;
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

template <int N>
using IntC = std::integral_constant<int, N>;

// S: K tiles held in registers ahead of LDS (K / BK must be a multiple of S).
// GS: quantisation group along K, 128 or 32 (a thread's 32 K of a tile then
// form one group); 16 with BITS = 4 is NVFP4 (a thread's 32 K hold two groups).
template <int BITS, int GS, bool GATEUP, int S>
__global__ void __launch_bounds__(256, 2) ffn_gemm_kernel(GemmParams p) {
  // two LDS buffers, each an A tile then a B tile (BM and BN rows of BK bf16)
  __shared__ __attribute__((aligned(16))) uint8_t lds[2][2 * kTileBytes];
  // Blocks are dealt to the 8 XCDs round-robin; the n_blocks N tiles of one
  // M tile go to consecutive blocks of the same XCD, so the A tile is read
  // into that XCD's L2 once and reused by all of them.
  const int xcd = blockIdx.x % 8, local = blockIdx.x / 8;
  const int msub = local % kMGroup;
  const int nb = (local / kMGroup) % p.n_blocks;
  const int mslot = (local / kMGroup / p.n_blocks) * (8 * kMGroup) + xcd * kMGroup + msub;
  int e, m0, rows;
  if (!find_tile(p, mslot, &e, &m0, &rows)) return;
  constexpr bool NV = GS == 16;

  const int tid = threadIdx.x;
  const int lane = tid % kWave;
  const int wave = tid / kWave;
  const int wm = wave / 2, wn = wave % 2;

  // Loads go through buffer resources: one 32-bit byte offset per stream and
  // the K-tile step in the scalar offset.  G2 rows are contiguous from the
  // tile's first row; G1 rows are gathered tokens.
  const uint16_t *a_base = GATEUP ? p.a_src : p.a_src + (size_t)m0 * p.K;
  const uint32_t a_bytes = (uint32_t)(GATEUP ? p.T : rows) * (uint32_t)p.K * 2u;
  const __amdgpu_buffer_rsrc_t a_rs = __builtin_amdgcn_make_buffer_rsrc((void *)a_base, (short)0, (int)a_bytes, kBufWord3);
  // A staging: thread -> rows (tid >> 3) + 32 j (j < 4), chunk tid & 7.  Rows
  // past the tile read the tile's last row instead: every load is
  // unconditional (branches around loads defeat the compiler's load
  // counting), and those rows only feed C rows that are never stored.
  const int ar = tid >> 3, ac = tid & 7;
  uint32_t a_off[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int r = min(ar + 32 * j, rows - 1);
    const int src = GATEUP ? min(max(p.sorted_rows[m0 + r], 0) / p.k, p.T - 1) : r;
    a_off[j] = (uint32_t)(src * p.K + ac * 8) * 2u;
  }
  // B staging: thread -> weight row tid / 2 of the tile, code words
  // (tid % 2) * WPL .. + WPL of the K tile, i.e. LDS chunks (tid % 2) * 4 .. + 4.
  // G1 tiles give each wave column 32 gate rows then the 32 matching up rows.
  constexpr int WPT = BK * BITS / 32;         // code words per tile row: 8 (INT4), 4 (INT2), 16 (INT8), 12 (FP6)
  constexpr int WPL = WPT / 2;                // words per thread: 32 K of one row
  const int br = tid >> 1, bh = tid & 1;
  int wrow;
  if (GATEUP) {
    const int wn_b = br / 64, cc = br % 64;
    const int i = nb * 64 + wn_b * 32 + (cc % 32);
    wrow = (cc < 32) ? i : p.I + i;
  } else {
    wrow = nb * BN + br;
  }
  const int wpr = p.K * BITS / 32, gpr = p.K / GS;     // code words and groups per weight row
  const size_t erow0 = (size_t)e * p.n_rows_w;          // the expert's first weight row
  const uint64_t *te = p.tab ? p.tab + (size_t)e * kTabStride + p.tab_off : nullptr;
  const uint32_t *e_codes = te ? (const uint32_t *)sload(te) : p.codes + erow0 * wpr;
  // NVFP4 scales are single bytes
  const uint16_t *e_scales = te ? (const uint16_t *)sload(te + 1)
                                : (NV ? (const uint16_t *)((const uint8_t *)p.scales + erow0 * gpr) : p.scales + erow0 * gpr);
  const uint8_t *e_zeros = te ? (const uint8_t *)sload(te + 2) : (BITS == 2 ? p.zeros + erow0 * gpr : p.zeros);
  const __amdgpu_buffer_rsrc_t b_rs =
      __builtin_amdgcn_make_buffer_rsrc((void *)e_codes, (short)0, p.n_rows_w * wpr * 4, kBufWord3);
  const __amdgpu_buffer_rsrc_t s_rs =
      __builtin_amdgcn_make_buffer_rsrc((void *)e_scales, (short)0, p.n_rows_w * gpr * (NV ? 1 : 2), kBufWord3);
  const __amdgpu_buffer_rsrc_t z_rs = __builtin_amdgcn_make_buffer_rsrc(
      (void *)e_zeros, (short)0, BITS == 2 ? p.n_rows_w * gpr : 0, kBufWord3);
  const uint32_t b_off = (uint32_t)(wrow * wpr + bh * WPL) * 4u;  // bytes
  // elements; with GS = 32 the thread's half of a tile is group 2 kt + bh,
  // with NVFP4 groups 4 kt + 2 bh and + 1
  const uint32_t s_off = (uint32_t)(wrow * gpr) + (GS == 32 ? bh : NV ? 2 * bh : 0);

  // ---- pipeline: one barrier per K tile.  While the MFMAs read buffer kt & 1,
  // tile kt + 1 is dequantised into the other buffer and tile kt + 1 + S is
  // requested from global memory.  Tile t lives in register stage t % S; the
  // K loop is unrolled by S so that every stage index is a constant (a
  // register copy between stages would wait for its load), and it has no
  // exits: K / BK is a multiple of S.
  //
  // MV = 16-row MFMA blocks of this wave's 64 rows that hold data (an
  // expert's last tile is often mostly empty).  It is a template constant of
  // the loop, so the loop body has no branches; waves of one block may run
  // different variants (they meet at the same barriers).
  const int nk = p.K / BK;
  const int mvalid = rows - wm * 64;
  const int mv = __builtin_amdgcn_readfirstlane(mvalid <= 0 ? 0 : mvalid >= 64 ? 4 : (mvalid + 15) / 16);
  auto run = [&](auto mv_c) {
    constexpr int MV = decltype(mv_c)::value;
    // ---- register stages
    u32x4 a_st[S][4];
    uint32_t b_st[S][WPL];
    uint32_t sc_st[S], z_st[S];  // raw bf16 scale / zero-point (no math on a load in flight)
    auto load_tile = [&](int kt, int s) {
  #pragma unroll
      for (int j = 0; j < 4; ++j) a_st[s][j] = __builtin_amdgcn_raw_buffer_load_b128(a_rs, a_off[j], kt * (BK * 2), 0);
      if constexpr (BITS == 6) {
        const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(b_rs, b_off, kt * (WPT * 4), 0);
        const u32x2 u = __builtin_amdgcn_raw_buffer_load_b64(b_rs, b_off + 16, kt * (WPT * 4), 0);
  #pragma unroll
        for (int w = 0; w < 4; ++w) b_st[s][w] = v[w];
        b_st[s][4] = u[0];
        b_st[s][5] = u[1];
      } else if constexpr (BITS == 8) {
  #pragma unroll
        for (int h = 0; h < 2; ++h) {
          const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(b_rs, b_off + 16 * h, kt * (WPT * 4), 0);
  #pragma unroll
          for (int w = 0; w < 4; ++w) b_st[s][4 * h + w] = v[w];
        }
      } else if constexpr (BITS == 4) {
        const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(b_rs, b_off, kt * (WPT * 4), 0);
  #pragma unroll
        for (int w = 0; w < 4; ++w) b_st[s][w] = v[w];
      } else {
        const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(b_rs, b_off, kt * (WPT * 4), 0);
        b_st[s][0] = v[0];
        b_st[s][1] = v[1];
      }
      if constexpr (NV)
        sc_st[s] = __builtin_amdgcn_raw_buffer_load_b16(s_rs, s_off, kt * 4, 0);  // two E4M3 bytes
      else
        sc_st[s] = __builtin_amdgcn_raw_buffer_load_b16(s_rs, s_off * 2u, GS == 32 ? kt * 4 : (kt / 2) * 2, 0);
      if constexpr (BITS == 2) z_st[s] = __builtin_amdgcn_raw_buffer_load_b8(z_rs, s_off, kt / 2, 0);
    };
    auto store_tile = [&](int s, uint8_t *buf) {
  #pragma unroll
      for (int j = 0; j < 4; ++j) *(u32x4 *)(buf + swz(ar + 32 * j, ac)) = a_st[s][j];
      uint8_t *bb = buf + kTileBytes;
      if constexpr (NV) {  // words 0, 1: the first group of 16, words 2, 3: the second
        const float s0 = e4m3_to_f32(sc_st[s] & 0xFFu), s1 = e4m3_to_f32((sc_st[s] >> 8) & 0xFFu);
  #pragma unroll
        for (int w = 0; w < 4; ++w) {
          uint32_t o[4];
          dequant8_e2m1(b_st[s][w], w < 2 ? s0 : s1, o);
          *(u32x4 *)(bb + swz(br, bh * 4 + w)) = u32x4{o[0], o[1], o[2], o[3]};
        }
        return;
      }
      const float sc = BITS == 6 ? fp16_to_f32(sc_st[s]) : bf16_to_f32(sc_st[s]);
      const float zs = -((BITS == 4) ? 8.f : BITS == 8 ? 128.f : BITS == 6 ? 0.f : (float)z_st[s]) * sc;
      if constexpr (BITS == 6) {
        // the thread's 32 codes at once (exact bf16 values), then times the scale
        const u32x16 v = fp6x32_to_bf16(u32x6{b_st[s][0], b_st[s][1], b_st[s][2], b_st[s][3], b_st[s][4], b_st[s][5]});
  #pragma unroll
        for (int c = 0; c < 4; ++c) {
          uint32_t o[4];
  #pragma unroll
          for (int i = 0; i < 4; ++i) o[i] = pack_bf16x2(bf16lo(v[4 * c + i]) * sc, bf16hi(v[4 * c + i]) * sc);
          *(u32x4 *)(bb + swz(br, bh * 4 + c)) = u32x4{o[0], o[1], o[2], o[3]};
        }
        return;
      }
  #pragma unroll
      for (int w = 0; w < WPL; ++w) {
        if constexpr (BITS == 8) {
          if (w & 1) continue;  // words w, w + 1 fill one 16-byte chunk
          uint32_t o[4];
          dequant4_int8(b_st[s][w], sc, zs, o);
          dequant4_int8(b_st[s][w + 1], sc, zs, o + 2);
          *(u32x4 *)(bb + swz(br, bh * 4 + w / 2)) = u32x4{o[0], o[1], o[2], o[3]};
        } else if constexpr (BITS == 4) {
          uint32_t o[4];
          dequant8_int4(b_st[s][w], sc, zs, o);
          *(u32x4 *)(bb + swz(br, bh * 4 + w)) = u32x4{o[0], o[1], o[2], o[3]};
        } else {
          uint32_t o[8];
          dequant16_int2(b_st[s][w], sc, zs, o);
          *(u32x4 *)(bb + swz(br, bh * 4 + 2 * w)) = u32x4{o[0], o[1], o[2], o[3]};
          *(u32x4 *)(bb + swz(br, bh * 4 + 2 * w + 1)) = u32x4{o[4], o[5], o[6], o[7]};
        }
      }
    };
    f32x4 acc[4][4];
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
      for (int ni = 0; ni < 4; ++ni) acc[mi][ni] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < S; ++s) load_tile(min(s, nk - 1), s);
    store_tile(0, lds[0]);
    load_tile(min(S, nk - 1), 0);
    __syncthreads();
    for (int kt0 = 0; kt0 < nk; kt0 += S) {
#pragma unroll
      for (int d = 0; d < S; ++d) {
        const int kt = kt0 + d;
        const uint8_t *ba = lds[kt & 1], *bb = lds[kt & 1] + kTileBytes;
        if constexpr (MV > 0) {
#pragma unroll
          for (int kk = 0; kk < BK / 32; ++kk) {
            const int ch = kk * 4 + lane / 16;
            bf16x8 af[MV], bfr[4];
#pragma unroll
            for (int mi = 0; mi < MV; ++mi) af[mi] = *(const bf16x8 *)(ba + swz(wm * 64 + mi * 16 + lane % 16, ch));
#pragma unroll
            for (int ni = 0; ni < 4; ++ni) bfr[ni] = *(const bf16x8 *)(bb + swz(wn * 64 + ni * 16 + lane % 16, ch));
#pragma unroll
            for (int mi = 0; mi < MV; ++mi)
#pragma unroll
              for (int ni = 0; ni < 4; ++ni)
                acc[mi][ni] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[mi], bfr[ni], acc[mi][ni], 0, 0, 0);
          }
        }
        const int sn = (d + 1) % S;  // stage of tile kt + 1 (a constant once unrolled)
        // Past the end the last tile is stored and loaded again: harmless, and
        // it keeps the loop free of branches around memory operations.
        store_tile(sn, lds[(kt + 1) & 1]);
        load_tile(min(kt + 1 + S, nk - 1), sn);
        __syncthreads();
      }
    }
    // ---- epilogue: C[m][n] of (mi, ni, r) is m = 4*(lane/16) + r, n = lane % 16
    // NVFP4: the products carry the A and weight tensor scales; G1 quantises h
    // in groups of 16 columns (the 16 lanes of one m)
    // (a table row holds the address of the tensor scale in the zero-point slot)
    const float osc = NV ? p.act_g * sload(te ? (const float *)sload(te + 2) : p.gscale + e) : 1.f;
#pragma unroll
    for (int mi = 0; mi < MV; ++mi)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = wm * 64 + mi * 16 + 4 * (lane / 16) + r;
        if (m >= rows) continue;
        const size_t orow = (size_t)(m0 + m);
        if (GATEUP) {
#pragma unroll
          for (int ni = 0; ni < 2; ++ni) {
            const float g = acc[mi][ni][r] * osc, u = acc[mi][ni + 2][r] * osc;
            float hv = g / (1.f + __expf(-g)) * u;
            if constexpr (NV) hv = quant16_lanes(hv, p.out_g);
            const int col = nb * 64 + wn * 32 + ni * 16 + lane % 16;
            p.out[orow * p.I + col] = f32_to_bf16(hv);
          }
        } else {
#pragma unroll
          for (int ni = 0; ni < 4; ++ni) {
            const int col = nb * BN + wn * 64 + ni * 16 + lane % 16;
            p.out[orow * p.H + col] = f32_to_bf16(acc[mi][ni][r] * osc);
          }
        }
      }
  };
  switch (mv) {
    case 4: run(IntC<4>{}); break;
    case 3: run(IntC<3>{}); break;
    case 2: run(IntC<2>{}); break;
    case 1: run(IntC<1>{}); break;
    default: run(IntC<0>{}); break;
  }
}

// Re-zeroes h after the down GEMM has read it: the workspace is all-zero
// between calls, which the decode path's tagged h words rely on.
__global__ void __launch_bounds__(256) zero_kernel(u32x4 *p, size_t n16) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += (size_t)gridDim.x * 256)
    p[i] = u32x4{0u, 0u, 0u, 0u};
}

}  // namespace

hipError_t launch_zero16(void *p, size_t bytes, hipStream_t st) {
  const size_t n16 = bytes / 16;
  if (n16 == 0) return hipSuccess;
  const size_t zb = (n16 + 255) / 256;
  zero_kernel<<<(unsigned)(zb < 2048 ? zb : 2048), 256, 0, st>>>((u32x4 *)p, n16);
  return hipGetLastError();
}

hipError_t launch_ffn_prefill(const FfnArgs &a, const DeviceInfo &, hipStream_t st) {
  const int nrows = a.T * a.k;
  const int Amax = a.E < nrows ? a.E : nrows;
  long slots = ((long)nrows + (long)Amax * (BM - 1)) / BM;
  slots = (slots + 8 * kMGroup - 1) / (8 * kMGroup) * (8 * kMGroup);  // whole rounds of the 8 XCDs
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
  g1.tab = a.tab;
  g1.tab_off = 0;
  g1.gscale = a.w13_g;
  g1.act_g = a.gx;
  g1.out_g = a.gh;
  // NVFP4: the quantised activations (q * s, bf16) follow h in the workspace
  uint16_t *xq = hbuf + (size_t)nrows * a.I;
  if (a.nvfp4) {
    const hipError_t e = launch_quant_nvfp4(a.x, (int64_t)a.T * a.H, a.gx, xq, nullptr, st);
    if (e != hipSuccess) return e;
    g1.a_src = xq;
  }

  GemmParams g2 = g1;
  g2.a_src = hbuf;
  g2.K = a.I;
  g2.codes = a.w2_codes;
  g2.scales = a.w2_scales;
  g2.zeros = a.w2_zeros;
  g2.out = a.y_perm;
  g2.n_rows_w = a.H;
  g2.tab_off = 3;
  g2.gscale = a.w2_g;
  g2.act_g = a.gh;

  g1.n_blocks = a.I / 64;
  g2.n_blocks = a.H / BN;
  // Hybrid: for INT4 and 2-bit g128 the experts with at most kHybridRows rows
  // take the middle-batch kernel (weights read once, no per-element
  // dequantisation) and the GEMMs skip them; the two write disjoint h and
  // y_perm rows.
  const bool hybrid = !a.nvfp4 && mid_layout_ok(a.H, a.I, a.bits, a.group);
  g1.min_rows = g2.min_rows = hybrid ? kHybridRows : 0;
  dim3 grid1((unsigned)(slots * g1.n_blocks)), grid2((unsigned)(slots * g2.n_blocks));
  // two register stages: K % 128 == 0 makes K / BK even
  auto run = [&](auto g1k, auto g2k) {
    if (hybrid) {
      const hipError_t e = launch_mid_gemm(a, hbuf, kHybridRows, true, st);
      if (e != hipSuccess) return e;
    }
    g1k<<<grid1, 256, 0, st>>>(g1);
    if (hybrid) {
      const hipError_t e = launch_mid_gemm(a, hbuf, kHybridRows, false, st);
      if (e != hipSuccess) return e;
    }
    g2k<<<grid2, 256, 0, st>>>(g2);
    return hipGetLastError();
  };
  hipError_t err;
  if (a.nvfp4)
    err = run(ffn_gemm_kernel<4, 16, true, 2>, ffn_gemm_kernel<4, 16, false, 2>);
  else if (a.bits == 4 && a.group == 128)
    err = run(ffn_gemm_kernel<4, 128, true, 2>, ffn_gemm_kernel<4, 128, false, 2>);
  else if (a.bits == 4)
    err = run(ffn_gemm_kernel<4, 32, true, 2>, ffn_gemm_kernel<4, 32, false, 2>);
  else if (a.bits == 8 && a.group == 128)
    err = run(ffn_gemm_kernel<8, 128, true, 2>, ffn_gemm_kernel<8, 128, false, 2>);
  else if (a.bits == 8)
    err = run(ffn_gemm_kernel<8, 32, true, 2>, ffn_gemm_kernel<8, 32, false, 2>);
  else if (a.bits == 6)
    err = run(ffn_gemm_kernel<6, 128, true, 2>, ffn_gemm_kernel<6, 128, false, 2>);
  else
    err = run(ffn_gemm_kernel<2, 128, true, 2>, ffn_gemm_kernel<2, 128, false, 2>);
  if (err != hipSuccess) return err;
  // h is T*k*I bf16 (I % 128 == 0, so a whole number of 16-byte chunks),
  // followed for NVFP4 by the T*H quantised activations
  const size_t n16 = ((size_t)nrows * a.I + (a.nvfp4 ? (size_t)a.T * a.H : 0)) * sizeof(uint16_t) / 16;
  const size_t zb = (n16 + 255) / 256;
  zero_kernel<<<(unsigned)(zb < 2048 ? zb : 2048), 256, 0, st>>>((u32x4 *)hbuf, n16);
  return hipGetLastError();
}

}  // namespace bqmoe
