// Router: logits in the fixed float32 order, top-k with lower-index ties,
// softmax over the selected logits.
//
// Summation order (identical in both kernels): h is split into 64 contiguous
// slices of L = H/64 elements; a slice sum starts at 0 and adds its products
// in ascending h (each bf16*bf16 product is exact in float32, so fma == add of
// the product); the 64 slice sums are combined as a balanced pairwise tree in
// index order; the optional bias is added last.  The pages keep routers in
// 16-bit precision because near-tied logits flip routing under small
// perturbations (page "Qwen3.8-Flash-Next FP6-INT8", "Precision map"); fixing
// the order makes the selected experts reproducible bit for bit.
#include <math.h>

#include "common.cuh"
#include "internal.h"
#include "route_dev.cuh"

namespace bqmoe {
namespace {

// ------------------------------------------------------------ small T
// Two launch shapes compute the logits (lane s = slice s, sequential over its
// h): route_small_lds_kernel (H a power of two from 512 to 4096) stages four
// experts' weight rows and two tokens' rows in LDS per block;
// route_small_kernel (other H) gives each expert a block of up to eight
// waves, four tokens per wave.  Each logit is stored as a 64-bit word, the
// float bits under a nonzero tag, with a device-coherent store.  Blocks
// 0 .. nsel-1 (nsel = min(T, E)) then run the top-k of tokens b, b + nsel,
// ...: they read the token's E words until every one carries the tag (each
// word is self-validating, so no counter and no store wait are needed), then
// clear them for the next call.  Every block of the grid is co-resident (one
// per expert, or one per 4 experts x 2 tokens, a few waves each), so the
// wait ends; it is bounded anyway and a timeout only raises the error flag.

// Outputs of the grouping by expert, when the router launch also groups the
// rows (T*k <= kFusedRows).
struct GroupOut {
  int32_t *offsets, *sorted_rows, *row_pos, *active;
  int n_active_slots;
};

constexpr int kSmallMaxWaves = 8;  // waves per block of the small router kernel

// The selection part of the small router launches, run by one wave of block
// e < min(T, E) once the block's own logits are stored: the top-k and
// softmax of tokens e, e + nsel, ... and, with GROUP, the grouping of the
// rows by expert.  group_lds: LDS of (kFusedRows + E) ints.
template <bool GROUP>
__device__ void small_selection(int e, int T, int E, int k, int32_t *ids, float *gates, uint64_t *tl, float *lg_out,
                                int *ctl, int max_spins, const GroupOut &go, int *group_lds) {
  const int lane = lane_id();
  const int nsel = min(T, E);
  if (e >= nsel) return;
  // token t's logits: poll the tagged words, then clear them for the next call
  auto logits_of = [&](int t) {
    return TaggedLogits{tl + (size_t)t * E, E, max_spins, ctl, true, lg_out ? lg_out + (size_t)t * E : nullptr};
  };
  if constexpr (!GROUP) {
    for (int t = e; t < T; t += nsel)
      topk_softmax_any(logits_of(t), E, k, ids + (size_t)t * k, gates + (size_t)t * k);
  } else {
    const int n = T * k;
    if (nsel == 1) {
      // One selector: every id is in its LDS; at n <= 64 the grouping runs in registers.
      for (int t = 0; t < T; ++t)
        topk_softmax_any(logits_of(t), E, k, ids + (size_t)t * k, gates + (size_t)t * k, group_lds + t * k);
      __builtin_amdgcn_wave_barrier();
      if (n <= kWave) {
        int kr = E + 1;
        if (lane < n) {
          const int id = group_lds[lane];
          kr = (id >= 0 && id < E) ? id : E;
        }
        wave_group_rows_small(kr, n, E, go.offsets, go.sorted_rows, go.row_pos, go.active, go.n_active_slots);
      } else {
        wave_group_rows(group_lds, n, E, group_lds + kFusedRows, go.offsets, go.sorted_rows, go.row_pos, go.active,
                        go.n_active_slots);
      }
      return;
    }
    // Several selectors publish their ids; the last one to finish reads them
    // back and groups the rows.
    for (int t = e; t < T; t += nsel)
      topk_softmax_any<true>(logits_of(t), E, k, ids + (size_t)t * k, gates + (size_t)t * k);
    wait_vmem();  // the ids are stored before this selector counts itself done
    int last = 0;
    if (lane == 0) last = atomicAdd(&ctl[kCtlRouteSel], 1) == nsel - 1;
    if (!__builtin_amdgcn_readfirstlane(last)) return;
    if (lane == 0) __hip_atomic_store(&ctl[kCtlRouteSel], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (n <= kWave) {
      int kr = E + 1;
      if (lane < n) {
        const int id = __hip_atomic_load(ids + lane, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        kr = (id >= 0 && id < E) ? id : E;
      }
      wave_group_rows_small(kr, n, E, go.offsets, go.sorted_rows, go.row_pos, go.active, go.n_active_slots);
    } else {
      int *key = group_lds, *cur = group_lds + kFusedRows;
      for (int r = lane; r < n; r += kWave) {
        const int id = __hip_atomic_load(ids + r, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        key[r] = (id >= 0 && id < E) ? id : E;
      }
      __builtin_amdgcn_wave_barrier();
      wave_group_rows(key, n, E, cur, go.offsets, go.sorted_rows, go.row_pos, go.active, go.n_active_slots);
    }
  }
}

template <int VEC, bool GROUP>
__global__ void __launch_bounds__(kSmallMaxWaves * 64) route_small_kernel(const uint16_t *__restrict__ x,
                                                         const uint16_t *__restrict__ w, const float *bias, int T,
                                                         int H, int E, int k, int32_t *ids, float *gates,
                                                         uint64_t *tl, float *lg_out, int *ctl, int max_spins,
                                                         GroupOut go) {
  extern __shared__ int group_lds[];  // GROUP with several selectors: key[kFusedRows], then cur[E]
  const int e = blockIdx.x;
  // the block's waves share expert e's tokens, kTB at a time; only wave 0
  // goes on to the selection
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  router_logits_wave<VEC>(x, w, bias, T, H, E, e, tl, wv, blockDim.x / kWave);
  if (wv != 0) return;
  small_selection<GROUP>(e, T, E, k, ids, gates, tl, lg_out, ctl, max_spins, go, group_lds);
}

// The same launch with the rows staged in LDS (H a power of two from 512 to
// 4096): a block takes kLdsExperts experts (one per wave) and kLdsTokens
// tokens.  Its 256 threads load the weight rows and the activation rows with
// coalesced 16-byte loads (1 KB per instruction), all in flight together,
// into the padded slice layout; each wave then runs its expert's fixed-order
// dots (lane s chains slice s, then the pairwise tree, then the bias) for the
// tokens, two chains interleaved.  Loading a slice per lane from memory
// instead touches 64 lines per instruction, and with several waves per CU
// those lines do not stay in the L1.  Blocks past the (expert, token) tiles
// only select; block b < min(T, E) selects after its own logits.
constexpr int kLdsExperts = 4, kLdsTokens = 2;
constexpr int kLdsRows = kLdsExperts + kLdsTokens;
template <bool GROUP>
__global__ void __launch_bounds__(256) route_small_lds_kernel(const uint16_t *__restrict__ x,
                                                             const uint16_t *__restrict__ w, const float *bias,
                                                             int T, int H, int E, int k, int32_t *ids, float *gates,
                                                             uint64_t *tl, float *lg_out, int *ctl, int max_spins,
                                                             GroupOut go) {
  extern __shared__ __attribute__((aligned(16))) uint32_t rows_lds[];
  const int sw64 = 64 * router_slice_words(H);
  int *group_lds = (int *)(rows_lds + kLdsRows * sw64);
  const int neg = (E + kLdsExperts - 1) / kLdsExperts, ntg = (T + kLdsTokens - 1) / kLdsTokens;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  if ((int)blockIdx.x < neg * ntg) {
    const int e0 = (blockIdx.x % neg) * kLdsExperts, t0 = (blockIdx.x / neg) * kLdsTokens;
    const int nch = H / 8, sh = __builtin_ctz(H / 512), sw = router_slice_words(H);
    // rows 0 .. kLdsExperts-1: weight rows e0 + r; then the token rows t0 + r
    // (clamped to the last expert / token; their results are not stored)
    u32x4 a[kLdsRows][2];
#pragma unroll
    for (int r = 0; r < kLdsRows; ++r) {
      const uint16_t *row = r < kLdsExperts ? w + (size_t)min(e0 + r, E - 1) * H
                                            : x + (size_t)min(t0 + r - kLdsExperts, T - 1) * H;
#pragma unroll
      for (int q = 0; q < 2; ++q) a[r][q] = ((const u32x4 *)row)[min((int)threadIdx.x + q * 256, nch - 1)];
    }
#pragma unroll
    for (int r = 0; r < kLdsRows; ++r)
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int c = threadIdx.x + q * 256;
        if (c < nch) *(u32x4 *)&rows_lds[r * sw64 + (c >> sh) * sw + (c & ((1 << sh) - 1)) * 4] = a[r][q];
      }
    __syncthreads();
    const int e = e0 + wv;
    if (e < E) {
      const int lane = lane_id();
      const uint32_t *wp = rows_lds + wv * sw64 + lane * sw;
      const uint32_t *xp0 = rows_lds + kLdsExperts * sw64 + lane * sw, *xp1 = xp0 + sw64;
      float acc0 = 0.f, acc1 = 0.f;
#pragma unroll 8
      for (int j = 0; j < H / 128; j += 4) {
        const u32x4 ww = *(const u32x4 *)(wp + j), x0 = *(const u32x4 *)(xp0 + j), x1 = *(const u32x4 *)(xp1 + j);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          acc0 = __builtin_fmaf(bf16lo(x0[r]), bf16lo(ww[r]), acc0);
          acc0 = __builtin_fmaf(bf16hi(x0[r]), bf16hi(ww[r]), acc0);
          acc1 = __builtin_fmaf(bf16lo(x1[r]), bf16lo(ww[r]), acc1);
          acc1 = __builtin_fmaf(bf16hi(x1[r]), bf16hi(ww[r]), acc1);
        }
      }
      const float b = bias ? bias[e] : 0.f;
      const float v0 = group_sum(acc0, kWave) + b, v1 = group_sum(acc1, kWave) + b;
      if (lane == 0) {
        __hip_atomic_store(tl + (size_t)t0 * E + e, kLogitTag | __float_as_uint(v0), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
        if (t0 + 1 < T)
          __hip_atomic_store(tl + (size_t)(t0 + 1) * E + e, kLogitTag | __float_as_uint(v1), __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  }
  if (wv != 0) return;
  small_selection<GROUP>(blockIdx.x, T, E, k, ids, gates, tl, lg_out, ctl, max_spins, go, group_lds);
}

// ------------------------------------------------------------ large T
// One block: 16 tokens x all experts (chunks of 256).  Thread (ty, tx) owns
// tokens 4*ty..4*ty+3 and experts c*256 + tx + 64*j, j = 0..3.  Each output
// keeps a running slice sum and a 6-level carry stack that combines the 64
// slice sums in the pairwise-tree order as they complete.
constexpr int kTileT = 16;
constexpr int kSub = 32;  // h elements staged in LDS per step

__global__ void __launch_bounds__(256) route_tiled_kernel(const uint16_t *__restrict__ x,
                                                          const uint16_t *__restrict__ w, const float *bias,
                                                          int T, int H, int E, int k, int32_t *ids,
                                                          float *gates, float *lg_out) {
  __shared__ __attribute__((aligned(16))) float xs[kSub][kTileT];
  __shared__ __attribute__((aligned(16))) float wsm[kSub][256];
  extern __shared__ __attribute__((aligned(16))) float lgs[];  // [kTileT][E]
  const int tid = threadIdx.x;
  const int tx = tid % 64, ty = tid / 64;
  const int t_base = blockIdx.x * kTileT;
  const int L = H / 64;

  for (int c0 = 0; c0 < E; c0 += 256) {
    float lvl[6][4][4];
    float acc[4][4];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int b = 0; b < 4; ++b) acc[a][b] = 0.f;

    int s = 0;         // current slice
    int in_slice = 0;  // elements of slice s consumed so far
    for (int h0 = 0; h0 < H; h0 += kSub) {
      __syncthreads();
      {
        // w rows c0 .. c0+255, elements h0 .. h0+31, stored transposed as fp32
        const int e = c0 + tid;
        if (e < E) {
          const u32x4 *src = (const u32x4 *)(w + (size_t)e * H + h0);
#pragma unroll
          for (int q = 0; q < kSub / 8; ++q) {
            const u32x4 p = src[q];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              wsm[q * 8 + 2 * r][tid] = bf16lo(p[r]);
              wsm[q * 8 + 2 * r + 1][tid] = bf16hi(p[r]);
            }
          }
        } else {
#pragma unroll
          for (int q = 0; q < kSub; ++q) wsm[q][tid] = 0.f;
        }
        if (tid < kTileT * (kSub / 8)) {
          const int t = tid / (kSub / 8), q = tid % (kSub / 8);
          const int tg = t_base + t;
          u32x4 p = {0u, 0u, 0u, 0u};
          if (tg < T) p = *(const u32x4 *)(x + (size_t)tg * H + h0 + q * 8);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            xs[q * 8 + 2 * r][t] = bf16lo(p[r]);
            xs[q * 8 + 2 * r + 1][t] = bf16hi(p[r]);
          }
        }
      }
      __syncthreads();
      for (int i = 0; i < kSub; ++i) {
        const f32x4 xv = *(const f32x4 *)&xs[i][4 * ty];
        float wv[4];
#pragma unroll
        for (int b = 0; b < 4; ++b) wv[b] = wsm[i][tx + 64 * b];
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
          for (int b = 0; b < 4; ++b) acc[a][b] = __builtin_fmaf(xv[a], wv[b], acc[a][b]);
        if (++in_slice == L) {
          // Slice s is complete.  Merge it into the carry stack: lev = number
          // of trailing one bits of s = number of left siblings waiting.
          int lev = 0;
          while (lev < 6 && ((s >> lev) & 1)) ++lev;
#pragma unroll
          for (int a = 0; a < 4; ++a)
#pragma unroll
            for (int b = 0; b < 4; ++b) {
              float v = acc[a][b];
#pragma unroll
              for (int q = 0; q < 6; ++q)
                if (q < lev) v = lvl[q][a][b] + v;  // left subtree + right subtree
#pragma unroll
              for (int q = 0; q < 6; ++q)
                if (q == lev) lvl[q][a][b] = v;
              acc[a][b] = (lev == 6) ? v : 0.f;   // lev == 6 only after slice 63
            }
          in_slice = 0;
          ++s;
        }
      }
    }
    // acc holds the tree value of every output
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const int e = c0 + tx + 64 * b;
        if (e < E) {
          const float lv = acc[a][b] + (bias ? bias[e] : 0.f);
          lgs[(4 * ty + a) * E + e] = lv;
          const int tg = t_base + 4 * ty + a;
          if (lg_out && tg < T) lg_out[(size_t)tg * E + e] = lv;
        }
      }
  }
  __syncthreads();
  const int wave = tid / kWave;
  for (int t = wave; t < kTileT; t += 4) {
    const int tg = t_base + t;
    if (tg < T) {
      const float *row = lgs + t * E;
      topk_softmax_any(
          [&](auto &v) {
            constexpr int NV = sizeof(v) / sizeof(v[0]);
#pragma unroll
            for (int j = 0; j < NV; ++j) {
              const int ee = lane_id() + kWave * j;
              v[j] = ee < E ? row[ee] : 0.f;
            }
          },
          E, k, ids + (size_t)tg * k, gates + (size_t)tg * k);
    }
  }
}

// ------------------------------------------------------------ large T, H % 2048 == 0
// 16 tokens x 256 experts per pass with 512 threads (two waves per SIMD):
// thread (ty, tx) of wave w owns tokens 4 (w % 4) .. +3 and experts
// c0 + 128 (w / 4) + 2 tx, +1.  32-h chunks of x and w are converted to
// float32 into LDS once per block; the next chunk is fetched into registers
// while the current one is consumed; each h's operands are read from LDS one
// step ahead of their use.  A slice ends on a chunk boundary (L % 32 == 0), so
// the carry merge is a uniform switch outside the unrolled h loop.
constexpr int kHC = 32;  // h per LDS chunk
typedef float f32x2 __attribute__((ext_vector_type(2)));

template <int LEV, int N>
__device__ __forceinline__ void carry_merge(float (&lvl)[6][N], float (&acc)[N]) {
#pragma unroll
  for (int i = 0; i < N; ++i) {
    float v = acc[i];
#pragma unroll
    for (int q = 0; q < LEV; ++q) v = lvl[q][i] + v;  // left subtree + right subtree
    if constexpr (LEV < 6) {
      lvl[LEV][i] = v;
      acc[i] = 0.f;
    } else {
      acc[i] = v;
    }
  }
}

__global__ void __launch_bounds__(512) route_tiled2_kernel(const uint16_t *__restrict__ x,
                                                           const uint16_t *__restrict__ w, const float *bias,
                                                           int T, int H, int E, int k, int32_t *ids, float *gates,
                                                           float *lg_out) {
  __shared__ __attribute__((aligned(16))) float xs[kHC][kTileT];
  __shared__ __attribute__((aligned(16))) float wsm[kHC][256];
  extern __shared__ __attribute__((aligned(16))) float lgs[];  // [kTileT][E]
  const int tid = threadIdx.x;
  const int wave = tid / kWave, tx = tid % kWave;
  const int tq = wave % 4, eh = wave / 4;  // token quad, expert half
  const int t_base = blockIdx.x * kTileT;
  const int cps = H / 64 / kHC;  // chunks per slice
  const int nch = H / kHC;
  // staging: thread tid converts 16 h of expert row c0 + tid / 2; threads
  // < 64 one 8-h piece of token tid / 4
  const int xt = t_base + (tid >> 2);
  const bool xvalid = tid < 64 && xt < T;
  const u32x4 *xrow = (const u32x4 *)(x + (size_t)min(xt, T - 1) * H) + (tid & 3);
  const int we = tid >> 1, wh = tid & 1;

  for (int c0 = 0; c0 < E; c0 += 256) {
    const bool wvalid = c0 + we < E;
    const u32x4 *wrow = (const u32x4 *)(w + (size_t)min(c0 + we, E - 1) * H) + 2 * wh;
    u32x4 pw[2], px = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int q = 0; q < 2; ++q) pw[q] = wrow[q];
    if (tid < 64) px = xrow[0];
    float acc[8], lvl[6][8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = 0.f;
    int s = 0;
    const float *xsp = &xs[0][4 * tq];
    const float *wsp = &wsm[0][128 * eh + 2 * tx];
    for (int ch = 0; ch < nch; ++ch) {
      __syncthreads();  // the previous chunk has been consumed
#pragma unroll
      for (int q = 0; q < 2; ++q)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int h = wh * 16 + q * 8 + 2 * r;
          wsm[h][we] = wvalid ? bf16lo(pw[q][r]) : 0.f;
          wsm[h + 1][we] = wvalid ? bf16hi(pw[q][r]) : 0.f;
        }
      if (tid < 64)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          xs[(tid & 3) * 8 + 2 * r][tid >> 2] = xvalid ? bf16lo(px[r]) : 0.f;
          xs[(tid & 3) * 8 + 2 * r + 1][tid >> 2] = xvalid ? bf16hi(px[r]) : 0.f;
        }
      __syncthreads();
      if (ch + 1 < nch) {
#pragma unroll
        for (int q = 0; q < 2; ++q) pw[q] = wrow[(ch + 1) * 4 + q];
        if (tid < 64) px = xrow[(ch + 1) * 4];
      }
      f32x4 xv = *(const f32x4 *)xsp;
      f32x2 wv = *(const f32x2 *)wsp;
#pragma unroll
      for (int i = 0; i < kHC; ++i) {
        f32x4 xn;
        f32x2 wn;
        if (i + 1 < kHC) {
          xn = *(const f32x4 *)(xsp + (i + 1) * kTileT);
          wn = *(const f32x2 *)(wsp + (i + 1) * 256);
        }
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
          for (int b = 0; b < 2; ++b) acc[a * 2 + b] = __builtin_fmaf(xv[a], wv[b], acc[a * 2 + b]);
        if (i + 1 < kHC) {
          xv = xn;
          wv = wn;
        }
      }
      if ((ch + 1) % cps == 0) {
        // slice s is complete: lev = trailing one bits of s = left siblings waiting
        switch (__builtin_ctz(~(unsigned)s)) {
          case 0: carry_merge<0>(lvl, acc); break;
          case 1: carry_merge<1>(lvl, acc); break;
          case 2: carry_merge<2>(lvl, acc); break;
          case 3: carry_merge<3>(lvl, acc); break;
          case 4: carry_merge<4>(lvl, acc); break;
          case 5: carry_merge<5>(lvl, acc); break;
          default: carry_merge<6>(lvl, acc); break;  // after slice 63
        }
        ++s;
      }
    }
    // acc holds the tree value of every output
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        const int e = c0 + 128 * eh + 2 * tx + b;
        if (e < E) {
          const float lv = acc[a * 2 + b] + (bias ? bias[e] : 0.f);
          lgs[(4 * tq + a) * E + e] = lv;
          const int tg = t_base + 4 * tq + a;
          if (lg_out && tg < T) lg_out[(size_t)tg * E + e] = lv;
        }
      }
  }
  __syncthreads();
  for (int t = wave; t < kTileT; t += 8) {
    const int tg = t_base + t;
    if (tg < T) {
      const float *row = lgs + t * E;
      topk_softmax_any(
          [&](auto &v) {
            constexpr int NV = sizeof(v) / sizeof(v[0]);
#pragma unroll
            for (int j = 0; j < NV; ++j) {
              const int ee = lane_id() + kWave * j;
              v[j] = ee < E ? row[ee] : 0.f;
            }
          },
          E, k, ids + (size_t)tg * k, gates + (size_t)tg * k);
    }
  }
}

// ------------------------------------------------------------ 32 < T <= 1024, H % 2048 == 0
// Logits and top-k as two launches, so that a batch spreads over
// (T / (4 TPW)) x (E / 64) x KS blocks instead of one block per 16 tokens:
//  * route_tiles_kernel: block (token tile, expert group, K part); wave w owns
//    tokens 4 TPW b + TPW w .. + TPW - 1 (its x operand is one broadcast LDS
//    read), lane l owns expert 64 g + l; K part p covers slices
//    [64 p / KS, 64 (p + 1) / KS), an aligned subtree of the slice tree.
//    32-h chunks of x and w are converted to float32 into LDS; each thread
//    keeps the next kPre chunks' loads in flight, so the wait for a chunk is
//    covered by the work on the kPre before it.  Same order as
//    above (slice chains, carry merge at each slice end), so each part ends
//    with its subtree sum, bit-identical to that node of the full tree.
//  * route_topk_kernel: one wave per token combines the KS subtree sums in
//    tree order, adds the bias (the logits, written out if asked for), runs
//    the top-k and softmax, and clears the partial sums in the workspace.
constexpr int kPre = 8;  // chunks of x and w in flight per thread (a part has a multiple of 8 chunks)
template <int TPW, int KS>
__global__ void __launch_bounds__(256) route_tiles_kernel(const uint16_t *__restrict__ x,
                                                          const uint16_t *__restrict__ w, int T, int H, int E,
                                                          float *part) {
  constexpr int TT = 4 * TPW;  // tokens per block
  constexpr int SUB = KS == 1 ? 6 : KS == 2 ? 5 : 4;  // tree level of a part's subtree
  __shared__ __attribute__((aligned(16))) float xs[kHC][TT];
  __shared__ __attribute__((aligned(16))) float wsm[kHC][kWave];
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  const int ngrp = (E + kWave - 1) / kWave;
  const int kp = blockIdx.x % KS, tile = blockIdx.x / KS;
  const int t_base = (tile / ngrp) * TT, e0 = (tile % ngrp) * kWave;
  const int cps = H / 64 / kHC;  // chunks per slice
  const int nch = H / KS / kHC;  // chunks of this part
  const int h0 = kp * (H / KS);
  // staging: thread tid converts 8 h of expert row e0 + tid / 4; threads
  // < 4 TT one 8-h piece of token tid / 4
  const int we = tid >> 2, wq = tid & 3;
  const bool wvalid = e0 + we < E;
  const u32x4 *wrow = (const u32x4 *)(w + (size_t)min(e0 + we, E - 1) * H + h0) + wq;
  const int xt = t_base + (tid >> 2);
  const bool xload = tid < 4 * TT, xvalid = xload && xt < T;
  const u32x4 *xrow = (const u32x4 *)(x + (size_t)min(xt, T - 1) * H + h0) + wq;
  // kPre chunks in flight: chunk c sits in register stage c % kPre, so the
  // loop below is unrolled by kPre and every stage index is a constant
  u32x4 pw[kPre], px[kPre];
#pragma unroll
  for (int j = 0; j < kPre; ++j) {
    pw[j] = wrow[j * 4];
    px[j] = xload ? xrow[j * 4] : u32x4{0u, 0u, 0u, 0u};
  }
  float acc[TPW], lvl[6][TPW];
#pragma unroll
  for (int i = 0; i < TPW; ++i) acc[i] = 0.f;
  int s = 0;
  const float *xsp = &xs[0][TPW * wave];
  const float *wsp = &wsm[0][lane];
  for (int c0 = 0; c0 < nch; c0 += kPre) {
#pragma unroll
    for (int j = 0; j < kPre; ++j) {
      const int ch = c0 + j;
      __syncthreads();  // the previous chunk has been consumed
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        wsm[wq * 8 + 2 * r][we] = wvalid ? bf16lo(pw[j][r]) : 0.f;
        wsm[wq * 8 + 2 * r + 1][we] = wvalid ? bf16hi(pw[j][r]) : 0.f;
      }
      if (xload)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          xs[wq * 8 + 2 * r][tid >> 2] = xvalid ? bf16lo(px[j][r]) : 0.f;
          xs[wq * 8 + 2 * r + 1][tid >> 2] = xvalid ? bf16hi(px[j][r]) : 0.f;
        }
      __syncthreads();
      if (ch + kPre < nch) {
        pw[j] = wrow[(ch + kPre) * 4];
        if (xload) px[j] = xrow[(ch + kPre) * 4];
      }
#pragma unroll
      for (int i = 0; i < kHC; ++i) {
        const float wv = wsp[i * kWave];
        if constexpr (TPW == 4) {
          const f32x4 xv = *(const f32x4 *)(xsp + i * TT);
#pragma unroll
          for (int a = 0; a < 4; ++a) acc[a] = __builtin_fmaf(xv[a], wv, acc[a]);
        } else {
          const f32x2 xv = *(const f32x2 *)(xsp + i * TT);
#pragma unroll
          for (int a = 0; a < TPW; ++a) acc[a] = __builtin_fmaf(xv[a], wv, acc[a]);
        }
      }
      if ((ch + 1) % cps == 0) {
        // slice s (of this part) is complete: lev = trailing one bits of s
        switch (__builtin_ctz(~(unsigned)s)) {
          case 0: carry_merge<0>(lvl, acc); break;
          case 1: carry_merge<1>(lvl, acc); break;
          case 2: carry_merge<2>(lvl, acc); break;
          case 3: carry_merge<3>(lvl, acc); break;
          case 4: carry_merge<4>(lvl, acc); break;
          case 5: carry_merge<5>(lvl, acc); break;
          default: carry_merge<6>(lvl, acc); break;  // after slice 63
        }
        ++s;
      }
    }
  }
  // the part's subtree sum: the root (acc) for one part, else its top carry level
  const int e = e0 + lane;
  if (e < E) {
#pragma unroll
    for (int a = 0; a < TPW; ++a) {
      const int t = t_base + TPW * wave + a;
      if (t < T) part[((size_t)kp * T + t) * E + e] = SUB == 6 ? acc[a] : lvl[SUB < 6 ? SUB : 0][a];
    }
  }
}

template <int KS>
__global__ void __launch_bounds__(256) route_topk_kernel(float *part, const float *bias, float *lg_out, int T, int E,
                                                         int k, int32_t *ids, float *gates) {
  const int t = blockIdx.x * 4 + threadIdx.x / kWave;
  if (t >= T) return;  // wave-uniform
  topk_softmax_any(
      [&](auto &v) {
        constexpr int NV = sizeof(v) / sizeof(v[0]);
#pragma unroll
        for (int j = 0; j < NV; ++j) {
          const int ee = lane_id() + kWave * j;
          v[j] = 0.f;
          if (ee < E) {
            float p[KS];
#pragma unroll
            for (int q = 0; q < KS; ++q) {
              float *pp = part + ((size_t)q * T + t) * E + ee;
              p[q] = *pp;
              *pp = 0.f;  // the partial sums live in the workspace
            }
            float l = p[0];
            if constexpr (KS == 2) l = p[0] + p[1];
            if constexpr (KS == 4) l = (p[0] + p[1]) + (p[2] + p[3]);
            l = l + (bias ? bias[ee] : 0.f);
            if (lg_out) lg_out[(size_t)t * E + ee] = l;
            v[j] = l;
          }
        }
      },
      E, k, ids + (size_t)t * k, gates + (size_t)t * k);
}

}  // namespace

// Batches of 32 < T <= 1024 tokens (with H % 2048 == 0) run the logits as
// tiles of tokens x 64 experts x K parts plus a top-k launch; the partial
// sums live in the workspace.
constexpr int kRouteTilesMinT = 32, kRouteTilesMaxT = 1024;
static bool route_tiles(int T, int H) {
  return T > kRouteTilesMinT && T <= kRouteTilesMaxT && H % (64 * kHC) == 0;  // slices of whole chunks
}
constexpr int kRouteKS = 4;  // K parts (subtrees of 16 slices)

size_t route_workspace_bytes(int T, int E) {
  size_t b = kCtlBytes;
  if (T <= kRouteSmallT) b += (size_t)T * E * sizeof(uint64_t);  // tagged logits
  if (T > kRouteTilesMinT && T <= kRouteTilesMaxT) {              // partial sums of the tiled launch
    const size_t l = kCtlBytes + (size_t)kRouteKS * T * E * sizeof(float);
    if (l > b) b = l;
  }
  return b;
}

// The LDS-staged small router: H a power of two from 512 to 4096, and its
// LDS (six padded rows plus the grouping arrays) within 64 KiB.
static bool small_lds_ok(int T, int H, int E) {
  (void)T;
  return router_lds_ok(H) && kLdsRows * router_lds_row_bytes(H) + (size_t)(kFusedRows + E) * sizeof(int) <= 64 * 1024;
}

template <bool GROUP>
static void launch_route_small(const uint16_t *x, const uint16_t *w_router, const float *bias, int T, int H, int E,
                               int k, int32_t *ids, float *gates, float *logits, void *ws, const GroupOut &go,
                               hipStream_t st) {
  int *ctl = (int *)ws;
  uint64_t *tl = (uint64_t *)((char *)ws + kCtlBytes);
  const int L = H / 64;
  const int spins = wait_spin_limit();
  const size_t glds = GROUP ? (size_t)(kFusedRows + E) * sizeof(int) : 0;
  if (small_lds_ok(T, H, E)) {
    const int tiles = ((E + kLdsExperts - 1) / kLdsExperts) * ((T + kLdsTokens - 1) / kLdsTokens);
    const int nsel = T < E ? T : E;
    route_small_lds_kernel<GROUP><<<dim3((unsigned)(tiles > nsel ? tiles : nsel)), 256,
                                    kLdsRows * router_lds_row_bytes(H) + glds, st>>>(
        x, w_router, bias, T, H, E, k, ids, gates, tl, logits, ctl, spins, go);
    return;
  }
  // one wave per kTB tokens, up to kSmallMaxWaves
  const int nw = min(kSmallMaxWaves, (T + kTB - 1) / kTB);
  dim3 grid(E), block(kWave * nw);
  const size_t lds = glds;
  if (L % 8 == 0)
    route_small_kernel<8, GROUP><<<grid, block, lds, st>>>(x, w_router, bias, T, H, E, k, ids, gates, tl, logits,
                                                           ctl, spins, go);
  else if (L % 4 == 0)
    route_small_kernel<4, GROUP><<<grid, block, lds, st>>>(x, w_router, bias, T, H, E, k, ids, gates, tl, logits,
                                                           ctl, spins, go);
  else
    route_small_kernel<2, GROUP><<<grid, block, lds, st>>>(x, w_router, bias, T, H, E, k, ids, gates, tl, logits,
                                                           ctl, spins, go);
}

bool route_groups_rows(int T, int k) { return T <= kRouteSmallT && T * k <= kFusedRows; }

hipError_t launch_route_group(const uint16_t *x, const uint16_t *w_router, const float *bias, int T, int H, int E,
                              int k, int32_t *ids, float *gates, float *logits, int32_t *offsets,
                              int32_t *sorted_rows, int32_t *row_pos, int32_t *active, void *ws, hipStream_t st) {
  const int n = T * k;
  const GroupOut go{offsets, sorted_rows, row_pos, active, 1 + (E < n ? E : n)};
  launch_route_small<true>(x, w_router, bias, T, H, E, k, ids, gates, logits, ws, go, st);
  return hipGetLastError();
}

hipError_t launch_route(const uint16_t *x, const uint16_t *w_router, const float *bias, int T, int H, int E,
                        int k, int32_t *ids, float *gates, float *logits, void *ws, hipStream_t st) {
  if (route_tiles(T, H)) {
    float *part = (float *)((char *)ws + kCtlBytes);
    const int ngrp = (E + kWave - 1) / kWave;
    route_tiles_kernel<2, kRouteKS><<<dim3((unsigned)(((T + 7) / 8) * ngrp * kRouteKS)), 256, 0, st>>>(
        x, w_router, T, H, E, part);
    route_topk_kernel<kRouteKS><<<dim3((unsigned)((T + 3) / 4)), 256, 0, st>>>(part, bias, logits, T, E, k, ids,
                                                                               gates);
  } else if (T <= kRouteSmallT) {
    launch_route_small<false>(x, w_router, bias, T, H, E, k, ids, gates, logits, ws, GroupOut{}, st);
  } else {
    dim3 grid((T + kTileT - 1) / kTileT), block(256);
    if (H % (64 * kHC) == 0)
      route_tiled2_kernel<<<grid, dim3(512), (size_t)kTileT * E * sizeof(float), st>>>(x, w_router, bias, T, H, E, k,
                                                                                        ids, gates, logits);
    else
      route_tiled_kernel<<<grid, block, (size_t)kTileT * E * sizeof(float), st>>>(x, w_router, bias, T, H, E, k, ids,
                                                                                   gates, logits);
  }
  return hipGetLastError();
}

}  // namespace bqmoe
