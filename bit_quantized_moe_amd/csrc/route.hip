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

namespace bqmoe {
namespace {

constexpr int kMaxE = 1024;
constexpr int kMaxK = 32;

// ------------------------------------------------------------ top-k of one token
// One wave selects the k largest of lg[0..E) (ties: lower index first) and
// writes ids / softmax gates.  COHERENT: lg is global memory written by other
// blocks of this kernel, read with device-coherent loads; otherwise lg is LDS.
template <bool COHERENT>
__device__ void topk_softmax_wave(const float *lg, int E, int k, int32_t *ids_out, float *g_out) {
  const int lane = lane_id();
  float v[kMaxE / kWave];
#pragma unroll
  for (int j = 0; j < kMaxE / kWave; ++j) {
    const int e = lane + kWave * j;
    if constexpr (COHERENT)
      v[j] = (e < E) ? __hip_atomic_load(lg + e, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : -INFINITY;
    else
      v[j] = (e < E) ? lg[e] : -INFINITY;
  }
  uint32_t used = 0;
  int my_e = 0;
  float my_v = 0.f;
  for (int slot = 0; slot < k; ++slot) {
    float bv = -INFINITY;
    int be = 0x7fffffff;
#pragma unroll
    for (int j = 0; j < kMaxE / kWave; ++j) {
      const int e = lane + kWave * j;
      const bool ok = (e < E) && !((used >> j) & 1u);
      if (ok && (v[j] > bv || (v[j] == bv && e < be))) {
        bv = v[j];
        be = e;
      }
    }
#pragma unroll
    for (int d = kWave / 2; d >= 1; d >>= 1) {
      const float ov = __shfl_xor(bv, d, kWave);
      const int oe = __shfl_xor(be, d, kWave);
      if (ov > bv || (ov == bv && oe < be)) {
        bv = ov;
        be = oe;
      }
    }
    if (be == 0x7fffffff) be = slot % E;  // only reachable with non-finite logits
    if ((be % kWave) == lane) used |= 1u << (be / kWave);
    if (lane == slot) {
      my_e = be;
      my_v = bv;
    }
  }
  const float m = __shfl(my_v, 0, kWave);
  const float ex = (lane < k) ? expf(my_v - m) : 0.f;
  const float sum = wave_sum_xor(ex, kWave);
  if (lane < k) {
    ids_out[lane] = my_e;
    g_out[lane] = ex / sum;
  }
}

// ------------------------------------------------------------ small T
// Grid: ceil(E/4) blocks of 4 waves; wave -> one expert, lane s -> slice s.
// The last block to finish runs top-k for every token.
__device__ __forceinline__ void bf16x8_to_f32(const u32x4 &p, float *f) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    f[2 * q] = bf16lo(p[q]);
    f[2 * q + 1] = bf16hi(p[q]);
  }
}

template <int VEC>  // bf16 elements per load: 8 (16 B), 4 (8 B) or 2 (4 B)
__global__ void __launch_bounds__(256) route_small_kernel(const uint16_t *__restrict__ x,
                                                          const uint16_t *__restrict__ w, const float *bias,
                                                          int T, int H, int E, int k, int32_t *ids,
                                                          float *gates, float *lg, int *ctl) {
  constexpr int MAXP = 8;  // 16-byte slice pieces held in registers (L <= 64)
  const int wave = threadIdx.x / kWave;
  const int lane = lane_id();
  const int e = blockIdx.x * 4 + wave;
  const int L = H / 64;
  if (e < E) {
    const uint16_t *wrow = w + (size_t)e * H + (size_t)lane * L;
    const float b = bias ? bias[e] : 0.f;
    if (VEC == 8 && L <= 8 * MAXP) {
      // the whole slice of w and of one token's x in registers, all loads in flight together
      const int np = L / 8;
      u32x4 wp[MAXP];
#pragma unroll
      for (int q = 0; q < MAXP; ++q)
        if (q < np) wp[q] = *(const u32x4 *)(wrow + 8 * q);
      for (int t = 0; t < T; ++t) {
        const uint16_t *xr = x + (size_t)t * H + (size_t)lane * L;
        u32x4 xp[MAXP];
#pragma unroll
        for (int q = 0; q < MAXP; ++q)
          if (q < np) xp[q] = *(const u32x4 *)(xr + 8 * q);
        float acc = 0.f;
#pragma unroll
        for (int q = 0; q < MAXP; ++q)
          if (q < np) {
            float xf[8], wf[8];
            bf16x8_to_f32(xp[q], xf);
            bf16x8_to_f32(wp[q], wf);
#pragma unroll
            for (int r = 0; r < 8; ++r) acc = __builtin_fmaf(xf[r], wf[r], acc);  // ascending h
          }
        const float sum = wave_tree_sum(acc);  // pairwise tree over the 64 slice sums
        if (lane == 0)
          __hip_atomic_store(lg + (size_t)t * E + e, sum + b, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    } else {
      for (int t0 = 0; t0 < T; t0 += 4) {
        float acc[4] = {0.f, 0.f, 0.f, 0.f};
        for (int i = 0; i < L; i += VEC) {
          float wf[VEC];
          if constexpr (VEC == 8) {
            bf16x8_to_f32(*(const u32x4 *)(wrow + i), wf);
          } else if constexpr (VEC == 4) {
            const u32x2 pw = *(const u32x2 *)(wrow + i);
            wf[0] = bf16lo(pw[0]);
            wf[1] = bf16hi(pw[0]);
            wf[2] = bf16lo(pw[1]);
            wf[3] = bf16hi(pw[1]);
          } else {
            const uint32_t pw = *(const uint32_t *)(wrow + i);
            wf[0] = bf16lo(pw);
            wf[1] = bf16hi(pw);
          }
#pragma unroll
          for (int tt = 0; tt < 4; ++tt) {
            if (t0 + tt < T) {
              const uint16_t *xr = x + (size_t)(t0 + tt) * H + (size_t)lane * L + i;
              float xf[VEC];
              if constexpr (VEC == 8) {
                bf16x8_to_f32(*(const u32x4 *)xr, xf);
              } else if constexpr (VEC == 4) {
                const u32x2 px = *(const u32x2 *)xr;
                xf[0] = bf16lo(px[0]);
                xf[1] = bf16hi(px[0]);
                xf[2] = bf16lo(px[1]);
                xf[3] = bf16hi(px[1]);
              } else {
                const uint32_t px = *(const uint32_t *)xr;
                xf[0] = bf16lo(px);
                xf[1] = bf16hi(px);
              }
#pragma unroll
              for (int q = 0; q < VEC; ++q) acc[tt] = __builtin_fmaf(xf[q], wf[q], acc[tt]);
            }
          }
        }
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
          const float sum = wave_tree_sum(acc[tt]);  // pairwise tree over the 64 slice sums
          if (lane == 0 && t0 + tt < T)
            __hip_atomic_store(lg + (size_t)(t0 + tt) * E + e, sum + b, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
      }
    }
  }
  // The last block to finish selects the experts of every token.  Logits were
  // stored device-coherently; each wave waits for its stores before the block
  // is counted, and the last block reads them back device-coherently.
  __shared__ int s_last;
  wait_vmem();
  __syncthreads();
  if (threadIdx.x == 0) {
    const int prev = atomicAdd(&ctl[kCtlRouteDone], 1);
    s_last = (prev == (int)gridDim.x - 1);
  }
  __syncthreads();
  if (!s_last) return;
  for (int t = wave; t < T; t += 4)
    topk_softmax_wave<true>(lg + (size_t)t * E, E, k, ids + (size_t)t * k, gates + (size_t)t * k);
  if (threadIdx.x == 0) __hip_atomic_store(&ctl[kCtlRouteDone], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
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
    if (tg < T) topk_softmax_wave<false>(lgs + t * E, E, k, ids + (size_t)tg * k, gates + (size_t)tg * k);
  }
}

}  // namespace

size_t route_workspace_bytes(int T, int E) {
  size_t b = kCtlBytes;
  if (T <= kRouteSmallT) b += (size_t)T * E * sizeof(float);
  return b;
}

hipError_t launch_route(const uint16_t *x, const uint16_t *w_router, const float *bias, int T, int H, int E,
                        int k, int32_t *ids, float *gates, float *logits, void *ws, hipStream_t st) {
  int *ctl = (int *)ws;
  if (T <= kRouteSmallT) {
    float *lg = logits ? logits : (float *)((char *)ws + kCtlBytes);
    const int L = H / 64;
    dim3 grid((E + 3) / 4), block(256);
    if (L % 8 == 0)
      route_small_kernel<8><<<grid, block, 0, st>>>(x, w_router, bias, T, H, E, k, ids, gates, lg, ctl);
    else if (L % 4 == 0)
      route_small_kernel<4><<<grid, block, 0, st>>>(x, w_router, bias, T, H, E, k, ids, gates, lg, ctl);
    else
      route_small_kernel<2><<<grid, block, 0, st>>>(x, w_router, bias, T, H, E, k, ids, gates, lg, ctl);
  } else {
    dim3 grid((T + kTileT - 1) / kTileT), block(256);
    route_tiled_kernel<<<grid, block, (size_t)kTileT * E * sizeof(float), st>>>(x, w_router, bias, T, H, E, k, ids,
                                                                                 gates, logits);
  }
  return hipGetLastError();
}

}  // namespace bqmoe
