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


// ------------------------------------------------------------ top-k of one token
// Selection order: logit descending, then expert index ascending.  A logit
// becomes an order-preserving uint32 (with -0 folded into +0, so equal floats
// give equal keys) and the pair (key, ~e) is compared as one 64-bit key, so a
// plain maximum over the wave picks the next slot.
__device__ __forceinline__ uint32_t ord_key(float v) {
  const uint32_t b = __builtin_bit_cast(uint32_t, v + 0.0f);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
__device__ __forceinline__ float key_value(uint32_t u) {
  return __builtin_bit_cast(float, (u & 0x80000000u) ? (u & 0x7fffffffu) : ~u);
}
__device__ __forceinline__ void key_max(uint32_t &hi, uint32_t &lo, uint32_t ohi, uint32_t olo) {
  const bool take = (ohi > hi) || (ohi == hi && olo > lo);
  hi = take ? ohi : hi;
  lo = take ? olo : lo;
}
#define BQ_DPP_U32(v, ctrl) ((uint32_t)__builtin_amdgcn_update_dpp(0, (int)(v), (ctrl), 0xF, 0xF, false))
// Maximum (hi, lo) over the 64 lanes, in every lane.
__device__ __forceinline__ void wave_key_max(uint32_t &hi, uint32_t &lo) {
  key_max(hi, lo, BQ_DPP_U32(hi, 0xB1), BQ_DPP_U32(lo, 0xB1));
  key_max(hi, lo, BQ_DPP_U32(hi, 0x4E), BQ_DPP_U32(lo, 0x4E));
  key_max(hi, lo, BQ_DPP_U32(hi, 0x141), BQ_DPP_U32(lo, 0x141));
  key_max(hi, lo, BQ_DPP_U32(hi, 0x140), BQ_DPP_U32(lo, 0x140));
  key_max(hi, lo, xor16_lanes(hi), xor16_lanes(lo));
  const uint32_t h0 = __builtin_amdgcn_readlane((int)hi, 0), l0 = __builtin_amdgcn_readlane((int)lo, 0);
  const uint32_t h1 = __builtin_amdgcn_readlane((int)hi, 32), l1 = __builtin_amdgcn_readlane((int)lo, 32);
  hi = h0;
  lo = l0;
  key_max(hi, lo, h1, l1);
}

// One wave selects the k largest logits and writes ids and softmax gates.
// NV = values per lane (E <= 64 * NV); load(v) fills v[j] with the logit of
// expert lane + 64 j (any value where that index is >= E).
// PUBLISH: ids are stored with device-coherent stores (read back by another
// block).  key_lds, when given, receives a copy of the ids.
template <int NV, bool PUBLISH, typename Load>
__device__ void topk_softmax_wave(Load load, int E, int k, int32_t *ids_out, float *g_out, int *key_lds) {
  const int lane = lane_id();
  float v[NV];
  load(v);
  uint32_t key[NV];
#pragma unroll
  for (int j = 0; j < NV; ++j) key[j] = (lane + kWave * j < E) ? ord_key(v[j]) : 0u;  // 0: never selected (k <= E)
  uint32_t used = 0, my_hi = 0;
  int my_e = 0;
  for (int slot = 0; slot < k; ++slot) {
    uint32_t hi = 0, lo = 0;
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      const int e = lane + kWave * j;
      if (e < E && !((used >> j) & 1u)) key_max(hi, lo, key[j], ~(uint32_t)e);
    }
    wave_key_max(hi, lo);
    const int be = (int)~lo;
    if ((be % kWave) == lane) used |= 1u << (be / kWave);
    if (lane == slot) {
      my_e = be;
      my_hi = hi;
    }
  }
  const float mine = key_value(my_hi);
  const float m = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, mine)));
  const float ex = (lane < k) ? expf(mine - m) : 0.f;
  const float sum = group_sum(ex, kWave);
  if (lane < k) {
    if constexpr (PUBLISH)
      __hip_atomic_store(ids_out + lane, my_e, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    else
      ids_out[lane] = my_e;
    g_out[lane] = ex / sum;
    if (key_lds) key_lds[lane] = my_e;
  }
}

template <bool PUBLISH = false, typename Load>
__device__ __forceinline__ void topk_softmax_any(Load load, int E, int k, int32_t *ids_out, float *g_out,
                                                 int *key_lds = nullptr) {
  if (E <= 64)
    topk_softmax_wave<1, PUBLISH>(load, E, k, ids_out, g_out, key_lds);
  else if (E <= 128)
    topk_softmax_wave<2, PUBLISH>(load, E, k, ids_out, g_out, key_lds);
  else if (E <= 256)
    topk_softmax_wave<4, PUBLISH>(load, E, k, ids_out, g_out, key_lds);
  else if (E <= 512)
    topk_softmax_wave<8, PUBLISH>(load, E, k, ids_out, g_out, key_lds);
  else
    topk_softmax_wave<16, PUBLISH>(load, E, k, ids_out, g_out, key_lds);
}

// ------------------------------------------------------------ grouping by expert
// The stable grouping of n rows by expert (the result of moe_permute), done by
// one wave in LDS: a histogram, one exclusive scan for the offsets and the
// active list, then placement of the rows 64 at a time in row order.  Within a
// batch of 64, lanes with the same key find each other by bit-plane ballots,
// so a lane's rank among them is the number of lower lanes with its key.
// key[r] is the expert of row r, or E for a dropped row; cur holds E ints.
constexpr int kFusedRows = 256;  // largest T*k grouped inside the router launch

__device__ int wave_exclusive_scan(int v, int *total) {
  const int lane = lane_id();
  int inc = v;
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    const int o = __shfl_up(inc, d, kWave);
    if (lane >= d) inc += o;
  }
  *total = __shfl(inc, kWave - 1, kWave);
  return inc - v;
}

__device__ void wave_group_rows(const int *key, int n, int E, int *cur, int32_t *offsets, int32_t *sorted_rows,
                                int32_t *row_pos, int32_t *active, int n_active_slots) {
  const int lane = lane_id();
  for (int e = lane; e < E; e += kWave) cur[e] = 0;
  __builtin_amdgcn_wave_barrier();
  for (int r = lane; r < n; r += kWave) {
    const int kk = key[r];
    if (kk < E) atomicAdd(&cur[kk], 1);
  }
  __builtin_amdgcn_wave_barrier();
  // lane owns the experts [e0, e1)
  const int seg = (E + kWave - 1) / kWave;
  const int e0 = min(E, lane * seg), e1 = min(E, e0 + seg);
  int rows = 0, acts = 0;
  for (int e = e0; e < e1; ++e) {
    const int c = cur[e];
    rows += c;
    acts += c > 0;
  }
  int n_valid = 0, n_act = 0;
  int base = wave_exclusive_scan(rows, &n_valid);
  int abase = wave_exclusive_scan(acts, &n_act);
  __builtin_amdgcn_wave_barrier();
  for (int e = e0; e < e1; ++e) {
    const int c = cur[e];
    offsets[e] = base;
    cur[e] = base;
    if (c > 0) active[1 + abase++] = e;
    base += c;
  }
  if (lane == 0) {
    offsets[E] = n_valid;
    active[0] = n_act;
  }
  for (int i = 1 + n_act + lane; i < n_active_slots; i += kWave) active[i] = -1;
  __builtin_amdgcn_wave_barrier();
  int nbits = 1;
  while ((1 << nbits) < E + 2) ++nbits;
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int rb = 0; rb < n; rb += kWave) {
    const int r = rb + lane;
    const int kk = (r < n) ? key[r] : E + 1;  // E + 1: lanes past the last row
    uint64_t peers = __ballot(1);
    for (int b = 0; b < nbits; ++b) {
      const uint64_t m = __ballot((kk >> b) & 1);
      peers &= ((kk >> b) & 1) ? m : ~m;
    }
    const int rank = __popcll(peers & below);
    if (kk < E) {
      const int pos = cur[kk] + rank;
      sorted_rows[pos] = r;
      row_pos[r] = pos;
    } else if (kk == E) {
      row_pos[r] = -1;
    }
    // every lane has read its cursor before the first lane of each key moves it
    __builtin_amdgcn_wave_barrier();
    if (rank == 0 && kk < E) cur[kk] += __popcll(peers);
    __builtin_amdgcn_wave_barrier();
  }
}

// The same grouping for n <= 64 rows, in registers: lane r holds row r's key
// (E for a dropped row, E + 1 past the last row) and every count is a loop
// over the n keys read back one lane at a time.
__device__ void wave_group_rows_small(int kr, int n, int E, int32_t *offsets, int32_t *sorted_rows, int32_t *row_pos,
                                      int32_t *active, int n_active_slots) {
  const int lane = lane_id();
  int pos = 0;
  bool first = true;  // no lower row has this key
  for (int q = 0; q < n; ++q) {
    const int kq = __builtin_amdgcn_readlane(kr, q);
    pos += (kq < kr) || (kq == kr && q < lane);
    first = first && !(kq == kr && q < lane);
  }
  if (lane < n) {
    if (kr < E) {
      sorted_rows[pos] = lane;
      row_pos[lane] = pos;
    } else {
      row_pos[lane] = -1;
    }
  }
  // heads: the first row of every expert that has rows
  const uint64_t heads = __ballot(lane < n && kr < E && first);
  const int n_act = __popcll(heads);
  for (int e = lane; e <= E; e += kWave) {
    int below = 0, act_below = 0, here = 0;
    for (int q = 0; q < n; ++q) {
      const int kq = __builtin_amdgcn_readlane(kr, q);
      below += kq < e;
      act_below += ((heads >> q) & 1ull) && kq < e;
      here += kq == e;
    }
    offsets[e] = below;
    if (e < E && here > 0) active[1 + act_below] = e;
  }
  for (int i = 1 + n_act + lane; i < n_active_slots; i += kWave) active[i] = -1;
  if (lane == 0) active[0] = n_act;
}

// ------------------------------------------------------------ small T
// Grid: E blocks of one wave; block e computes the logits of expert e for
// every token (lane s = slice s, sequential over its h) and stores each as a
// 64-bit word, the float bits under a nonzero tag, with a device-coherent
// store.  Blocks 0 .. nsel-1 (nsel = min(T, E)) run the top-k of tokens
// b, b + nsel, ...: they read the token's E words until every one carries the
// tag (each word is self-validating, so no counter and no store wait are
// needed), then clear them for the next call.  All E one-wave blocks are
// co-resident, so the wait ends; it is bounded anyway and a timeout only
// raises the error flag.
constexpr int kTB = 4;  // tokens whose activation slices are loaded together
constexpr uint64_t kLogitTag = 1ull << 32;

// VEC bf16 elements per load: 8 (16 B), 4 (8 B) or 2 (4 B); kept packed.
template <int VEC>
struct Vec {
  uint32_t u[VEC / 2];
};
template <int VEC>
__device__ __forceinline__ Vec<VEC> load_vec(const uint16_t *p) {
  Vec<VEC> r;
  if constexpr (VEC == 8) {
    const u32x4 v = *(const u32x4 *)p;
    r.u[0] = v[0], r.u[1] = v[1], r.u[2] = v[2], r.u[3] = v[3];
  } else if constexpr (VEC == 4) {
    const u32x2 v = *(const u32x2 *)p;
    r.u[0] = v[0], r.u[1] = v[1];
  } else {
    r.u[0] = *(const uint32_t *)p;
  }
  return r;
}
// acc += x . w over the VEC elements, ascending (bf16 x bf16 is exact in fp32,
// so each fma adds the exact product)
template <int VEC>
__device__ __forceinline__ float fma_vec(const Vec<VEC> &xv, const Vec<VEC> &wv, float acc) {
#pragma unroll
  for (int q = 0; q < VEC / 2; ++q) {
    acc = __builtin_fmaf(bf16lo(xv.u[q]), bf16lo(wv.u[q]), acc);
    acc = __builtin_fmaf(bf16hi(xv.u[q]), bf16hi(wv.u[q]), acc);
  }
  return acc;
}

// Outputs of the grouping by expert, when the router launch also groups the
// rows (T*k <= kFusedRows).
struct GroupOut {
  int32_t *offsets, *sorted_rows, *row_pos, *active;
  int n_active_slots;
};

template <int VEC, bool GROUP>
__global__ void __launch_bounds__(64) route_small_kernel(const uint16_t *__restrict__ x,
                                                         const uint16_t *__restrict__ w, const float *bias, int T,
                                                         int H, int E, int k, int32_t *ids, float *gates,
                                                         uint64_t *tl, float *lg_out, int *ctl, int max_spins,
                                                         GroupOut go) {
  constexpr int NVC = 64 / VEC;  // loads per 64-element chunk of a slice
  const int lane = lane_id();
  const int e = blockIdx.x;
  const int L = H / 64;
  const uint16_t *wrow = w + (size_t)e * H + (size_t)lane * L;
  const float b = bias ? bias[e] : 0.f;
  for (int t0 = 0; t0 < T; t0 += kTB) {
    float acc[kTB];
#pragma unroll
    for (int tt = 0; tt < kTB; ++tt) acc[tt] = 0.f;
    const int ntt = min(kTB, T - t0);
    for (int c0 = 0; c0 < L; c0 += 64) {
      const int nv = min(64, L - c0) / VEC;
      // this chunk of the weight slice and of up to kTB tokens' activation slices
      Vec<VEC> wv[NVC], xv[kTB][NVC];
#pragma unroll
      for (int q = 0; q < NVC; ++q)
        if (q < nv) wv[q] = load_vec<VEC>(wrow + c0 + q * VEC);
#pragma unroll
      for (int tt = 0; tt < kTB; ++tt)
        if (tt < ntt) {
          const uint16_t *xr = x + (size_t)(t0 + tt) * H + (size_t)lane * L + c0;
#pragma unroll
          for (int q = 0; q < NVC; ++q)
            if (q < nv) xv[tt][q] = load_vec<VEC>(xr + q * VEC);
        }
#pragma unroll
      for (int tt = 0; tt < kTB; ++tt)
        if (tt < ntt) {
#pragma unroll
          for (int q = 0; q < NVC; ++q)
            if (q < nv) acc[tt] = fma_vec<VEC>(xv[tt][q], wv[q], acc[tt]);
        }
    }
#pragma unroll
    for (int tt = 0; tt < kTB; ++tt) {
      const float sum = group_sum(acc[tt], kWave);  // pairwise tree over the 64 slice sums
      if (lane == 0 && t0 + tt < T)
        __hip_atomic_store(tl + (size_t)(t0 + tt) * E + e, kLogitTag | __float_as_uint(sum + b), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  const int nsel = min(T, E);
  if (e >= nsel) return;
  // Loader of token t's logits: poll the tagged words, then clear them.
  auto logits_of = [&](int t) {
    return [=](auto &v) {
      constexpr int NV = sizeof(v) / sizeof(v[0]);
      uint64_t *row = tl + (size_t)t * E;
      uint64_t wv[NV];
      for (int spins = 0;; ++spins) {
        bool ready = true;
#pragma unroll
        for (int j = 0; j < NV; ++j) {
          const int ee = lane + kWave * j;
          wv[j] = ee < E ? __hip_atomic_load(row + ee, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : kLogitTag;
          ready = ready && (wv[j] & kLogitTag);
        }
        if (__ballot(!ready) == 0) break;
        if (spins >= max_spins) {
          if (lane == 0) atomicOr(&ctl[kCtlError], 1);
          break;
        }
        __builtin_amdgcn_s_sleep(1);
      }
#pragma unroll
      for (int j = 0; j < NV; ++j) {
        const int ee = lane + kWave * j;
        v[j] = __uint_as_float((uint32_t)wv[j]);
        if (ee < E) {
          __hip_atomic_store(row + ee, (uint64_t)0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          if (lg_out) lg_out[(size_t)t * E + ee] = v[j];
        }
      }
    };
  };
  extern __shared__ int group_lds[];  // GROUP with several selectors: key[kFusedRows], then cur[E]
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

}  // namespace

size_t route_workspace_bytes(int T, int E) {
  size_t b = kCtlBytes;
  if (T <= kRouteSmallT) b += (size_t)T * E * sizeof(uint64_t);  // tagged logits
  return b;
}

template <bool GROUP>
static void launch_route_small(const uint16_t *x, const uint16_t *w_router, const float *bias, int T, int H, int E,
                               int k, int32_t *ids, float *gates, float *logits, void *ws, const GroupOut &go,
                               hipStream_t st) {
  int *ctl = (int *)ws;
  uint64_t *tl = (uint64_t *)((char *)ws + kCtlBytes);
  const int L = H / 64;
  const int spins = 1 << 22;
  dim3 grid(E), block(kWave);
  const size_t lds = GROUP ? (size_t)(kFusedRows + E) * sizeof(int) : 0;
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
  if (T <= kRouteSmallT) {
    launch_route_small<false>(x, w_router, bias, T, H, E, k, ids, gates, logits, ws, GroupOut{}, st);
  } else {
    dim3 grid((T + kTileT - 1) / kTileT), block(256);
    route_tiled_kernel<<<grid, block, (size_t)kTileT * E * sizeof(float), st>>>(x, w_router, bias, T, H, E, k, ids,
                                                                                 gates, logits);
  }
  return hipGetLastError();
}

}  // namespace bqmoe
