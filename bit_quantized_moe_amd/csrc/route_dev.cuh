// Device-side pieces of the router shared by the router kernels and the fused
// decode-layer kernel: the fixed-order logit of one expert computed by one
// wave, the top-k + softmax of one token by one wave, and the stable grouping
// of routed rows by expert by one wave.  See route.hip for the summation order.
#pragma once

#include <math.h>

#include "common.cuh"

namespace bqmoe {
namespace {

// ------------------------------------------------------------ top-k of one token
// Selection order: logit descending, then expert index ascending.  A logit
// becomes an order-preserving uint32 key (with -0 folded into +0, so equal
// floats give equal keys; every finite logit gives a key above 0).  Each
// slot takes the wave maximum of the keys, then the lowest expert index that
// holds it (from one ballot per value a lane holds), and zeroes that key.
__device__ __forceinline__ uint32_t ord_key(float v) {
  const uint32_t b = __builtin_bit_cast(uint32_t, v + 0.0f);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
__device__ __forceinline__ float key_value(uint32_t u) {
  return __builtin_bit_cast(float, (u & 0x80000000u) ? (u & 0x7fffffffu) : ~u);
}
#define BQ_DPP_U32(v, ctrl) ((uint32_t)__builtin_amdgcn_update_dpp(0, (int)(v), (ctrl), 0xF, 0xF, false))
// Maximum over the 64 lanes (wave-uniform): four in-row DPP steps, then the
// four row maxima from readlanes.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, BQ_DPP_U32(v, 0xB1));   // quad_perm [1,0,3,2]
  v = max(v, BQ_DPP_U32(v, 0x4E));   // quad_perm [2,3,0,1]
  v = max(v, BQ_DPP_U32(v, 0x141));  // row_half_mirror
  v = max(v, BQ_DPP_U32(v, 0x140));  // row_mirror
  const uint32_t r0 = __builtin_amdgcn_readlane((int)v, 0), r1 = __builtin_amdgcn_readlane((int)v, 16);
  const uint32_t r2 = __builtin_amdgcn_readlane((int)v, 32), r3 = __builtin_amdgcn_readlane((int)v, 48);
  return max(max(r0, r1), max(r2, r3));
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
  uint32_t my_key = 0;
  int my_e = 0;
  for (int slot = 0; slot < k; ++slot) {
    uint32_t mx = key[0];
#pragma unroll
    for (int j = 1; j < NV; ++j) mx = max(mx, key[j]);
    mx = wave_max_u32(mx);
    // lowest expert index with the maximum: the first j whose ballot is not
    // empty, at its lowest lane
    int be = 0;
#pragma unroll
    for (int j = NV - 1; j >= 0; --j) {
      const uint64_t b = __ballot(key[j] == mx);
      if (b) be = kWave * j + (__ffsll((unsigned long long)b) - 1);
    }
    be = min(be, E - 1);  // only reachable with non-finite logits (key 0): ids stay valid experts
#pragma unroll
    for (int j = 0; j < NV; ++j)
      if (lane + kWave * j == be) key[j] = 0u;
    if (lane == slot) {
      my_e = be;
      my_key = mx;
    }
  }
  const float mine = key_value(my_key);
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

// One wave computes the logits of expert e for tokens 0..T-1 (lane s sums
// slice s of H/64 elements in ascending h, then the 64 slice sums are combined
// as a balanced pairwise tree, then the bias is added) and stores each as a
// tagged 64-bit word tl[t * E + e] with a device-coherent store.  TB tokens'
// activation slices are loaded together (register cost ~ 16 * VEC * TB / 8).
// The wave takes the groups of TB tokens g0, g0 + gs, ... (several waves of
// a block share one expert's tokens this way).
// FULL: every slice is a whole number of 64-element chunks, so the chunk
// loop needs no guards (straight-line code; branches are costly here).
template <int VEC, int TB, bool FULL>
__device__ __forceinline__ void router_logits_wave_impl(const uint16_t *__restrict__ x,
                                                        const uint16_t *__restrict__ w, const float *bias, int T,
                                                        int H, int E, int e, uint64_t *tl, int g0, int gs) {
  constexpr int NVC = 64 / VEC;  // loads per 64-element chunk of a slice
  const int lane = lane_id();
  const int L = H / 64;
  const uint16_t *wrow = w + (size_t)e * H + (size_t)lane * L;
  const float b = bias ? bias[e] : 0.f;
  for (int t0 = g0 * TB; t0 < T; t0 += gs * TB) {
    float acc[TB];
#pragma unroll
    for (int tt = 0; tt < TB; ++tt) acc[tt] = 0.f;
    const int ntt = min(TB, T - t0);
    for (int c0 = 0; c0 < L; c0 += 64) {
      const int nv = FULL ? NVC : min(64, L - c0) / VEC;
      // this chunk of the weight slice and of up to TB tokens' activation slices
      Vec<VEC> wv[NVC], xv[TB][NVC];
#pragma unroll
      for (int q = 0; q < NVC; ++q)
        if (FULL || q < nv) wv[q] = load_vec<VEC>(wrow + c0 + q * VEC);
#pragma unroll
      for (int tt = 0; tt < TB; ++tt)
        if (TB == 1 || tt < ntt) {
          const uint16_t *xr = x + (size_t)(t0 + tt) * H + (size_t)lane * L + c0;
#pragma unroll
          for (int q = 0; q < NVC; ++q)
            if (FULL || q < nv) xv[tt][q] = load_vec<VEC>(xr + q * VEC);
        }
#pragma unroll
      for (int tt = 0; tt < TB; ++tt)
        if (TB == 1 || tt < ntt) {
#pragma unroll
          for (int q = 0; q < NVC; ++q)
            if (FULL || q < nv) acc[tt] = fma_vec<VEC>(xv[tt][q], wv[q], acc[tt]);
        }
    }
#pragma unroll
    for (int tt = 0; tt < TB; ++tt) {
      const float sum = group_sum(acc[tt], kWave);  // pairwise tree over the 64 slice sums
      if (lane == 0 && t0 + tt < T)
        __hip_atomic_store(tl + (size_t)(t0 + tt) * E + e, kLogitTag | __float_as_uint(sum + b), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

template <int VEC, int TB = kTB>
__device__ __forceinline__ void router_logits_wave(const uint16_t *__restrict__ x, const uint16_t *__restrict__ w,
                                                   const float *bias, int T, int H, int E, int e, uint64_t *tl,
                                                   int g0 = 0, int gs = 1) {
  if ((H / 64) % 64 == 0)
    router_logits_wave_impl<VEC, TB, true>(x, w, bias, T, H, E, e, tl, g0, gs);
  else
    router_logits_wave_impl<VEC, TB, false>(x, w, bias, T, H, E, e, tl, g0, gs);
}

// Router logits from LDS, for H a power of two from 512 to 4096 (slices of
// L = H/64 elements, a multiple of 8).  A slice occupies L/2 words plus 4 of padding, so every
// 16-byte chunk of a row lands 16-byte aligned and lane s reads its slice with
// 16-byte LDS loads.  The global reads are then fully coalesced (one 1 KB
// stretch per load instruction), where slice-per-lane global loads touch 64
// lines per instruction and take several times longer.
__device__ __forceinline__ int router_slice_words(int H) { return H / 128 + 4; }
__host__ __device__ __forceinline__ size_t router_lds_row_bytes(int H) { return (size_t)64 * (H / 128 + 4) * 4; }
// The fused layer's LDS router: the activation row plus two weight rows (a
// block takes two experts; two waves load each row, one wave runs its dot).
__host__ __device__ __forceinline__ bool router_lds_ok(int H) {
  return H >= 512 && H <= 4096 && (H & (H - 1)) == 0;
}
__host__ __device__ __forceinline__ size_t router_lds_bytes(int H) { return 3 * router_lds_row_bytes(H); }

// Chunks [c0, c1) (8 elements each) of a bf16 row of H elements into dst in
// the padded slice layout; thread t of nthreads loads chunks c0 + t + q * nthreads.
template <int PER>
__device__ __forceinline__ void row_to_slices(const uint16_t *__restrict__ row, int H, uint32_t *dst, int c0, int c1,
                                              int t, int nthreads) {
  const int sw = router_slice_words(H);
  const int sh = __builtin_ctz(H / 512);  // 16-byte chunks per slice = 1 << sh
  u32x4 a[PER];
  // every load is issued (threads past c1 re-read the last chunk), so they
  // are all in flight together; only the stores are guarded
#pragma unroll
  for (int q = 0; q < PER; ++q) a[q] = ((const u32x4 *)row)[min(c0 + t + q * nthreads, c1 - 1)];
#pragma unroll
  for (int q = 0; q < PER; ++q) {
    const int c = c0 + t + q * nthreads;
    if (c < c1) *(u32x4 *)&dst[(c >> sh) * sw + (c & ((1 << sh) - 1)) * 4] = a[q];
  }
}

// Two rows at once (chunk ranges of each, as above), so that both sets of
// loads are in flight together.
template <int PA, int PB>
__device__ __forceinline__ void rows_to_slices(const uint16_t *__restrict__ ra, uint32_t *da, int a0, int a1, int ta,
                                               int na, const uint16_t *__restrict__ rb, uint32_t *db, int b0, int b1,
                                               int tb, int nb, int H) {
  const int sw = router_slice_words(H);
  const int sh = __builtin_ctz(H / 512);
  u32x4 a[PA], b[PB];
#pragma unroll
  for (int q = 0; q < PA; ++q) a[q] = ((const u32x4 *)ra)[min(a0 + ta + q * na, a1 - 1)];
#pragma unroll
  for (int q = 0; q < PB; ++q) b[q] = ((const u32x4 *)rb)[min(b0 + tb + q * nb, b1 - 1)];
#pragma unroll
  for (int q = 0; q < PA; ++q) {
    const int c = a0 + ta + q * na;
    if (c < a1) *(u32x4 *)&da[(c >> sh) * sw + (c & ((1 << sh) - 1)) * 4] = a[q];
  }
#pragma unroll
  for (int q = 0; q < PB; ++q) {
    const int c = b0 + tb + q * nb;
    if (c < b1) *(u32x4 *)&db[(c >> sh) * sw + (c & ((1 << sh) - 1)) * 4] = b[q];
  }
}

// Lane s chains slice s of x . w (both in the padded layout) in ascending h,
// then the 64 slice sums are combined by the pairwise tree and the bias added.
__device__ __forceinline__ float router_dot_slices(const uint32_t *xs, const uint32_t *ws, int H, float b) {
  const int lane = lane_id();
  const int sw = router_slice_words(H);
  const uint32_t *xp = xs + lane * sw, *wp = ws + lane * sw;
  float acc = 0.f;
#pragma unroll 8
  for (int j = 0; j < H / 128; j += 4) {
    const u32x4 xx = *(const u32x4 *)(xp + j), ww = *(const u32x4 *)(wp + j);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      acc = __builtin_fmaf(bf16lo(xx[r]), bf16lo(ww[r]), acc);
      acc = __builtin_fmaf(bf16hi(xx[r]), bf16hi(ww[r]), acc);
    }
  }
  return group_sum(acc, kWave) + b;
}

// Loader (for topk_softmax_any) of one token's E tagged logit words: reads
// them with device-coherent loads until every word carries the tag, then, if
// clear, zeroes them; out (if not null) receives the float values.  A wait
// longer than max_spins sets the error flag in ctl and goes on.
struct TaggedLogits {
  uint64_t *row;
  int E, max_spins;
  int *ctl;
  bool clear;
  float *out;
  template <typename V>
  __device__ __forceinline__ void operator()(V &v) const {
    constexpr int NV = sizeof(v) / sizeof(v[0]);
    const int lane = lane_id();
    uint64_t wv[NV];
    for (int spins = 0;; ++spins) {
      bool ready = true;
#pragma unroll
      for (int j = 0; j < NV; ++j) {
        // lanes past E re-read the last word (no branch around the load)
        const int ee = lane + kWave * j;
        const uint64_t got = __hip_atomic_load(row + min(ee, E - 1), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        wv[j] = ee < E ? got : kLogitTag;
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
    for (int j = 0; j < NV; ++j) v[j] = __uint_as_float((uint32_t)wv[j]);
    // every word has been read: clear them (lanes past E clear the last word again)
    if (clear)
#pragma unroll
      for (int j = 0; j < NV; ++j)
        __hip_atomic_store(row + min(lane + kWave * j, E - 1), (uint64_t)0, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    if (out)
#pragma unroll
      for (int j = 0; j < NV; ++j)
        if (lane + kWave * j < E) out[lane + kWave * j] = v[j];
  }
};

}  // namespace
}  // namespace bqmoe
