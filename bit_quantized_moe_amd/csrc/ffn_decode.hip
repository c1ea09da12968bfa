// Decode-path expert FFN (T <= 16 tokens): one fused kernel that streams each
// selected expert's packed weights from HBM exactly once.
//
// The pages locate the decode cost in the expert GEMV that reads each selected
// expert in place (page "Qwen3.8-Flash-Next on one 24 GB GPU", "What the
// patch does": an N-contiguous batch-1 GEMV measured at 320 GB/s in-kernel;
// page "Qwen3.8-Flash-Next FP6-INT8", "Step budget and hardware floors": the
// expert GEMV is about 6 ms of each added decode stream) and dispatch to a GEMV
// up to 16 rows (same page, "Quantization quality").  This kernel is a
// from-scratch gfx950 design on the canonical K-packed layout.
//
// Work items (a persistent grid walks them in order, phase-1 items first):
//  * phase 1, (expert, 16 gate/up row pairs): the four waves of a block split
//    the K groups of the 32 rows; every wave issues all of its weight loads
//    (one 16-byte slice per lane, row and group) before any math;
//  * phase 2, (expert, 128 down rows): each wave takes two sets of 16 rows
//    over the full K.  The weight loads are issued first, then the block
//    waits until every phase-1 item of the expert is published.
//
// The dot products run on the matrix cores: v_mfma_f32_16x16x32_bf16 with the
// expert's routed activation rows as the 16-row A operand (a row repeated when
// there are fewer) and the unpacked codes of 16 weight rows as B, so the K
// reduction happens inside the MFMA accumulation and needs no cross-lane
// shuffles.  Unpack: a code field u in the low byte under a 0x43 high byte is
// the bf16 value 128 + u.  Per 128-wide group the accumulator holds
// sum((128 + u) x), and s * (acc - (128 + zero) * sum(x)) = s * sum((u - zero) x)
// (zero = 8 for INT4 offset-binary codes).  The activations are staged in LDS
// in the K order the unpacked pairs come out in, with their per-group sums.
//
// Hand-off without cache flushes or counters on the critical path: phase 1
// writes each h value as a 32-bit word, the bf16 bits under a nonzero tag, with
// a device-coherent (sc1) store; a phase-2 block reads h with device-coherent
// loads and simply reads again until every word it needs carries the tag.
// Every word is self-validating, so no store has to be waited for and no
// counter bumped before the data can be used.  The last phase-2 item of an
// expert (a per-expert done counter on its own 128-byte line) clears the
// expert's h words, so the buffer is all-zero again when the kernel ends.  The
// grid never exceeds the co-resident block count and a block finishes all of
// its phase-1 items before its first phase-2 item, so every wait ends; the
// waits are bounded anyway and a timeout only raises an error flag.
#include <mutex>
#include <type_traits>

#include "common.cuh"
#include "gemv_ops.cuh"
#include "internal.h"
#include "route_dev.cuh"

namespace bqmoe {
namespace {

constexpr int kRows1 = 16;   // gate/up row pairs per phase-1 item
constexpr int kRows2 = 128;  // down rows per phase-2 item (two sets of 16 per wave)
constexpr int kRMax = 4;     // routed rows staged per pass when T > 1
constexpr int kRedFloats = 4 * 2 * 16 * 16;  // phase-1 cross-wave partials

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
  const uint64_t *tab;  // per-expert address table (kTabStride entries per expert) or null
  const float *g13, *g2;  // NVFP4: per-expert weight tensor scales
  float gx, gh;           // NVFP4: tensor scales of the (quantised) x and of h
  uint16_t *y_perm;
  uint32_t *hbuf;  // [T*k, I] words: kHReady | bf16 bits once written, 0 before
  int *ctl;
  int max_spins;
  // fused decode layer only
  const uint16_t *w_router;
  const float *bias;
  uint64_t *tl;         // [T, E] tagged logit words
  uint64_t *rec;        // [T * k] routing record in sorted order: kRecTag | row << 48 | id << 32 | gate bits
  uint32_t *ybuf;       // [T*k, H] words: kHReady | bf16 y_perm value once written, 0 before
  uint16_t *y;          // [T, H] bf16 out
  int32_t *ids_out;     // [T, k] or null
  float *gates_out;     // [T, k] or null
  float *logits_out;    // [T, E] or null
  uint32_t magic;  // 0x43434343 (the bf16 high byte of 128); an argument so that it sits in an SGPR
};

// Per active slot a: finished phase-2 items, on its own 128-byte line.
__device__ __forceinline__ int *done2(int *ctl, int a) { return ctl + kCtlCounters + a * kCtrStride; }
// Fused layer: blocks done with their items (so with the routing record), spread over kRoutedN lines
// after the Amax slot counters (block b counts on line b % kRoutedN).
constexpr int kRoutedN = 16;
__device__ __forceinline__ int *routed_ctr(int *ctl, int amax, int i) {
  return ctl + kCtlCounters + (amax + i) * kCtrStride;
}
// Item queues (a grid with more items than blocks): queue q hands out, in
// order, the items past the first round whose index - grid is q modulo the
// queue count; block b draws from queue b % queues (its XCD under the
// round-robin dispatch of blocks).  One counter per queue, on its own line
// after the routed counters.
constexpr int kQueues = 8;
__device__ __forceinline__ int *queue_ctr(int *ctl, int amax, int q) {
  return ctl + kCtlCounters + (amax + kRoutedN + q) * kCtrStride;
}
constexpr uint32_t kHReady = 1u << 16;  // tag of a written h word
constexpr uint64_t kRecTag = 1ull << 63;  // tag of a written routing record word

// ---------------------------------------------------------------- LDS staging
// Activation row r (K bf16) goes to LDS act + r * (K*2 + 16) in operand order,
// in chunks of 8 (INT4, INT8) or 16 (INT2) elements; its per-group sums go to
// Xs[g*16 + m] for the MFMA rows m that read it (row m reads activation row
// min(m, R-1)), g counting groups of GS.
//
// Chunks of activation row 0 that every thread loads before its weights:
// chunks t + 256 i, i < NPRE, of thread t (NPRE = 2 covers K = 4096 for INT4).
// Vector memory loads retire in issue order, so only loads issued before the
// weights can be waited for without waiting for the weights too.
struct PreAct {
  uint32_t d[8];
};


// Through a buffer resource of the row (32-bit offsets), so that no 64-bit
// addresses stay live across the weight loads that follow.
template <int BITS, int NPRE>
__device__ __forceinline__ void pre_load(const uint16_t *src0, int K, PreAct &pa) {
  const int nch = K / kChunkE<BITS>;
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc((void *)src0, (short)0, K * 2, 0x00020000);
#pragma unroll
  for (int i = 0; i < NPRE; ++i) {
    const int q = threadIdx.x + 256 * i;
    if (q < nch) {
#pragma unroll
      for (int t = 0; t < kChunkE<BITS> / 2; t += 4) {
        const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rs, (uint32_t)(q * kChunkE<BITS> * 2 + t * 4), 0, 0);
        pa.d[4 * i + t] = v[0];
        pa.d[4 * i + t + 1] = v[1];
        pa.d[4 * i + t + 2] = v[2];
        pa.d[4 * i + t + 3] = v[3];
      }
    }
  }
}

// Per-group sums of the staged rows 0..R-1 (GS / 16 threads per group, 16
// elements each) into Xs; starts and ends with a block barrier.
template <int GS>
__device__ __forceinline__ void stage_group_sums(const uint8_t *act, float *Xs, int R, int K) {
  constexpr int NP = GS / 16;
  const int pitch = K * 2 + 16;
  lds_barrier();
  const int G = K / GS;
  for (int r = 0; r < R; ++r) {
    for (int t = threadIdx.x; t < G * NP; t += 256) {
      const int g = t / NP, part = t % NP;
      const u32x4 *p = (const u32x4 *)(act + r * pitch + (g * GS + part * 16) * 2);
      const u32x4 v0 = p[0], v1 = p[1];
      float sum = 0.f;
#pragma unroll
      for (int z = 0; z < 4; ++z) {
        sum = dot2_bf16(v0[z], 0x3F803F80u, sum);
        sum = dot2_bf16(v1[z], 0x3F803F80u, sum);
      }
      sum = group_sum(sum, NP);
      if (part == 0) {
        if (r == R - 1) {
          for (int m = r; m < 16; ++m) Xs[g * 16 + m] = sum;
        } else {
          Xs[g * 16 + r] = sum;
        }
      }
    }
  }
  lds_barrier();
}

// Stages activation rows 0..R-1 (src(r): row r's global address); chunks
// q < q0 of row 0 come from pa (q0 = 256 * NPRE or 0).  Ends with a block barrier.
// NVFP4 activations quantised in LDS: rows 0..R-1 (natural order), one
// thread per group of 16 (the steps of the activation quantiser, tensor
// scale G), each group replaced by q * s.  Starts and ends with a barrier.
__device__ __forceinline__ void quantize_rows_lds(uint8_t *act, int R, int K, float G) {
  const int pitch = K * 2 + 16, ng = K / 16;
  lds_barrier();
  for (int t = threadIdx.x; t < R * ng; t += 256) {
    u32x4 *p = (u32x4 *)(act + (t / ng) * pitch + (t % ng) * 32);
    const u32x4 a = p[0], b = p[1];
    float v[16];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[2 * j] = bf16lo(a[j]);
      v[2 * j + 1] = bf16hi(a[j]);
      v[8 + 2 * j] = bf16lo(b[j]);
      v[8 + 2 * j + 1] = bf16hi(b[j]);
    }
    float amax = 0.f;
#pragma unroll
    for (int j = 0; j < 16; ++j) amax = fmaxf(amax, fabsf(v[j]));
    const float s = round_e4m3(amax / (6.f * G));
    const float sg = s * G;
    uint32_t o[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float q0 = sg > 0.f ? round_e2m1(v[2 * j] / sg) : 0.f;
      const float q1 = sg > 0.f ? round_e2m1(v[2 * j + 1] / sg) : 0.f;
      o[j] = pack_bf16x2(q0 * s, q1 * s);
    }
    p[0] = u32x4{o[0], o[1], o[2], o[3]};
    p[1] = u32x4{o[4], o[5], o[6], o[7]};
  }
  lds_barrier();
}

// QX: quantise the staged rows to NVFP4 first (tensor scale G; the fused layer).
template <int BITS, int GS, int NPRE, bool QX = false, typename Src>
__device__ __forceinline__ void stage_rows(uint8_t *act, float *Xs, Src src, int R, int K, int q0,
                                           const PreAct *pa, float G = 0.f) {
  const int pitch = K * 2 + 16;
  const int nch = K / kChunkE<BITS>;
  if (q0 > 0) {
#pragma unroll
    for (int i = 0; i < NPRE; ++i) {
      const int q = threadIdx.x + 256 * i;
      if (q < nch) store_act_chunk<BITS>(act, q, pa->d + 4 * i);
    }
  }
  for (int r = 0; r < R; ++r) {
    const uint16_t *s = src(r);
    for (int q = (r == 0 ? q0 : 0) + threadIdx.x; q < nch; q += 256) {
      uint32_t d[kChunkE<BITS> / 2];
      load_act_chunk<BITS>(s, q, d);
      store_act_chunk<BITS>(act + r * pitch, q, d);
    }
  }
  if constexpr (QX) quantize_rows_lds(act, R, K, G);
  stage_group_sums<GS>(act, Xs, R, K);
}

// Stages h rows 0..R-1 (h0: row 0's words, rows I words apart) once phase 1
// has written them: each thread reads its chunks with device-coherent loads
// until every word carries kHReady.  Returns false if a wait timed out.
template <int BITS, int GS>
__device__ __forceinline__ bool stage_h_rows(uint8_t *act, float *Xs, const uint32_t *h0, int R, int I,
                                             int max_spins) {
  constexpr int CE = kChunkE<BITS>;
  const int pitch = I * 2 + 16;
  const int nch = I / CE;
  bool ok = true;
  for (int r = 0; r < R; ++r) {
    for (int q = threadIdx.x; q < nch; q += 256) {
      const uint32_t *src = h0 + (size_t)r * I + q * CE;
      uint32_t w[CE];
      for (int spins = 0;; ++spins) {
        uint32_t all = kHReady;
#pragma unroll
        for (int t = 0; t < CE; ++t) {
          w[t] = __hip_atomic_load(src + t, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          all &= w[t];
        }
        if (all) break;
        if (spins >= max_spins) {
          ok = false;
          break;
        }
        __builtin_amdgcn_s_sleep(1);
      }
      uint32_t d[CE / 2];
#pragma unroll
      for (int t = 0; t < CE / 2; ++t) d[t] = (w[2 * t] & 0xFFFFu) | (w[2 * t + 1] << 16);
      store_act_chunk<BITS>(act + r * pitch, q, d);
    }
  }
  stage_group_sums<GS>(act, Xs, R, I);
  return ok;
}

// One-token phase 2, pipelined per K group: wave w stages the h groups
// g = w + 4 j as their words arrive (polling between its MFMA groups), and
// every wave runs the groups in K order as each one is staged; a staged group
// is announced by an LDS flag.  A wave has at most kHPend such groups.
constexpr int kHPend = 4;

// Operand-order slot of element i of an activation chunk (inverse of the
// pair order of the unpacked codes, see order_pairs).
template <int BITS>
__device__ __forceinline__ int chunk_slot(int i) {
  return BITS >= 5 ? i : BITS == 4 ? (i >> 1) + 4 * (i & 1) : (i >> 2) + 4 * (i & 3);
}

// One polling round for the wave's lowest pending unit (bit j of pend: unit
// wv + 4 j of 128 K): every lane reads two of its h words.  Once all carry
// kHReady the unit goes to act in operand order, its group sums (the
// arithmetic of stage_group_sums) to the 16 rows of Xs, and gflag[g] is set.
// Returns the units still pending.
template <int BITS, int GS>
__device__ uint32_t service_h(uint32_t pend, const uint32_t *h, uint8_t *act, float *Xs, int *gflag, int wv) {
  constexpr int CE = kChunkE<BITS>;
  const int lane = lane_id();
  const int j = __builtin_ctz(pend);
  const int g = wv + 4 * j;
  const uint32_t *src = h + g * kGroup + 2 * lane;
  const uint32_t w0 = __hip_atomic_load(src, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const uint32_t w1 = __hip_atomic_load(src + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (__ballot(!(w0 & w1 & kHReady))) return pend;
  const int e = g * kGroup + 2 * lane;  // element of the row (even)
  uint16_t *row = (uint16_t *)act;
  row[(e / CE) * CE + chunk_slot<BITS>(e % CE)] = (uint16_t)(w0 & 0xFFFFu);
  row[(e / CE) * CE + chunk_slot<BITS>(e % CE + 1)] = (uint16_t)(w1 & 0xFFFFu);
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
  float sum = 0.f;
  if (lane < 8) {
    const u32x4 *pp = (const u32x4 *)(act + (g * kGroup + lane * 16) * 2);
    const u32x4 v0 = pp[0], v1 = pp[1];
#pragma unroll
    for (int z = 0; z < 4; ++z) {
      sum = dot2_bf16(v0[z], 0x3F803F80u, sum);
      sum = dot2_bf16(v1[z], 0x3F803F80u, sum);
    }
  }
  if constexpr (GS == 128) {
    sum = group_sum(sum, 8);
    const float v = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, sum)));
    if (lane < 16) Xs[g * 16 + lane] = v;
  } else {
    // groups of 32: the sums of lanes 0, 2, 4, 6; lane 16 j + m writes group j, row m
    sum = group_sum(sum, 2);
    const int j = lane >> 4;
    const int src = __builtin_amdgcn_readlane(__builtin_bit_cast(int, sum), 0);
    const int s1 = __builtin_amdgcn_readlane(__builtin_bit_cast(int, sum), 2);
    const int s2 = __builtin_amdgcn_readlane(__builtin_bit_cast(int, sum), 4);
    const int s3 = __builtin_amdgcn_readlane(__builtin_bit_cast(int, sum), 6);
    const int v = j == 0 ? src : j == 1 ? s1 : j == 2 ? s2 : s3;
    Xs[(4 * g + j) * 16 + (lane & 15)] = __builtin_bit_cast(float, v);
  }
  if (lane == 0) __hip_atomic_store(gflag + g, 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
  return pend & ~(1u << j);
}


// Per-expert metadata of active slot a (wave-uniform; through the scalar cache).
// With one token, the a-th active expert (ascending) owns sorted row a.
struct Meta {
  int e, o0, o1;
};
template <bool ONE>
__device__ __forceinline__ Meta meta(const DecodeParams &p, int a, int nrows) {
  Meta r;
  r.e = min(max(sload(p.active + 1 + a), 0), p.E - 1);
  if constexpr (ONE) {
    r.o0 = min(a, nrows);
    r.o1 = min(a + 1, nrows);
  } else {
    r.o0 = min(max(sload(p.offsets + r.e), 0), nrows);
    r.o1 = min(max(sload(p.offsets + r.e + 1), r.o0), nrows);
  }
  return r;
}


// ONE: T == 1 (every active expert has exactly one routed row, of token 0).
// FAST: every wave's phase-1 unit range and the phase-2 K split into full
// chunks of kCG units (INT4 and 2-bit with groups of 128: H % 4096 == 0 and
// I % 1024 == 0); the first chunk of weights is then requested before the
// activations are staged.
// Fused layer routing record.  The selector block ranks the T*k rows by
// (expert, row) - the order of moe_permute - and stores, at each sorted
// position i, one tagged word: kRecTag | row << 48 | expert << 32 | gate bits.
// Every block then derives its grouping from the words alone.
constexpr int kRecRowBits = 15;  // rows < 2^15
constexpr int kRecIdBits = 16;   // experts < 2^16

// Sorted position of the rows r = lane + 64 c (c < NC, r < n) among the rows
// q < n by (ids[q], q), from bit-plane ballots: walking the id bits from the
// top, the lanes that agree with r on the bits so far and have a 0 where r has
// a 1 are below r.  Rows of an earlier chunk, or a lower lane, with r's id
// are below it too.  nbits covers every id.
template <int NC>
__device__ __forceinline__ void wave_rank_rows(const int (&id)[NC], int n, int nbits, int (&pos)[NC]) {
  const int lane = lane_id();
  const uint64_t below = lane == 0 ? 0ull : (~0ull >> (64 - lane));
#pragma unroll
  for (int c = 0; c < NC; ++c) pos[c] = 0;
#pragma unroll
  for (int d = 0; d < NC; ++d) {
    if (kWave * d >= n) break;
    const uint64_t vm = __ballot(lane + kWave * d < n);
    uint64_t eq[NC];
    int less[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      eq[c] = vm;
      less[c] = 0;
    }
    for (int b = nbits - 1; b >= 0; --b) {
      const uint64_t m = __ballot((id[d] >> b) & 1) & vm;
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        if ((id[c] >> b) & 1) {
          less[c] += __popcll(eq[c] & ~m);
          eq[c] &= m;
        } else {
          eq[c] &= ~m;
        }
      }
    }
#pragma unroll
    for (int c = 0; c < NC; ++c) pos[c] += less[c] + (d < c ? __popcll(eq[c]) : d == c ? __popcll(eq[c] & below) : 0);
  }
}

// Selector wave: ranks the n rows (ids and gates in LDS) and stores the record.
// NC = 0: n <= 16, ranked by comparing each row's (id, row) key with every
// other row's, fetched with independent readlanes (a short dependence chain).
template <int NC>
__device__ void publish_sorted_record(const int32_t *ids, const float *gates, int n, int E, uint64_t *rec) {
  const int lane = lane_id();
  constexpr int NR = NC > 0 ? NC : 1;
  int id[NR], pos[NR];
#pragma unroll
  for (int c = 0; c < NR; ++c) {
    const int r = lane + kWave * c;
    id[c] = r < n ? ids[r] : 0;
  }
  if constexpr (NC == 0) {
    // lanes past n get the largest key, so they are never counted as lower
    const int key = lane < n ? (id[0] << 4) | lane : 0x7fffffff;
    pos[0] = 0;
#pragma unroll
    for (int q = 0; q < 16; ++q) pos[0] += __builtin_amdgcn_readlane(key, q) < key;
  } else {
    wave_rank_rows<NC>(id, n, 32 - __clz(max(E - 1, 0)), pos);
  }
#pragma unroll
  for (int c = 0; c < NR; ++c) {
    const int r = lane + kWave * c;
    if (r < n) {
      const uint64_t w = kRecTag | ((uint64_t)r << 48) | ((uint64_t)(uint32_t)id[c] << 32) | __float_as_uint(gates[r]);
      __hip_atomic_store(rec + pos[c], w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// Every block, one wave: reads the n record words (re-reading, with a short
// back-off, until all carry the tag) and fills, for sorted position i, row
// sorted[i] (rowpos[sorted[i]] = i, gates[sorted[i]] = its gate) and, for the
// a-th expert with rows (ascending), act[1 + a] = expert and start[a] = its
// first sorted position; act[0] = number of such experts, start[act[0]] = n.
// Returns false if a wait ran out (the values are then clamped, not exact).
__device__ bool read_sorted_record(const uint64_t *rec, int n, int E, int max_spins, int32_t *sorted,
                                   int32_t *rowpos, float *gates, int32_t *act, int32_t *start) {
  const int lane = lane_id();
  const uint64_t below = lane == 0 ? 0ull : (~0ull >> (64 - lane));
  bool ok = true;
  int base = 0, prev_last = -1;
  for (int c0 = 0; c0 < n; c0 += kWave) {
    const int i = c0 + lane;
    uint64_t w = kRecTag;
    for (int spins = 0;; ++spins) {
      if (i < n) w = __hip_atomic_load(rec + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (__ballot(!(w & kRecTag)) == 0) break;
      if (spins >= max_spins) {
        ok = false;
        break;
      }
      const int nz = min(1 << min(spins, 2), 4);
      for (int z = 0; z < nz; ++z) __builtin_amdgcn_s_sleep(2);
    }
    const int row = min((int)((w >> 48) & ((1u << kRecRowBits) - 1)), n - 1);
    const int e = min((int)((w >> 32) & ((1u << kRecIdBits) - 1)), E - 1);
    int prev = __shfl_up(e, 1, kWave);
    if (lane == 0) prev = prev_last;
    const bool head = i < n && e != prev;
    const uint64_t hm = __ballot(head);
    if (i < n) {
      sorted[i] = row;
      rowpos[row] = i;
      gates[row] = __uint_as_float((uint32_t)w);
    }
    if (head) {
      const int slot = base + __popcll(hm & below);
      act[1 + slot] = e;
      start[slot] = i;
    }
    base += __popcll(hm);
    prev_last = __shfl(e, kWave - 1, kWave);
  }
  if (lane == 0) {
    act[0] = base;
    start[base] = n;
  }
  return ok;
}

// LAYER: the whole decode layer in one launch.  Before its items (a) the
// first blocks compute the router logits (two experts per block, staged in
// LDS by slice, or one wave per expert where H does not suit), stored as
// tagged words;
// (b) block 0 runs every token's top-k (the same functions as the router
// kernels, so the same bits), ranks the T*k rows by (expert, row) and
// publishes them in that order as tagged words; (c) every block reads those
// words and derives the grouping in LDS.  After its items, block b < H/128 combines
// columns [128 b, 128 b + 128) of y from the tagged y_perm words.
template <int BITS, int GS, bool ONE, bool FAST, bool LAYER, bool TAB>
__global__ void __launch_bounds__(256, 3) ffn_decode_kernel(DecodeParams p) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  constexpr int RM = ONE ? 1 : kRMax;
  constexpr int GB = kGroupBytes<BITS>;
  // SPU: scales per 128-K unit (NVFP4: its 8 scale bytes counted as 4 pairs)
  constexpr int CG = kCG<BITS, GS>, SPU = BITS == 5 ? 4 : kSPU<GS>;
  constexpr bool NV = BITS == 5;
  // a lane's activation bytes within a unit: K 32 lsub (groups of 128) or
  // 8 lsub, then +32 per MFMA (groups of 32, after the slice transpose)
  constexpr int LA = GS == 32 ? 16 : 64;
  // activation chunks per thread loaded ahead of the phase-1 weights
  constexpr int NPRE = (BITS != 2 && ONE) ? 2 : 1;
  const uint32_t magic = p.magic;
  const int lane = lane_id();
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int m = lane % 16, lsub = lane / 16;
  const int nrows = p.T * p.k;
  const int per1 = p.I / kRows1, per2 = p.H / kRows2;
  const int G1 = p.H / kGroup, G2 = p.I / kGroup;
  const int pitch1 = p.H * 2 + 16, pitch2 = p.I * 2 + 16;
  const int pmax = pitch1 > pitch2 ? pitch1 : pitch2;
  uint8_t *act = lds;
  float *Xs = (float *)(lds + RM * pmax);
  float *red = Xs + 16 * SPU * (G1 > G2 ? G1 : G2);
  // fused layer: routing results in LDS after the FFN's own arrays, or after
  // the router's rows where those are larger (they share the start of LDS)
  int *s_next = (int *)(red + kRedFloats);  // the block's next item (item queues)
  const size_t ffn_bytes = (size_t)((uint8_t *)(red + kRedFloats) - lds) + 16;
  const bool lds_router = LAYER && router_lds_ok(p.H);
  const size_t rbytes = lds_router ? router_lds_bytes(p.H) : 0;
  int32_t *s_ids = (int32_t *)(lds + (ffn_bytes > rbytes ? ffn_bytes : rbytes));  // [T*k] selector block only
  float *s_gates = (float *)(s_ids + nrows);       // [T*k] gate of flat row r
  int32_t *s_sorted = (int32_t *)(s_gates + nrows);
  int32_t *s_rowpos = s_sorted + nrows;
  int32_t *s_act = s_rowpos + nrows;  // [1 + T*k]
  int32_t *s_start = s_act + nrows + 1;  // [1 + T*k]
  if constexpr (LAYER) {
    // (a) router logits: wave w of block b takes experts 4 b + w, 4 (b + grid) + w, ...
    if (lds_router && p.E <= 2 * (int)gridDim.x) {
      // block b takes experts 2 b + pair (waves 2 pair, 2 pair + 1): both waves
      // load half of the weight row each and the block each token's
      // activations, with coalesced loads, re-laid in LDS by slice; the
      // pair's first wave runs the dot
      if ((int)blockIdx.x * 2 < p.E) {
        const int sw64 = 64 * router_slice_words(p.H);
        const int pair = wv >> 1, half = wv & 1, nch = p.H / 8;
        uint32_t *xl = (uint32_t *)lds;
        uint32_t *wl = xl + sw64 * (1 + pair);
        const int e = blockIdx.x * 2 + pair;
        const bool has = e < p.E;
        // the weight half-row and token 0's activations in one batch of loads
        // (a wave without an expert loads its pair's row, unused)
        rows_to_slices<4, 2>(p.w_router + (size_t)min(e, p.E - 1) * p.H, wl, half * (nch / 2),
                             (half + 1) * (nch / 2), lane, kWave, p.x, xl, 0, nch, threadIdx.x, 256, p.H);
        const float b = has && p.bias ? p.bias[e] : 0.f;
        for (int t = 0; t < p.T; ++t) {
          if (t > 0) {
            lds_barrier();  // every wave is done with the previous token
            row_to_slices<2>(p.x + (size_t)t * p.H, p.H, xl, 0, nch, threadIdx.x, 256);
          }
          lds_barrier();
          if (has && half == 0) {
            const float v = router_dot_slices(xl, wl, p.H, b);
            if (lane == 0)
              __hip_atomic_store(p.tl + (size_t)t * p.E + e, kLogitTag | __float_as_uint(v), __ATOMIC_RELAXED,
                                 __HIP_MEMORY_SCOPE_AGENT);
          }
        }
      }
    } else {
      const int L = p.H / 64;
      for (int e = blockIdx.x * 4 + wv; e < p.E; e += gridDim.x * 4) {
        if (L % 8 == 0)
          router_logits_wave<8, 1>(p.x, p.w_router, p.bias, p.T, p.H, p.E, e, p.tl);
        else if (L % 4 == 0)
          router_logits_wave<4, 1>(p.x, p.w_router, p.bias, p.T, p.H, p.E, e, p.tl);
        else
          router_logits_wave<2, 1>(p.x, p.w_router, p.bias, p.T, p.H, p.E, e, p.tl);
      }
    }
    // (b) block 0 selects: wave w runs the top-k of tokens w, w + 4, ...
    // (reading and then clearing their logits), then wave 0 ranks all T*k
    // rows and publishes them in sorted order.  One block doing the whole
    // selection lets every other block read a single ready-made record.
    if (blockIdx.x == 0) {
      for (int t = wv; t < p.T; t += 4) {
        const TaggedLogits ld{p.tl + (size_t)t * p.E, p.E, p.max_spins, p.ctl, true,
                              p.logits_out ? p.logits_out + (size_t)t * p.E : nullptr};
        int32_t *ids = s_ids + t * p.k;
        float *g = s_gates + t * p.k;
        topk_softmax_any(ld, p.E, p.k, ids, g);
        __builtin_amdgcn_wave_barrier();
        if (lane < p.k) {
          if (p.ids_out) p.ids_out[t * p.k + lane] = ids[lane];
          if (p.gates_out) p.gates_out[t * p.k + lane] = g[lane];
        }
      }
      lds_barrier();
      if (wv == 0) {
        if (nrows <= 16)
          publish_sorted_record<0>(s_ids, s_gates, nrows, p.E, p.rec);
        else if (nrows <= kWave)
          publish_sorted_record<1>(s_ids, s_gates, nrows, p.E, p.rec);
        else if (nrows <= 2 * kWave)
          publish_sorted_record<2>(s_ids, s_gates, nrows, p.E, p.rec);
        else
          publish_sorted_record<4>(s_ids, s_gates, nrows, p.E, p.rec);
      }
    }
    // (c) every block reads the record and derives its grouping
    if (wv == 0 &&
        !read_sorted_record(p.rec, nrows, p.E, p.max_spins, s_sorted, s_rowpos, s_gates, s_act, s_start) &&
        lane == 0)
      atomicOr(&p.ctl[kCtlError], 1);
    lds_barrier();
  }
  // With one token every active slot holds one of its k distinct experts, so
  // the item partition uses Amax (= k) without first reading the count.
  const int A = ONE ? p.Amax : LAYER ? min(max(s_act[0], 0), p.Amax) : min(max(sload(p.active), 0), p.Amax);
  const int n1 = A * per1, n2 = A * per2;
  const int Gw1 = (G1 + 3) / 4;  // phase-1 groups per wave
  auto get_meta = [&](int a) -> Meta {
    if constexpr (LAYER) {
      Meta r;
      // A slot's first row is below nrows whatever the record held (one
      // token's phase 2 reads and writes row o0 even for an empty slot, which
      // only a record read after a timed-out wait can produce).
      r.e = min(max(s_act[1 + a], 0), p.E - 1);
      r.o0 = min(max(s_start[a], 0), nrows - 1);
      r.o1 = min(max(s_start[a + 1], r.o0), nrows);
      return r;
    } else {
      return meta<ONE>(p, a, nrows);
    }
  };

  bool routed = false;  // fused layer: this block has counted itself done with the record
  // More items than blocks: after its first item (its own index) a block
  // draws the next from its queue, so blocks whose items ran fast take more
  // of them.  Every queue item is phase 2 unless every first item is phase 1,
  // and a queue hands out its items in index order (phase 1 first), so a
  // phase-2 item only ever waits for phase-1 items that are being worked on.
  const int n_items = n1 + n2, grid = gridDim.x;
  const bool dyn = n_items > grid;
  const int nq = grid < kQueues ? grid : kQueues, qx = blockIdx.x % nq;
  const int q_items = n_items - grid > qx ? (n_items - grid - qx + nq - 1) / nq : 0;  // items of this queue
  const int q_blocks = (grid - qx + nq - 1) / nq;                                    // blocks drawing from it
  int *qc = queue_ctr(p.ctl, p.Amax, qx);
  int ticket = -1;  // thread 0: position drawn from the queue while the current item runs
  auto draw = [&]() {
    if (dyn && threadIdx.x == 0 && ticket < 0) ticket = atomicAdd(qc, 1);
  };
  for (int item = blockIdx.x; item < n_items;) {
    if (item < n1) {
      // ============================================================ phase 1
      // One token: the experts are interleaved (item = i A + a).  The blocks
      // dispatched first (one per CU) get their weights first, so every
      // expert has its early rows there and its phase 2 starts on the early
      // half of h while the rest streams in (measured 0.2-0.4 us shorter
      // than expert by expert).  With more tokens the items go expert by
      // expert, so that early experts finish their phase 1 (and their
      // phase 2 can start) while later ones run.
      const int a = ONE ? item % A : item / per1, i0 = (ONE ? item / A : item - a * per1) * kRows1;
      const Meta md = get_meta(a);
      const int g0 = wv * Gw1, ng = max(min(Gw1, G1 - g0), 0);
      const size_t erows = (size_t)md.e * 2 * p.I;  // first row of the expert
      const ExpertW xw = TAB ? expert_from_table(p.tab, md.e, 0)
                             : ExpertW{(const uint8_t *)p.w13c + erows * (G1 * GB),
                                         (const uint8_t *)p.w13s + erows * (G1 * 2 * SPU), p.w13z + erows * G1};
      Off o2[2] = {row_off<SPU>(i0 + m, G1, g0, GB, lsub), row_off<SPU>(p.I + i0 + m, G1, g0, GB, lsub)};
      if constexpr (NV) {  // the lane's two scale bytes of each unit
        o2[0].s += 2 * lsub;
        o2[1].s += 2 * lsub;
      }
      const int nch = ng / CG;
      // activation row of sorted position q
      auto xrow = [&](int q) -> const uint16_t * {
        const int t = ONE ? 0 : min(max(LAYER ? s_sorted[q] : sload(p.sorted_rows + q), 0) / p.k, p.T - 1);
        return p.x + (size_t)t * p.H;
      };
      PreAct pa;
      int q0 = 0;
      Chunk<BITS, GS> wgu[2];
      if constexpr (FAST) {
        if (md.o0 < md.o1) {
          pre_load<BITS, NPRE>(xrow(md.o0), p.H, pa);
          q0 = 256 * NPRE;
        }
        load_chunk<BITS, GS>(xw, o2[0], wgu[0]);
        load_chunk<BITS, GS>(xw, o2[1], wgu[1]);
      }
      draw();  // after the weight loads, so the atomic holds none of them up
      for (int rb = md.o0; rb < md.o1; rb += RM) {
        const int R = ONE ? 1 : min(RM, md.o1 - rb);
        // the fused NVFP4 layer quantises the activations it stages (the stage
        // call gets them quantised already)
        stage_rows<BITS, GS, NPRE, LAYER && NV>(act, Xs, [&](int r) { return xrow(rb + r); }, R, p.H,
                                                 rb == md.o0 ? q0 : 0, &pa, p.gx);
        const int arow = ONE ? 0 : min(m, R - 1);
        const uint8_t *ap = act + arow * pitch1 + lsub * LA + g0 * (kGroup * 2);
        const float *xs = Xs + g0 * 16 * SPU + (ONE ? 0 : 4 * lsub);
        f32x4 tgu[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
        if constexpr (FAST) {
          for (int ch = 0; ch < nch; ++ch) {
            if (ch > 0) {
              load_chunk<BITS, GS>(xw, add_groups<SPU>(o2[0], ch * CG, GB), wgu[0]);
              load_chunk<BITS, GS>(xw, add_groups<SPU>(o2[1], ch * CG, GB), wgu[1]);
            }
            chunk_gemv<BITS, GS, ONE, 2>(wgu, ap + ch * CG * (kGroup * 2), xs + ch * CG * 16 * SPU, magic, tgu);
          }
          if (nch > 1 && rb + RM < md.o1) {  // the next pass starts again from the first chunk
            load_chunk<BITS, GS>(xw, o2[0], wgu[0]);
            load_chunk<BITS, GS>(xw, o2[1], wgu[1]);
          }
        } else {
          groups_gemv_slow<BITS, GS, ONE, 2>(xw, o2, ng, ap, xs, magic, tgu);
        }
        const f32x4 tg = tgu[0], tu = tgu[1];
        // cross-wave sum of the 16 x 16 gate / up partials: red[wave][gate|up][row][col]
        float *rw = red + wv * 512;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          rw[(4 * lsub + i) * 16 + m] = tg[i];
          rw[256 + (4 * lsub + i) * 16 + m] = tu[i];
        }
        lds_barrier();
        if (threadIdx.x < R * 16) {  // all in wave 0
          const int mm = threadIdx.x / 16, n = threadIdx.x % 16;
          float gv = 0.f, uv = 0.f;
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            gv += red[w * 512 + mm * 16 + n];
            uv += red[w * 512 + 256 + mm * 16 + n];
          }
          float hv;
          if constexpr (NV) {  // tensor scales, then h quantised in its group of 16 (lanes 16 mm .. +15)
            const float osc = p.gx * sload(TAB ? (const float *)xw.zeros : p.g13 + md.e);
            hv = quant16_lanes(silu_f(gv * osc) * (uv * osc), p.gh);
          } else {
            hv = silu_f(gv) * uv;
          }
          __hip_atomic_store(p.hbuf + (size_t)(rb + mm) * p.I + i0 + n, kHReady | (uint32_t)f32_to_bf16(hv),
                             __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        lds_barrier();
      }
    } else {
      // ============================================================ phase 2
      const int it = item - n1;
      const int a = it / per2, n0 = (it - a * per2) * kRows2 + wv * 32;
      const Meta md = get_meta(a);
      const size_t erows = (size_t)md.e * p.H;
      const ExpertW xw = TAB ? expert_from_table(p.tab, md.e, 3)
                             : ExpertW{(const uint8_t *)p.w2c + erows * (G2 * GB),
                                         (const uint8_t *)p.w2s + erows * (G2 * 2 * SPU), p.w2z + erows * G2};
      Off o2[2] = {row_off<SPU>(n0 + m, G2, 0, GB, lsub), row_off<SPU>(n0 + 16 + m, G2, 0, GB, lsub)};
      if constexpr (NV) {
        o2[0].s += 2 * lsub;
        o2[1].s += 2 * lsub;
      }
      const int nch = G2 / CG;
      // NVFP4 output scale; a table row holds the address of the tensor scale
      // where other formats keep their zero-points
      const float osc2 = NV ? p.gh * sload(TAB ? (const float *)xw.zeros : p.g2 + md.e) : 1.f;
      Chunk<BITS, GS> wd[2];
      if constexpr (FAST) {
        load_chunk<BITS, GS>(xw, o2[0], wd[0]);
        load_chunk<BITS, GS>(xw, o2[1], wd[1]);
      }
      draw();
      // Fused layer: a phase-2 block counts itself done with the routing
      // record once its weight loads are issued (the atomic then completes
      // while the block waits for h, and holds up no load of its own).
      if (LAYER && !routed) {
        if (threadIdx.x == 0) atomicAdd(routed_ctr(p.ctl, p.Amax, blockIdx.x % kRoutedN), 1);
        routed = true;
      }
      // One token with full chunks (the host keeps I / 128 <= 4 kHPend for
      // it): the per-group pipeline.
      constexpr bool kPipe = ONE && FAST;
      if constexpr (kPipe) {
        int *gflag = (int *)red + 64;
        if (threadIdx.x < G2) gflag[threadIdx.x] = 0;
        lds_barrier();
        const uint32_t *h = p.hbuf + (size_t)md.o0 * p.I;
        uint32_t pend = (1u << ((G2 - wv + 3) / 4)) - 1u;
        pend = service_h<BITS, GS>(pend, h, act, Xs, gflag, wv);
        const uint8_t *ap = act + lsub * LA;
        f32x4 ty[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
        bool ok = true;
        for (int ch = 0; ch < nch; ++ch) {
          if (ch > 0) {
            load_chunk<BITS, GS>(xw, add_groups<SPU>(o2[0], ch * CG, GB), wd[0]);
            load_chunk<BITS, GS>(xw, add_groups<SPU>(o2[1], ch * CG, GB), wd[1]);
          }
#pragma unroll
          for (int c = 0; c < CG; ++c) {
            const int g = ch * CG + c;
            for (int spins = 0;; ++spins) {
              if (__hip_atomic_load(gflag + g, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP)) break;
              if (spins >= p.max_spins) {
                ok = false;
                break;
              }
              if (pend)
                pend = service_h<BITS, GS>(pend, h, act, Xs, gflag, wv);
              else
                __builtin_amdgcn_s_sleep(1);
            }
            Word<BITS> w2[2];
            w2[0] = wd[0].w[c];
            w2[1] = wd[1].w[c];
            if constexpr (NV) {
              const uint32_t sc[2] = {wd[0].s[c], wd[1].s[c]};
              nv_unit_acc<2>(w2, sc, ap + g * (kGroup * 2), ty);
            } else if constexpr (GS == 32) {
              const uint32_t sc[2][2] = {{wd[0].s[2 * c], wd[0].s[2 * c + 1]}, {wd[1].s[2 * c], wd[1].s[2 * c + 1]}};
              unit32_acc<BITS, ONE, 2>(w2, ap + g * (kGroup * 2), sc, Xs + g * 64, magic, ty);
            } else {
              f32x4 cg[2];
              group_mfma<BITS, 2>(w2, ap + g * (kGroup * 2), magic, cg);
#pragma unroll
              for (int r = 0; r < 2; ++r) {
                const float sc = scale_f32<BITS>((wd[r].s[c / 2] >> (16 * (c & 1))) & 0xFFFFu);
                const float zo = zero_off<BITS>((wd[r].z[c / 4] >> (8 * (c % 4))) & 0xFFu);
                group_acc<ONE>(cg[r], sc, zo, Xs + g * 16, ty[r]);
              }
            }
          }
        }
        if (!ok && threadIdx.x % kWave == 0) atomicOr(&p.ctl[kCtlError], 1);
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
          const size_t yo = (size_t)md.o0 * p.H + n0 + 16 * s2 + m;
          if (lsub == 0) {
            if constexpr (LAYER)
              __hip_atomic_store(p.ybuf + yo, kHReady | (uint32_t)f32_to_bf16(ty[s2][0] * osc2), __ATOMIC_RELAXED,
                                 __HIP_MEMORY_SCOPE_AGENT);
            else
              p.y_perm[yo] = f32_to_bf16(ty[s2][0] * osc2);
          }
        }
        lds_barrier();  // LDS is rewritten by the next item
      }
      for (int rb = md.o0; rb < (kPipe ? md.o0 : md.o1); rb += RM) {
        const int R = ONE ? 1 : min(RM, md.o1 - rb);
        if (!stage_h_rows<BITS, GS>(act, Xs, p.hbuf + (size_t)rb * p.I, R, p.I, p.max_spins))
          atomicOr(&p.ctl[kCtlError], 1);
        const int arow = ONE ? 0 : min(m, R - 1);
        const uint8_t *ap = act + arow * pitch2 + lsub * LA;
        const float *xs = Xs + (ONE ? 0 : 4 * lsub);
        f32x4 ty[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
        if constexpr (FAST) {
          for (int ch = 0; ch < nch; ++ch) {
            if (ch > 0) {
              load_chunk<BITS, GS>(xw, add_groups<SPU>(o2[0], ch * CG, GB), wd[0]);
              load_chunk<BITS, GS>(xw, add_groups<SPU>(o2[1], ch * CG, GB), wd[1]);
            }
            chunk_gemv<BITS, GS, ONE, 2>(wd, ap + ch * CG * (kGroup * 2), xs + ch * CG * 16 * SPU, magic, ty);
          }
          if (nch > 1 && rb + RM < md.o1) {
            load_chunk<BITS, GS>(xw, o2[0], wd[0]);
            load_chunk<BITS, GS>(xw, o2[1], wd[1]);
          }
        } else {
          groups_gemv_slow<BITS, GS, ONE, 2>(xw, o2, G2, ap, xs, magic, ty);
        }
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
          const size_t yo = (size_t)rb * p.H + n0 + 16 * s2 + m;
          auto put = [&](size_t o, float v) {
            if constexpr (LAYER)
              __hip_atomic_store(p.ybuf + o, kHReady | (uint32_t)f32_to_bf16(v * osc2), __ATOMIC_RELAXED,
                                 __HIP_MEMORY_SCOPE_AGENT);
            else
              p.y_perm[o] = f32_to_bf16(v * osc2);
          };
          if (ONE) {
            if (lsub == 0) put(yo, ty[s2][0]);
          } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int mm = 4 * lsub + i;
              if (mm < R) put(yo + (size_t)mm * p.H, ty[s2][i]);
            }
          }
        }
        lds_barrier();  // LDS is rewritten by the next pass
      }
      // The last phase-2 item of the expert clears the expert's h words and
      // its done counter: every phase-2 item has read h by then.
      int *flag = (int *)red;
      if (threadIdx.x == 0) *flag = atomicAdd(done2(p.ctl, a), 1) == per2 - 1;
      lds_barrier();
      if (*flag) {
        const int n = (md.o1 - md.o0) * p.I;
        uint32_t *h = p.hbuf + (size_t)md.o0 * p.I;
        for (int i = threadIdx.x; i < n; i += 256)
          __hip_atomic_store(h + i, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (threadIdx.x == 0) __hip_atomic_store(done2(p.ctl, a), 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      lds_barrier();  // the flag is read before the next item reuses LDS
    }
    if (!dyn) {
      item += grid;
      continue;
    }
    // the next item from the ticket; the draw that returns the queue's last
    // ticket (q_items + q_blocks - 1: every block's final draw is past its
    // items) re-zeroes the counter for the next call
    if (threadIdx.x == 0) {
      *s_next = ticket < q_items ? grid + qx + nq * ticket : n_items;
      if (ticket == q_items + q_blocks - 1) __hip_atomic_store(qc, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      ticket = -1;
    }
    lds_barrier();
    item = *s_next;
  }
  if constexpr (LAYER) {
    // Phase-1 blocks count after their items (not right after reading the
    // record): the atomic's completion would otherwise hold up the
    // activation loads of the first item.
    if (!routed && threadIdx.x == 0) atomicAdd(routed_ctr(p.ctl, p.Amax, blockIdx.x % kRoutedN), 1);
    // Block 0 clears the routing record once every block has counted itself
    // done with it, and re-zeroes the counters.  By then the phase-2 blocks
    // have counted long ago and the phase-1 blocks are finishing, so this
    // wait is over before block 0's combine below would find its y ready.
    if (blockIdx.x == 0) {
      if (wv == 0) {
        for (int spins = 0;; ++spins) {
          const int c = lane < kRoutedN ? __hip_atomic_load(routed_ctr(p.ctl, p.Amax, lane), __ATOMIC_RELAXED,
                                                            __HIP_MEMORY_SCOPE_AGENT)
                                        : 0;
          if (__builtin_amdgcn_readfirstlane((int)group_sum((float)c, kRoutedN)) >= (int)gridDim.x) break;
          if (spins >= p.max_spins) {
            if (lane == 0) atomicOr(&p.ctl[kCtlError], 1);
            break;
          }
          __builtin_amdgcn_s_sleep(1);
        }
      }
      lds_barrier();
      for (int i = threadIdx.x; i < nrows; i += 256)
        __hip_atomic_store(p.rec + i, (uint64_t)0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (threadIdx.x < kRoutedN)
        __hip_atomic_store(routed_ctr(p.ctl, p.Amax, threadIdx.x), 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    if ((int)blockIdx.x < per2) {
      // y[t, c] = sum over j ascending of g[t, j] * y_perm[row_pos[t k + j], c] in float32,
      // rounded once to bf16; each y_perm word is cleared once read.
      // The words of one token are read kCombB at a time with independent
      // loads (one round trip per batch), re-read until all carry the tag.
      constexpr int kCombB = 8;
      const int c = blockIdx.x * kRows2 + threadIdx.x % kRows2;
      bool ok = true;
      for (int t = threadIdx.x / kRows2; t < p.T; t += 256 / kRows2) {
        float acc = 0.f;
        for (int j0 = 0; j0 < p.k; j0 += kCombB) {
          uint32_t *wp[kCombB];
          uint32_t w[kCombB];
#pragma unroll
          for (int b = 0; b < kCombB; ++b)
            wp[b] = p.ybuf + (size_t)min(max(s_rowpos[t * p.k + min(j0 + b, p.k - 1)], 0), nrows - 1) * p.H + c;
          for (int spins = 0;; ++spins) {
            uint32_t all = kHReady;
#pragma unroll
            for (int b = 0; b < kCombB; ++b) {
              w[b] = __hip_atomic_load(wp[b], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
              all &= w[b];
            }
            if (all) break;
            if (spins >= p.max_spins) {
              ok = false;
              break;
            }
            __builtin_amdgcn_s_sleep(2);
          }
#pragma unroll
          for (int b = 0; b < kCombB; ++b) {
            if (j0 + b < p.k) {
              __hip_atomic_store(wp[b], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
              acc = __builtin_fmaf(s_gates[t * p.k + j0 + b], bf16_to_f32(w[b] & 0xFFFFu), acc);
            }
          }
        }
        p.y[(size_t)t * p.H + c] = f32_to_bf16(acc);
      }
      if (!ok) atomicOr(&p.ctl[kCtlError], 1);
    }
  }
}

template <int BITS, int GS, bool LAYER, bool TAB>
const void *decode_fn_fast(bool one, bool fast) {
  if (one)
    return fast ? (const void *)ffn_decode_kernel<BITS, GS, true, true, LAYER, TAB>
                : (const void *)ffn_decode_kernel<BITS, GS, true, false, LAYER, TAB>;
  return fast ? (const void *)ffn_decode_kernel<BITS, GS, false, true, LAYER, TAB>
              : (const void *)ffn_decode_kernel<BITS, GS, false, false, LAYER, TAB>;
}

template <bool LAYER, bool TAB>
const void *decode_fn_layer(int bits, bool one, bool fast) {
  return bits == 4 ? decode_fn_fast<4, 128, LAYER, TAB>(one, fast) : decode_fn_fast<2, 128, LAYER, TAB>(one, fast);
}

// The stage call of every format, with stacked arrays or an address table.
template <bool TAB>
const void *decode_fn_stage(int bits, int group, bool one, bool fast) {
  if (bits == 8) return group == 32 ? decode_fn_fast<8, 32, false, TAB>(one, fast)
                                    : decode_fn_fast<8, 128, false, TAB>(one, fast);
  if (bits == 6) return decode_fn_fast<6, 128, false, TAB>(one, fast);
  if (bits == 4 && group == 16) return decode_fn_fast<5, 128, false, TAB>(one, fast);  // NVFP4
  if (group == 32) return decode_fn_fast<4, 32, false, TAB>(one, fast);
  return decode_fn_layer<false, TAB>(bits, one, fast);
}

// The layer kernel reads stacked arrays only; the address-table variant is a
// separate instantiation so that the array kernels keep their registers.
const void *decode_kernel_fn(int bits, int group, bool one, bool fast, bool layer, bool tab) {
  if (layer) {  // every format; the NVFP4 layer quantises x as it stages it
    if (bits == 8) return group == 32 ? decode_fn_fast<8, 32, true, false>(one, fast)
                                      : decode_fn_fast<8, 128, true, false>(one, fast);
    if (bits == 6) return decode_fn_fast<6, 128, true, false>(one, fast);
    if (group == 32) return decode_fn_fast<4, 32, true, false>(one, fast);
    if (group == 16) return decode_fn_fast<5, 128, true, false>(one, fast);  // NVFP4
    return decode_fn_layer<true, false>(bits, one, fast);
  }
  return tab ? decode_fn_stage<true>(bits, group, one, fast) : decode_fn_stage<false>(bits, group, one, fast);
}

// Units per chunk of a format (kCG on the host).
int chunk_units(int bits, int group) {
  return group == 16 ? 4 : (bits >= 6 ? 4 : 8) / (group == 32 ? 2 : 1);  // group 16: NVFP4
}

// LDS of the fused layer's routing results (after the FFN's own arrays).
size_t layer_lds_bytes(int T, int k, int E) {
  (void)E;
  const long n = (long)T * k;
  return (size_t)(6 * n + 2) * 4;
}

size_t decode_lds_bytes(int H, int I, bool one, int group = kGroup) {
  const size_t kmax = H > I ? H : I;
  return (size_t)(one ? 1 : kRMax) * (kmax * 2 + 16) + 16 * (kmax / group) * 4 + kRedFloats * 4 + 16;
}

// Fused layer: the router rows (shared start of LDS) or the FFN arrays,
// whichever is larger, then the routing results.
size_t layer_lds_total(int T, int k, int E, int H, int I, int group = kGroup) {
  const size_t f = decode_lds_bytes(H, I, T == 1, group);
  const size_t r = router_lds_ok(H) ? router_lds_bytes(H) : 0;
  return (f > r ? f : r) + layer_lds_bytes(T, k, E);
}

// Co-resident blocks per CU of one decode instantiation (cached per device, kernel and LDS size).
int resident_blocks_per_cu(const void *fn, int device, size_t lds) {
  static std::mutex mu;
  static const void *c_fn[64];
  static int c_dev[64], c_nb[64], n_cached = 0;
  static size_t c_lds[64];
  std::lock_guard<std::mutex> lk(mu);
  for (int i = 0; i < n_cached; ++i)
    if (c_fn[i] == fn && c_dev[i] == device && c_lds[i] == lds) return c_nb[i];
  int nb = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, fn, 256, lds) != hipSuccess) return 0;
  if (n_cached < 64) {
    c_fn[n_cached] = fn;
    c_dev[n_cached] = device;
    c_nb[n_cached] = nb;
    c_lds[n_cached] = lds;
    ++n_cached;
  }
  return nb;
}

}  // namespace

bool decode_layout_ok(int H, int I, int bits, int group) {
  (void)bits;
  return I % kRows1 == 0 && H % kRows2 == 0 && decode_lds_bytes(H, I, false, group) <= 64 * 1024;
}

size_t ffn_ctl_bytes(int T, int k, int E) {
  const long amax = E < (long)T * k ? E : (long)T * k;
  size_t b = (size_t)(kCtlCounters + (amax + kRoutedN + kQueues) * kCtrStride) * 4;
  if (b < kCtlBytes) b = kCtlBytes;
  return (b + 255) / 256 * 256;
}

static void fill_params(DecodeParams &p, const FfnArgs &a, void *ws) {
  p = DecodeParams{};
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
  p.tab = a.tab;
  p.g13 = a.w13_g;
  p.g2 = a.w2_g;
  p.gx = a.gx;
  p.gh = a.gh;
  p.y_perm = a.y_perm;
  p.ctl = (int *)ws;
  p.hbuf = (uint32_t *)((char *)ws + ffn_ctl_bytes(a.T, a.k, a.E));
  p.max_spins = wait_spin_limit();
  p.magic = kMagic43;
}

static hipError_t launch_decode(DecodeParams &p, const FfnArgs &a, bool layer, const DeviceInfo &dev, hipStream_t st) {
  const bool one = a.T == 1;
  // full chunks; with one token also few enough h units for the phase-2 pipeline
  const int cg = chunk_units(a.bits, a.group);
  const bool fast = (a.H / kGroup) % (4 * cg) == 0 && (a.I / kGroup) % cg == 0 && (!one || a.I / kGroup <= 4 * kHPend);
  const void *fn = decode_kernel_fn(a.bits, a.group, one, fast, layer, a.tab != nullptr);
  // NVFP4 (group 16) sizes its LDS like groups of 32 (SPU = 4 in the kernel)
  const size_t lds = layer ? layer_lds_total(a.T, a.k, a.E, a.H, a.I, a.group == 16 ? 32 : a.group)
                           : decode_lds_bytes(a.H, a.I, one, a.group == 16 ? 32 : a.group);
  const int per_cu = resident_blocks_per_cu(fn, dev.device, lds);
  if (per_cu < 1) return hipErrorInvalidConfiguration;
  long blocks = (long)p.Amax * (a.I / kRows1 + a.H / kRows2);
  const long resident = (long)dev.num_cus * per_cu;
  if (blocks > resident) blocks = resident;
  if (blocks < 1) blocks = 1;
  void *args[] = {&p};
  return hipLaunchKernel(fn, dim3((unsigned)blocks), dim3(256), args, lds, st);
}

hipError_t launch_ffn_decode(const FfnArgs &a, const DeviceInfo &dev, hipStream_t st) {
  DecodeParams p;
  fill_params(p, a, a.ws);
  return launch_decode(p, a, false, dev, st);
}

// Fused layer workspace: control block, tagged h, tagged logits, tagged y_perm.
static size_t al256(size_t v) { return (v + 255) / 256 * 256; }
size_t layer_workspace_bytes(int T, int k, int E, int H, int I) {
  const size_t n = (size_t)T * k;
  return ffn_ctl_bytes(T, k, E) + al256(n * I * 4) + al256((size_t)T * E * 8) + al256(n * H * 4) + al256(n * 8);
}

bool layer_shape_ok(int T, int k, int E, int H, int I, int bits, int group) {
  if (group == 16) group = 32;  // NVFP4 sizes its LDS like groups of 32
  return T >= 1 && T <= kLayerMaxT && (long)T * k <= 4 * kWave && E <= (1 << kRecIdBits) &&
         decode_layout_ok(H, I, bits, group) && layer_lds_total(T, k, E, H, I, group) <= 64 * 1024;
}

hipError_t launch_layer_decode(const FfnArgs &a, const LayerArgs &l, const DeviceInfo &dev, hipStream_t st) {
  DecodeParams p;
  fill_params(p, a, a.ws);
  const size_t n = (size_t)a.T * a.k;
  char *base = (char *)a.ws + ffn_ctl_bytes(a.T, a.k, a.E);
  p.hbuf = (uint32_t *)base;
  p.tl = (uint64_t *)(base + al256(n * a.I * 4));
  p.ybuf = (uint32_t *)(base + al256(n * a.I * 4) + al256((size_t)a.T * a.E * 8));
  p.rec = (uint64_t *)((char *)p.ybuf + al256(n * a.H * 4));
  p.w_router = l.w_router;
  p.bias = l.bias;
  p.y = l.y;
  p.ids_out = l.ids;
  p.gates_out = l.gates;
  p.logits_out = l.logits;
  return launch_decode(p, a, true, dev, st);
}

}  // namespace bqmoe
