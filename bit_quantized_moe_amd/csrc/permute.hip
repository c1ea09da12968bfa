// Stable grouping of the T*k (token, slot) rows by expert: a counting sort.
// Every step is order-independent (counting) or done in row order by one
// wave, so the result is deterministic and equal to a stable sort of the rows
// by expert id.  Three variants by size: all rows ranked in one block
// (n <= 256), one 1024-thread block (n <= kOneBlockMax), and two launches over
// blocks of rows for larger batches.
#include "common.cuh"
#include "internal.h"

namespace bqmoe {
namespace {

constexpr int kWaves = 16;

// Block-wide exclusive scan of one int per thread (1024 threads).  Returns the
// exclusive prefix; *total receives the sum.
__device__ int block_exclusive_scan(int v, int *scratch /* [kWaves] */, int *total) {
  const int lane = lane_id();
  const int wave = threadIdx.x / kWave;
  int inc = v;
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    const int o = __shfl_up(inc, d, kWave);
    if (lane >= d) inc += o;
  }
  if (lane == kWave - 1) scratch[wave] = inc;
  __syncthreads();
  int base = 0, tot = 0;
  for (int w = 0; w < kWaves; ++w) {
    const int s = scratch[w];
    if (w < wave) base += s;
    tot += s;
  }
  __syncthreads();
  *total = tot;
  return base + inc - v;
}

__global__ void __launch_bounds__(1024) permute_kernel(const int32_t *__restrict__ ids, int n, int E,
                                                       int32_t *offsets, int32_t *sorted_rows,
                                                       int32_t *row_pos, int32_t *active, int n_active_slots) {
  extern __shared__ int sm[];
  int *hist = sm;                        // [kWaves][E]: per-wave counts, then per-wave cursors
  int *scr = sm + kWaves * E;            // [kWaves]
  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wave = tid / kWave;
  const int per = ((n + kWaves - 1) / kWaves + kWave - 1) / kWave * kWave;  // rows per wave, multiple of 64
  const int r0 = wave * per;
  const int r1 = min(n, r0 + per);

  for (int i = tid; i < kWaves * E; i += blockDim.x) hist[i] = 0;
  __syncthreads();
  // A: per-wave histograms (LDS atomics: the counts do not depend on order)
  for (int r = r0 + lane; r < r1; r += kWave) {
    const int id = ids[r];
    if (id >= 0 && id < E) atomicAdd(&hist[wave * E + id], 1);
  }
  __syncthreads();
  // B: expert totals -> offsets; per-wave cursors; active list
  int total = 0;
  if (tid < E)
    for (int w = 0; w < kWaves; ++w) total += hist[w * E + tid];
  int valid_rows = 0;
  const int off = block_exclusive_scan(tid < E ? total : 0, scr, &valid_rows);
  if (tid < E) {
    offsets[tid] = off;
    int cur = off;
    for (int w = 0; w < kWaves; ++w) {
      const int c = hist[w * E + tid];
      hist[w * E + tid] = cur;
      cur += c;
    }
  }
  if (tid == 0) offsets[E] = valid_rows;
  int n_act = 0;
  const int apos = block_exclusive_scan((tid < E && total > 0) ? 1 : 0, scr, &n_act);
  if (tid < E && total > 0) active[1 + apos] = tid;
  for (int i = 1 + n_act + tid; i < n_active_slots; i += blockDim.x) active[i] = -1;
  if (tid == 0) active[0] = n_act;
  __syncthreads();
  // C: each wave places its rows in row order, 64 at a time
  int nbits = 1;
  while ((1 << nbits) < E + 2) ++nbits;
  int *cursor = hist + wave * E;
  for (int rb = r0; rb < r1; rb += kWave) {
    const int r = rb + lane;
    int key = E + 1;  // lanes past the end of the wave's rows
    if (r < r1) {
      const int id = ids[r];
      key = (id >= 0 && id < E) ? id : E;
    }
    uint64_t peers = __ballot(1);
    for (int b = 0; b < nbits; ++b) {
      const uint64_t m = __ballot((key >> b) & 1);
      peers &= ((key >> b) & 1) ? m : ~m;
    }
    const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    const int rank = __popcll(peers & lt);
    const int cnt = __popcll(peers);
    const bool leader = rank == 0;
    if (key < E) {
      const int pos = cursor[key] + rank;
      sorted_rows[pos] = r;
      row_pos[r] = pos;
    } else if (key == E) {
      row_pos[r] = -1;
    }
    // every lane has read its cursor before the leaders advance them
    __builtin_amdgcn_wave_barrier();
    if (leader && key < E) cursor[key] += cnt;
    __builtin_amdgcn_wave_barrier();
  }
}

// Small batches (n = T*k <= 256): one block ranks every row against all rows
// in LDS, so the whole permutation takes a handful of dependent steps.  The
// rank of row r is #{r' : (id_r', r') < (id_r, r)}, i.e. its position in the
// stable sort by expert; invalid ids take the key E and sort last.
constexpr int kSmallN = 256;

__global__ void __launch_bounds__(kSmallN) permute_small_kernel(const int32_t *__restrict__ ids, int n, int E,
                                                               int32_t *offsets, int32_t *sorted_rows,
                                                               int32_t *row_pos, int32_t *active,
                                                               int n_active_slots) {
  __shared__ int key[kSmallN];
  __shared__ int skey[kSmallN];
  __shared__ int scr[kSmallN / kWave];
  const int r = threadIdx.x;
  int my = E;
  if (r < n) {
    const int id = ids[r];
    my = (id >= 0 && id < E) ? id : E;
  }
  key[r] = my;
  __syncthreads();
  int pos = 0;
  if (r < n) {
    for (int q = 0; q < n; ++q) {
      const int kq = key[q];
      pos += (kq < my) || (kq == my && q < r);
    }
    skey[pos] = my;
    if (my < E) sorted_rows[pos] = r;
    row_pos[r] = (my < E) ? pos : -1;
  }
  __syncthreads();
  // offsets[e] = number of valid rows with id < e = lower bound of e in skey
  for (int e = r; e <= E; e += blockDim.x) {
    int lo = 0, hi = n;
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (skey[mid] < e) lo = mid + 1; else hi = mid;
    }
    offsets[e] = lo;
  }
  // active experts: heads of runs in sorted order
  const int head = (r < n && skey[r] < E && (r == 0 || skey[r] != skey[r - 1])) ? 1 : 0;
  const uint64_t m = __ballot(head);
  const int lane = lane_id(), wave = r / kWave;
  const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  const int before_in_wave = __popcll(m & lt);
  if (lane == 0) scr[wave] = __popcll(m);
  __syncthreads();
  int base = 0, total = 0;
  for (int w = 0; w < kSmallN / kWave; ++w) {
    if (w < wave) base += scr[w];
    total += scr[w];
  }
  if (head) active[1 + base + before_in_wave] = skey[r];
  for (int i = 1 + total + r; i < n_active_slots; i += blockDim.x) active[i] = -1;
  if (r == 0) active[0] = total;
}

// ------------------------------------------------------------ large batches
// Blocks of R consecutive rows (R a multiple of 64, B = ceil(n / R) blocks).
// Workspace: a block counter in its first 256 bytes, then a [B, E] int32
// table; both are zero between calls.
//
//  1. permute_count_kernel: block b counts its rows per expert in LDS and
//     publishes the counts as table row b (device-coherent stores), then
//     counts itself done.  The last block to finish turns every column e of
//     the table into the exclusive prefix over blocks (the number of rows of
//     expert e in blocks before b), takes the expert totals to offsets and
//     the active list, and clears the counter.
//  2. permute_place_kernel: block b clears its table row after reading it;
//     wave w of the block takes rows [b R + w R/4, b R + (w+1) R/4), counts
//     them per expert in LDS, and starts expert e's cursor at offsets[e] +
//     table[b][e] + the counts of waves w' < w.  It then places its rows in
//     row order, 64 at a time, by ballot matching: a row's position is its
//     expert's cursor plus the number of earlier lanes with the same expert.
constexpr int kOneBlockMax = 4096;  // larger batches take the two-launch path
constexpr int kPlaceRows = 512;     // rows per block of the two-launch path (a multiple of 64)
constexpr int kMaxBlocks = 2048;    // more rows per block beyond kMaxBlocks * kPlaceRows rows
constexpr int kCountThreads = 256;
constexpr int kScanBatch = 32;      // table loads in flight per column in the last block's scan
constexpr int kPlaceWaves = 4;      // waves per placing block; a wave takes R / 4 rows

struct PermuteGrid {
  int R, B;
};
PermuteGrid permute_grid(int n) {
  constexpr int kStep = kPlaceWaves * kWave;  // R is a multiple of 256: every wave takes whole rounds of 64
  int R = kPlaceRows;
  if ((n + R - 1) / R > kMaxBlocks) R = ((n + kMaxBlocks - 1) / kMaxBlocks + kStep - 1) / kStep * kStep;
  return PermuteGrid{R, (n + R - 1) / R};
}

// Exclusive scan over the block of kCountThreads threads, one int each.
__device__ int count_block_scan(int v, int *scr /* [kCountThreads / kWave] */, int *total) {
  const int lane = lane_id(), wave = threadIdx.x / kWave;
  int inc = v;
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    const int o = __shfl_up(inc, d, kWave);
    if (lane >= d) inc += o;
  }
  if (lane == kWave - 1) scr[wave] = inc;
  __syncthreads();
  int base = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < kCountThreads / kWave; ++w) {
    const int s = scr[w];
    if (w < wave) base += s;
    tot += s;
  }
  __syncthreads();
  *total = tot;
  return base + inc - v;
}

__global__ void __launch_bounds__(kCountThreads) permute_count_kernel(const int32_t *__restrict__ ids, int n, int E,
                                                                      int R, int *ctr, int *tab, int32_t *offsets,
                                                                      int32_t *active, int n_active_slots) {
  extern __shared__ int cnt[];  // [E]
  __shared__ int scr[kCountThreads / kWave];
  __shared__ int s_last;
  const int tid = threadIdx.x, b = blockIdx.x, B = gridDim.x;
  for (int e = tid; e < E; e += kCountThreads) cnt[e] = 0;
  __syncthreads();
  const int r1 = min(n, (b + 1) * R);
  for (int r = b * R + tid; r < r1; r += kCountThreads) {
    const int id = ids[r];
    if (id >= 0 && id < E) atomicAdd(&cnt[id], 1);
  }
  __syncthreads();
  for (int e = tid; e < E; e += kCountThreads)
    __hip_atomic_store(tab + (size_t)b * E + e, cnt[e], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  wait_vmem();  // this thread's counts are stored before the block counts itself done
  __syncthreads();
  if (tid == 0) s_last = atomicAdd(ctr, 1) == B - 1;
  __syncthreads();
  if (!s_last) return;

  // ---- the last block: column prefixes, expert totals into cnt[]
  if (tid == 0) __hip_atomic_store(ctr, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  for (int e = tid; e < E; e += kCountThreads) {
    int run = 0;
    for (int b0 = 0; b0 < B; b0 += kScanBatch) {
      int v[kScanBatch];
#pragma unroll
      for (int u = 0; u < kScanBatch; ++u)  // rows past B read the last row again and are not used
        v[u] = __hip_atomic_load(tab + (size_t)min(b0 + u, B - 1) * E + e, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
      for (int u = 0; u < kScanBatch; ++u)
        if (b0 + u < B) {
          tab[(size_t)(b0 + u) * E + e] = run;
          run += v[u];
        }
    }
    cnt[e] = run;
  }
  __syncthreads();
  // offsets: exclusive scan of the totals, each thread taking up to
  // ceil(E / kCountThreads) consecutive experts
  const int per = (E + kCountThreads - 1) / kCountThreads;
  const int e0 = min(tid * per, E), e1 = min(e0 + per, E);
  int mine = 0, mine_act = 0;
  for (int e = e0; e < e1; ++e) {
    mine += cnt[e];
    mine_act += cnt[e] > 0;
  }
  int valid = 0, n_act = 0;
  int off = count_block_scan(mine, scr, &valid);
  int apos = count_block_scan(mine_act, scr, &n_act);
  for (int e = e0; e < e1; ++e) {
    offsets[e] = off;
    off += cnt[e];
    if (cnt[e] > 0) active[1 + apos++] = e;
  }
  if (tid == 0) {
    offsets[E] = valid;
    active[0] = n_act;
  }
  for (int i = 1 + n_act + tid; i < n_active_slots; i += kCountThreads) active[i] = -1;
}

__global__ void __launch_bounds__(kPlaceWaves * kWave) permute_place_kernel(const int32_t *__restrict__ ids, int n,
                                                                            int E, int R, int *tab,
                                                                            const int32_t *offsets,
                                                                            int32_t *sorted_rows, int32_t *row_pos) {
  extern __shared__ int sm[];
  int *cursor = sm;  // [kPlaceWaves][E]: per-wave counts, then per-wave cursors
  const int tid = threadIdx.x, lane = lane_id(), wave = tid / kWave, b = blockIdx.x;
  const int per = R / kPlaceWaves;  // a multiple of 64
  const int r0 = min(n, b * R + wave * per), r1 = min(n, r0 + per);
  for (int i = tid; i < kPlaceWaves * E; i += kPlaceWaves * kWave) cursor[i] = 0;
  __syncthreads();
  // keys of the wave's rows, kept for the placing rounds: the expert, E for a
  // dropped row, E + 1 past the end
  constexpr int kMaxRounds = kPlaceRows / (kPlaceWaves * kWave);
  int key[kMaxRounds];
  const bool in_regs = per <= kMaxRounds * kWave;
#pragma unroll
  for (int j = 0; j < kMaxRounds; ++j) {
    const int r = r0 + j * kWave + lane;
    int kk = E + 1;
    if (in_regs && r < r1) {
      const int id = ids[r];
      kk = (id >= 0 && id < E) ? id : E;
    }
    key[j] = kk;
  }
  if (in_regs) {
#pragma unroll
    for (int j = 0; j < kMaxRounds; ++j)
      if (key[j] < E) atomicAdd(&cursor[wave * E + key[j]], 1);
  } else {
    for (int r = r0 + lane; r < r1; r += kWave) {
      const int id = ids[r];
      if (id >= 0 && id < E) atomicAdd(&cursor[wave * E + id], 1);
    }
  }
  __syncthreads();
  // counts -> cursors: block start (table row b, cleared here) plus the earlier waves
  for (int e = tid; e < E; e += kPlaceWaves * kWave) {
    int *t = tab + (size_t)b * E + e;
    int cur = *t + offsets[e];
    *t = 0;
#pragma unroll
    for (int w = 0; w < kPlaceWaves; ++w) {
      const int c = cursor[w * E + e];
      cursor[w * E + e] = cur;
      cur += c;
    }
  }
  __syncthreads();
  int nbits = 1;
  while ((1 << nbits) < E + 2) ++nbits;
  const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  int *cw = cursor + wave * E;
  for (int j = 0; r0 + j * kWave < r1; ++j) {
    const int r = r0 + j * kWave + lane;
    int kk;
    if (in_regs) {
      kk = key[0];
#pragma unroll
      for (int i = 1; i < kMaxRounds; ++i)
        if (i == j) kk = key[i];
    } else {
      kk = E + 1;
      if (r < r1) {
        const int id = ids[r];
        kk = (id >= 0 && id < E) ? id : E;
      }
    }
    uint64_t peers = __ballot(1);
    for (int bit = 0; bit < nbits; ++bit) {
      const uint64_t m = __ballot((kk >> bit) & 1);
      peers &= ((kk >> bit) & 1) ? m : ~m;
    }
    const int rank = __popcll(peers & lt);
    if (kk < E) {
      const int pos = cw[kk] + rank;
      sorted_rows[pos] = r;
      row_pos[r] = pos;
    } else if (kk == E) {
      row_pos[r] = -1;
    }
    // every lane has read its cursor before the leaders advance them
    __builtin_amdgcn_wave_barrier();
    if (rank == 0 && kk < E) cw[kk] += __popcll(peers);
    __builtin_amdgcn_wave_barrier();
  }
}

}  // namespace

size_t permute_workspace_bytes(int T, int k, int E) {
  const long n = (long)T * k;
  if (n <= kOneBlockMax) return 0;
  const PermuteGrid g = permute_grid((int)n);
  return 256 + ((size_t)g.B * E * sizeof(int) + 255) / 256 * 256;
}

hipError_t launch_permute(const int32_t *ids, int T, int k, int E, int32_t *offsets, int32_t *sorted_rows,
                          int32_t *row_pos, int32_t *active, void *workspace, hipStream_t st) {
  const int n = T * k;
  const int slots = 1 + (E < n ? E : n);
  if (n <= kSmallN) {
    permute_small_kernel<<<1, kSmallN, 0, st>>>(ids, n, E, offsets, sorted_rows, row_pos, active, slots);
  } else if (n <= kOneBlockMax) {
    const size_t lds = (size_t)(kWaves * E + kWaves) * sizeof(int);
    permute_kernel<<<1, 1024, lds, st>>>(ids, n, E, offsets, sorted_rows, row_pos, active, slots);
  } else {
    const PermuteGrid g = permute_grid(n);
    int *ctr = (int *)workspace, *tab = (int *)((char *)workspace + 256);
    permute_count_kernel<<<g.B, kCountThreads, (size_t)E * sizeof(int), st>>>(ids, n, E, g.R, ctr, tab, offsets,
                                                                             active, slots);
    permute_place_kernel<<<g.B, kPlaceWaves * kWave, (size_t)kPlaceWaves * E * sizeof(int), st>>>(
        ids, n, E, g.R, tab, offsets, sorted_rows, row_pos);
  }
  return hipGetLastError();
}

}  // namespace bqmoe
