// Stable grouping of the T*k (token, slot) rows by expert: a counting sort in
// one 1024-thread block.  Every step is order-independent (LDS counting) or
// done in row order by one wave, so the result is deterministic and equal to a
// stable sort of the rows by expert id.
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

}  // namespace

size_t permute_workspace_bytes(int, int, int) { return 0; }

hipError_t launch_permute(const int32_t *ids, int T, int k, int E, int32_t *offsets, int32_t *sorted_rows,
                          int32_t *row_pos, int32_t *active, void *, hipStream_t st) {
  const int n = T * k;
  const int slots = 1 + (E < n ? E : n);
  if (n <= kSmallN) {
    permute_small_kernel<<<1, kSmallN, 0, st>>>(ids, n, E, offsets, sorted_rows, row_pos, active, slots);
  } else {
    const size_t lds = (size_t)(kWaves * E + kWaves) * sizeof(int);
    permute_kernel<<<1, 1024, lds, st>>>(ids, n, E, offsets, sorted_rows, row_pos, active, slots);
  }
  return hipGetLastError();
}

}  // namespace bqmoe
