// Device-side ragged-grid build: the CoRa metadata ("PyCoRa", "CoRa
// Metadata") computed on the GPU from a device cu_seqlens, with no host read
// ("So you wanna CUDA Graph", "Scheduling without max_seqlen": the flat tile
// list is a prefix sum of per-sequence tile counts, sized on the host by
// G_cap).
//
// One workgroup of 256 threads (four waves); the sequence lengths are read
// from HBM once and kept in LDS:
//   1. tile counts ceil(len_i / block_m) and their exclusive prefix sum
//      (each thread sums a contiguous chunk of sequences; chunk totals are
//      scanned within each wave by lane shuffles, then across the four
//      waves) -> block_offsets; grid_mapping one tile per thread, by a
//      binary search of the offsets;
//   2. longest-first order (length descending, ties to the lower index, the
//      order of a stable sort by length) of the M non-empty sequences only:
//      they are compacted first (a scan of the non-empty flags), so a launch
//      sized for a sequence capacity far above M -- a zero-length tail of
//      capacity slots -- orders M keys, not the capacity.  For up to kRankMax
//      of them every sequence counts the larger keys (len << 32 | ~i); above
//      that, a bitonic sort in LDS of the keys ((INT32_MAX - len) << 32 | i);
//   3. a second prefix sum of tile counts in that order gives every
//      sequence's position in tile_order; each slot is filled by its own
//      thread (binary search of the positions), last tile first.
// Entries from G to grid_cap are set to -1.  The kernel also clears the
// work-queue counters of the persistent launch that follows it, if given.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "vlp_internal.h"

namespace vlp {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kRankMax = 256;  // rank counting below this many sequences, bitonic sort above

__device__ __forceinline__ int tiles_for(int len, int block_m) {
  return len <= 0 ? 0 : 1 + (len - 1) / block_m;
}

// Exclusive scan of one value per thread over the workgroup; returns the
// thread's exclusive prefix and writes the total to *total.
__device__ int block_exclusive_scan(int v, int* wave_sums, int* total) {
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  int incl = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int t = __shfl_up(incl, off);
    if (lane >= off) incl += t;
  }
  if (lane == 63) wave_sums[w] = incl;
  __syncthreads();
  int base = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < kWaves; ++i) {
    const int x = wave_sums[i];
    base += i < w ? x : 0;
    tot += x;
  }
  *total = tot;
  __syncthreads();  // wave_sums may be reused by the next scan
  return base + incl - v;
}

__global__ __launch_bounds__(kThreads) void grid_build_kernel(const int32_t* __restrict__ cu, int num_seqs,
                                                              int block_m, int32_t* __restrict__ block_offsets,
                                                              int32_t* __restrict__ grid_mapping,
                                                              int32_t* __restrict__ tile_order, int grid_cap,
                                                              int32_t* __restrict__ task_counter,
                                                              int32_t* __restrict__ zero, int zero_count) {
  __shared__ int len_s[VLP_DEVICE_SORT_MAX_SEQS];
  __shared__ int bo_s[VLP_DEVICE_SORT_MAX_SEQS];
  __shared__ int order_s[VLP_DEVICE_SORT_MAX_SEQS];
  __shared__ int pos_s[VLP_DEVICE_SORT_MAX_SEQS];
  __shared__ unsigned long long keys[VLP_DEVICE_SORT_MAX_SEQS];
  __shared__ int wave_sums[kWaves];
  const int tid = threadIdx.x;
  const int per = (num_seqs + kThreads - 1) / kThreads;
  const int beg = min(num_seqs, tid * per);
  const int end = min(num_seqs, beg + per);
  const bool sorted = num_seqs <= VLP_DEVICE_SORT_MAX_SEQS;
  if (task_counter && tid < kTaskQueues) task_counter[tid * kCounterStride] = 0;
  for (int i = tid; i < zero_count; i += kThreads) zero[i] = 0;

  // 1. block_offsets and grid_mapping.
  int local = 0;
  for (int i = beg; i < end; ++i) {
    const int len = cu[i + 1] - cu[i];
    if (sorted) len_s[i] = len;
    local += tiles_for(len, block_m);
  }
  int g = 0;
  int run = block_exclusive_scan(local, wave_sums, &g);
  if (!sorted) {
    for (int i = beg; i < end; ++i) {
      const int nt = tiles_for(cu[i + 1] - cu[i], block_m);
      block_offsets[i] = run;
      for (int t = 0; t < nt; ++t)
        if (run + t < grid_cap) grid_mapping[run + t] = i;
      run += nt;
    }
    if (tid == 0) block_offsets[num_seqs] = g;
    for (int f = g + tid; f < grid_cap; f += kThreads) grid_mapping[f] = -1;
    for (int f = tid; f < grid_cap; f += kThreads) tile_order[f] = f < g ? f : -1;
    return;
  }
  for (int i = beg; i < end; ++i) {
    bo_s[i] = run;
    block_offsets[i] = run;
    run += tiles_for(len_s[i], block_m);
  }
  if (tid == 0) block_offsets[num_seqs] = g;
  __syncthreads();  // len_s and bo_s complete

  // grid_mapping, one tile per thread: the owner of tile f is the last
  // sequence that starts at or before f (empty sequences start where the
  // next one does and own nothing).
  const int gw = min(g, grid_cap);
  for (int f = tid; f < grid_cap; f += kThreads) {
    int owner = -1;
    if (f < gw) {
      int lo = 0, hi = num_seqs - 1;  // bo_s[0] = 0 <= f
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (bo_s[mid] <= f) lo = mid; else hi = mid - 1;
      }
      owner = lo;
    }
    grid_mapping[f] = owner;
  }

  // 2. the longest-first order of the non-empty sequences: order_s[r] = the
  // sequence at rank r < m.  pos_s first holds the compacted list of
  // non-empty sequences, in index order.
  local = 0;
  for (int i = beg; i < end; ++i) local += len_s[i] > 0;
  int m = 0;
  int at = block_exclusive_scan(local, wave_sums, &m);
  for (int i = beg; i < end; ++i)
    if (len_s[i] > 0) pos_s[at++] = i;
  __syncthreads();
  if (m <= kRankMax) {
    // One 64-bit key per non-empty sequence, larger for an earlier place
    // (length in the high word, the complement of the index below it, so
    // equal lengths keep index order); a sequence's rank is the number of
    // larger keys.  Every thread reads the same key in each step (an LDS
    // broadcast), and the loads are independent of one another.
    for (int a = tid; a < m; a += kThreads) {
      const int i = pos_s[a];
      keys[a] = (static_cast<unsigned long long>(static_cast<unsigned>(len_s[i])) << 32) |
                (0xffffffffu - static_cast<unsigned>(i));
    }
    __syncthreads();
    for (int a = tid; a < m; a += kThreads) {
      const unsigned long long ka = keys[a];
      int rank = 0;
#pragma unroll 8
      for (int b = 0; b < m; ++b) rank += keys[b] > ka;
      order_s[rank] = static_cast<int>(0xffffffffu - static_cast<unsigned>(ka & 0xffffffffu));
    }
  } else {
    int p2 = 1;
    while (p2 < m) p2 <<= 1;
    for (int a = tid; a < p2; a += kThreads) {
      if (a < m) {
        const int i = pos_s[a];
        const unsigned len = static_cast<unsigned>(len_s[i]);
        keys[a] = (static_cast<unsigned long long>(0x7fffffffu - len) << 32) | static_cast<unsigned>(i);
      } else {
        keys[a] = ~0ull;
      }
    }
    __syncthreads();
    for (int k = 2; k <= p2; k <<= 1) {
      for (int j = k >> 1; j > 0; j >>= 1) {
        for (int i = tid; i < p2; i += kThreads) {
          const int ixj = i ^ j;
          if (ixj > i) {
            const unsigned long long x = keys[i], y = keys[ixj];
            const bool ascending = (i & k) == 0;
            if ((x > y) == ascending) {
              keys[i] = y;
              keys[ixj] = x;
            }
          }
        }
        __syncthreads();
      }
    }
    for (int r = tid; r < m; r += kThreads) order_s[r] = static_cast<int>(keys[r] & 0xffffffffu);
  }
  __syncthreads();  // order_s complete; pos_s free again

  // 3. positions in the longest-first order (pos_s[r] = first slot of the
  // sequence at rank r), then one slot per thread: slot p belongs to the
  // last rank whose position is <= p and takes that sequence's tiles from
  // its last local tile down to tile 0.
  const int rper = (m + kThreads - 1) / kThreads;
  const int rbeg = min(m, tid * rper);
  const int rend = min(m, rbeg + rper);
  local = 0;
  for (int r = rbeg; r < rend; ++r) local += tiles_for(len_s[order_s[r]], block_m);
  int dummy = 0;
  int pos = block_exclusive_scan(local, wave_sums, &dummy);
  for (int r = rbeg; r < rend; ++r) {
    pos_s[r] = pos;
    pos += tiles_for(len_s[order_s[r]], block_m);
  }
  __syncthreads();
  for (int p = tid; p < gw; p += kThreads) {
    int lo = 0, hi = m - 1;  // pos_s[0] = 0 <= p (p < gw implies m >= 1)
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (pos_s[mid] <= p) lo = mid; else hi = mid - 1;
    }
    const int i = order_s[lo];
    const int nt = tiles_for(len_s[i], block_m);
    tile_order[p] = bo_s[i] + nt - 1 - (p - pos_s[lo]);
  }
  for (int p = gw + tid; p < grid_cap; p += kThreads) tile_order[p] = -1;
}

}  // namespace

hipError_t launch_grid_build(const int32_t* cu_seqlens, int32_t num_seqs, int32_t block_m,
                             int32_t* block_offsets, int32_t* grid_mapping, int32_t* tile_order,
                             int64_t grid_cap, int32_t* task_counter, hipStream_t s, int32_t* zero,
                             int32_t zero_count) {
  hipLaunchKernelGGL(grid_build_kernel, dim3(1), dim3(kThreads), 0, s, cu_seqlens, num_seqs, block_m,
                     block_offsets, grid_mapping, tile_order, static_cast<int>(grid_cap), task_counter, zero,
                     zero ? zero_count : 0);
  return hipGetLastError();
}

}  // namespace vlp
