// Device-side ragged-grid build: the CoRa metadata ("PyCoRa", "CoRa
// Metadata") computed on the GPU from a device cu_seqlens, with no host read
// ("So you wanna CUDA Graph", "Scheduling without max_seqlen": the flat tile
// list is a prefix sum of per-sequence tile counts, sized on the host by
// G_cap).
//
// One workgroup of 1024 threads:
//   1. tile counts ceil(len_i / block_m) and their exclusive prefix sum
//      (each thread scans a contiguous chunk of sequences; the chunk totals
//      are scanned in LDS) -> block_offsets, and grid_mapping filled per
//      sequence;
//   2. longest-first order: a bitonic sort in LDS of the 64-bit keys
//      ((INT32_MAX - len) << 32 | i), which orders by length descending with
//      ties to the lower index -- the same order as a stable sort by length;
//   3. a second prefix sum of tile counts in that order gives every
//      sequence's position in tile_order, filled last tile first.
// Entries from G to grid_cap are set to -1.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "vlp_internal.h"

namespace vlp {
namespace {

constexpr int kThreads = 1024;

__device__ __forceinline__ int tiles_for(int len, int block_m) {
  return len <= 0 ? 0 : 1 + (len - 1) / block_m;
}

// Exclusive scan of one value per thread over the workgroup; returns the
// thread's exclusive prefix and writes the total to *total.
__device__ int block_exclusive_scan(int v, int* part, int* total) {
  const int tid = threadIdx.x;
  part[tid] = v;
  __syncthreads();
  for (int off = 1; off < kThreads; off <<= 1) {
    const int add = tid >= off ? part[tid - off] : 0;
    __syncthreads();
    part[tid] += add;
    __syncthreads();
  }
  const int incl = part[tid];
  *total = part[kThreads - 1];
  __syncthreads();
  return incl - v;
}

__global__ __launch_bounds__(kThreads) void grid_build_kernel(const int32_t* __restrict__ cu, int num_seqs,
                                                              int block_m, int32_t* __restrict__ block_offsets,
                                                              int32_t* __restrict__ grid_mapping,
                                                              int32_t* __restrict__ tile_order, int grid_cap) {
  __shared__ int part[kThreads];
  __shared__ unsigned long long keys[VLP_DEVICE_SORT_MAX_SEQS];
  __shared__ int bo_lds[VLP_DEVICE_SORT_MAX_SEQS];
  const int tid = threadIdx.x;
  const int per = (num_seqs + kThreads - 1) / kThreads;
  const int beg = min(num_seqs, tid * per);
  const int end = min(num_seqs, beg + per);
  const bool sorted = num_seqs <= VLP_DEVICE_SORT_MAX_SEQS;

  // 1. block_offsets and grid_mapping.
  int local = 0;
  for (int i = beg; i < end; ++i) local += tiles_for(cu[i + 1] - cu[i], block_m);
  int g = 0;
  int run = block_exclusive_scan(local, part, &g);
  for (int i = beg; i < end; ++i) {
    const int nt = tiles_for(cu[i + 1] - cu[i], block_m);
    block_offsets[i] = run;
    if (sorted) bo_lds[i] = run;
    for (int t = 0; t < nt; ++t)
      if (run + t < grid_cap) grid_mapping[run + t] = i;
    run += nt;
  }
  if (tid == 0) block_offsets[num_seqs] = g;
  for (int f = g + tid; f < grid_cap; f += kThreads) {
    grid_mapping[f] = -1;
    tile_order[f] = -1;
  }

  if (!sorted) {
    for (int f = tid; f < g && f < grid_cap; f += kThreads) tile_order[f] = f;
    return;
  }

  // 2. bitonic sort of (length descending, index ascending).
  int p2 = 1;
  while (p2 < num_seqs) p2 <<= 1;
  for (int i = tid; i < p2; i += kThreads) {
    if (i < num_seqs) {
      const unsigned len = static_cast<unsigned>(cu[i + 1] - cu[i]);
      keys[i] = (static_cast<unsigned long long>(0x7fffffffu - len) << 32) | static_cast<unsigned>(i);
    } else {
      keys[i] = ~0ull;
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

  // 3. positions in the longest-first order, then the tiles of each sequence
  // from its last local tile down to tile 0.
  local = 0;
  for (int r = beg; r < end; ++r) {
    const int i = static_cast<int>(keys[r] & 0xffffffffu);
    local += tiles_for(cu[i + 1] - cu[i], block_m);
  }
  int dummy = 0;
  int pos = block_exclusive_scan(local, part, &dummy);
  for (int r = beg; r < end; ++r) {
    const int i = static_cast<int>(keys[r] & 0xffffffffu);
    const int nt = tiles_for(cu[i + 1] - cu[i], block_m);
    const int first = bo_lds[i];
    for (int u = 0; u < nt; ++u)
      if (pos + u < grid_cap) tile_order[pos + u] = first + nt - 1 - u;
    pos += nt;
  }
}

}  // namespace

hipError_t launch_grid_build(const int32_t* cu_seqlens, int32_t num_seqs, int32_t block_m,
                             int32_t* block_offsets, int32_t* grid_mapping, int32_t* tile_order,
                             int64_t grid_cap, hipStream_t s) {
  hipLaunchKernelGGL(grid_build_kernel, dim3(1), dim3(kThreads), 0, s, cu_seqlens, num_seqs, block_m,
                     block_offsets, grid_mapping, tile_order, static_cast<int>(grid_cap));
  return hipGetLastError();
}

}  // namespace vlp
