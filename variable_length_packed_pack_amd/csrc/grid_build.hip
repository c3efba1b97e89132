// Device-side ragged-grid build: the CoRa metadata ("PyCoRa", "CoRa
// Metadata") computed on the GPU from a device cu_seqlens, with no host read
// ("So you wanna CUDA Graph", "Scheduling without max_seqlen": the flat tile
// list is a prefix sum of per-sequence tile counts, sized on the host by
// G_cap).
//
// One workgroup (four waves up to 256 sequences, 16 above); the sequence
// lengths are read from HBM once and kept in LDS:
//   1. tile counts ceil(len_i / block_m) and their exclusive prefix sum
//      (each thread sums a contiguous chunk of sequences; chunk totals are
//      scanned within each wave by lane shuffles, then across the waves) ->
//      block_offsets; the same scan counts the non-empty sequences, which
//      are compacted into a list; grid_mapping one tile per thread, by a
//      binary search of the offsets;
//   2. longest-first order (length descending, ties to the lower index, the
//      order of a stable sort by length) of the M non-empty sequences only,
//      so a launch sized for a sequence capacity far above M -- a
//      zero-length tail of capacity slots -- orders M keys, not the
//      capacity: a bitonic sort of the keys ((INT32_MAX - len) << 32 | i)
//      held in registers;
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

// Two shapes: up to kSmallSeqs sequences one key per thread in four waves;
// above that 16 waves holding VLP_DEVICE_SORT_MAX_SEQS / 1024 keys each.
constexpr int kSmallSeqs = 256;
static_assert(VLP_DEVICE_SORT_MAX_SEQS % 1024 == 0, "sort capacity must be a multiple of the large workgroup");

__device__ __forceinline__ int tiles_for(int len, int block_m) {
  return len <= 0 ? 0 : 1 + (len - 1) / block_m;
}

// Lane exchanges within a wave for the sort below, VALU only (no trip
// through the LDS crossbar): DPP quad permutations (lane xor 1, 2, 3), the
// half-row and row mirrors (xor 7, 15), a half-row rotation (xor 8), and the
// row and half-wave swaps of two registers (xor 16, 32); the other distances
// are compositions of these.  A swap of x with itself leaves x's value and
// its partner's in the two results; which one holds the partner is read once
// from the swap of the lane ids (LaneSwap).
template <int CTRL>
__device__ __forceinline__ unsigned dpp(unsigned x) {
  return static_cast<unsigned>(__builtin_amdgcn_update_dpp(0, static_cast<int>(x), CTRL, 0xF, 0xF, false));
}

struct LaneSwap {
  bool second16, second32;  // the partner is the swap's second result
};

__device__ __forceinline__ LaneSwap lane_swap_roles(unsigned lane) {
  const auto r16 = __builtin_amdgcn_permlane16_swap(lane, lane, false, false);
  const auto r32 = __builtin_amdgcn_permlane32_swap(lane, lane, false, false);
  return {r16[1] == (lane ^ 16u), r32[1] == (lane ^ 32u)};
}

__device__ __forceinline__ unsigned xor16(unsigned x, const LaneSwap& ls) {
  const auto r = __builtin_amdgcn_permlane16_swap(x, x, false, false);
  return ls.second16 ? r[1] : r[0];
}

__device__ __forceinline__ unsigned xor32(unsigned x, const LaneSwap& ls) {
  const auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
  return ls.second32 ? r[1] : r[0];
}

// The value of lane (lane ^ M).
template <int M>
__device__ __forceinline__ unsigned lane_xor(unsigned x, const LaneSwap& ls) {
  if constexpr (M == 1) return dpp<0xB1>(x);
  else if constexpr (M == 2) return dpp<0x4E>(x);
  else if constexpr (M == 3) return dpp<0x1B>(x);
  else if constexpr (M == 4) return dpp<0x1B>(dpp<0x141>(x));  // xor 7, then xor 3
  else if constexpr (M == 7) return dpp<0x141>(x);
  else if constexpr (M == 8) return dpp<0x128>(x);  // rotation by half a row
  else if constexpr (M == 15) return dpp<0x140>(x);
  else if constexpr (M == 16) return xor16(x, ls);
  else if constexpr (M == 31) return dpp<0x140>(xor16(x, ls));
  else if constexpr (M == 32) return xor32(x, ls);
  else if constexpr (M == 63) return dpp<0x140>(xor16(xor32(x, ls), ls));
  else static_assert(M < 0, "no exchange for this lane distance");
}

// One compare-exchange seen from one element: the lower element of the pair
// keeps the smaller key, the upper one the larger.
__device__ __forceinline__ unsigned long long keep(unsigned long long mine, unsigned long long other, bool lower) {
  return (mine < other) == lower ? mine : other;
}

// Compare-exchange with the element at lane distance M (a mirror when M + 1
// is a power of two, else a half-cleaner step); H is the bit that tells the
// lower element of a pair.
template <int M, int H>
__device__ __forceinline__ unsigned long long wave_step(unsigned long long x, unsigned lane, const LaneSwap& ls) {
  const unsigned lo = lane_xor<M>(static_cast<unsigned>(x), ls);
  const unsigned hi = lane_xor<M>(static_cast<unsigned>(x >> 32), ls);
  return keep(x, (static_cast<unsigned long long>(hi) << 32) | lo, (lane & H) == 0);
}

// Sorts the 64 keys of a wave ascending across the lanes (bitonic network,
// each merge opening with a mirror step).
__device__ __forceinline__ unsigned long long wave_sort(unsigned long long x, unsigned lane, const LaneSwap& ls) {
  x = wave_step<1, 1>(x, lane, ls);
  x = wave_step<3, 2>(x, lane, ls);
  x = wave_step<1, 1>(x, lane, ls);
  x = wave_step<7, 4>(x, lane, ls);
  x = wave_step<2, 2>(x, lane, ls);
  x = wave_step<1, 1>(x, lane, ls);
  x = wave_step<15, 8>(x, lane, ls);
  x = wave_step<4, 4>(x, lane, ls);
  x = wave_step<2, 2>(x, lane, ls);
  x = wave_step<1, 1>(x, lane, ls);
  x = wave_step<31, 16>(x, lane, ls);
  x = wave_step<8, 8>(x, lane, ls);
  x = wave_step<4, 4>(x, lane, ls);
  x = wave_step<2, 2>(x, lane, ls);
  x = wave_step<1, 1>(x, lane, ls);
  x = wave_step<63, 32>(x, lane, ls);
  x = wave_step<16, 16>(x, lane, ls);
  x = wave_step<8, 8>(x, lane, ls);
  x = wave_step<4, 4>(x, lane, ls);
  x = wave_step<2, 2>(x, lane, ls);
  return wave_step<1, 1>(x, lane, ls);
}

// The half-cleaner steps of a merge below lane distance 64.
__device__ __forceinline__ unsigned long long wave_clean(unsigned long long x, unsigned lane, const LaneSwap& ls) {
  x = wave_step<32, 32>(x, lane, ls);
  x = wave_step<16, 16>(x, lane, ls);
  x = wave_step<8, 8>(x, lane, ls);
  x = wave_step<4, 4>(x, lane, ls);
  x = wave_step<2, 2>(x, lane, ls);
  return wave_step<1, 1>(x, lane, ls);
}

// Exclusive scans of two values per thread over the workgroup; returns the
// thread's exclusive prefixes and writes the totals to *total.
template <int WAVES>
__device__ int2 block_exclusive_scan2(int2 v, int2* wave_sums, int2* total) {
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  int2 incl = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int tx = __shfl_up(incl.x, off);
    const int ty = __shfl_up(incl.y, off);
    if (lane >= off) {
      incl.x += tx;
      incl.y += ty;
    }
  }
  if (lane == 63) wave_sums[w] = incl;
  __syncthreads();
  int2 base = make_int2(0, 0), tot = make_int2(0, 0);
#pragma unroll
  for (int i = 0; i < WAVES; ++i) {
    const int2 x = wave_sums[i];
    base.x += i < w ? x.x : 0;
    base.y += i < w ? x.y : 0;
    tot.x += x.x;
    tot.y += x.y;
  }
  *total = tot;
  __syncthreads();  // wave_sums may be reused by the next scan
  return make_int2(base.x + incl.x - v.x, base.y + incl.y - v.y);
}

template <int THREADS, int MAX_SEQS>
__global__ __launch_bounds__(THREADS) void grid_build_kernel(const int32_t* __restrict__ cu, int num_seqs,
                                                             int block_m, int32_t* __restrict__ block_offsets,
                                                             int32_t* __restrict__ grid_mapping,
                                                             int32_t* __restrict__ tile_order, int grid_cap,
                                                             int32_t* __restrict__ task_counter,
                                                             int32_t* __restrict__ zero, int zero_count) {
  constexpr int kWaves = THREADS / 64;
  constexpr int kItems = MAX_SEQS / THREADS;  // sort keys held per thread
  static_assert(kItems * THREADS == MAX_SEQS, "sort capacity must be a multiple of the workgroup");
  __shared__ int len_s[MAX_SEQS];
  __shared__ int bo_s[MAX_SEQS];
  __shared__ int order_s[MAX_SEQS];
  __shared__ int pos_s[MAX_SEQS];
  __shared__ unsigned long long keys[2][MAX_SEQS];
  __shared__ int2 wave_sums[kWaves];
  const int tid = threadIdx.x;
  const int per = (num_seqs + THREADS - 1) / THREADS;
  const int beg = min(num_seqs, tid * per);
  const int end = min(num_seqs, beg + per);
  const bool sorted = num_seqs <= MAX_SEQS;
  if (task_counter && tid < kTaskQueues) task_counter[tid * kCounterStride] = 0;
  for (int i = tid; i < zero_count; i += THREADS) zero[i] = 0;

  // 1. block_offsets, and the compacted list of non-empty sequences (pos_s,
  // in index order), from one scan of (tile count, non-empty) pairs.
  int2 local = make_int2(0, 0);
  for (int i = beg; i < end; ++i) {
    const int len = cu[i + 1] - cu[i];
    if (sorted) len_s[i] = len;
    local.x += tiles_for(len, block_m);
    local.y += len > 0;
  }
  int2 totals;
  int2 run = block_exclusive_scan2<kWaves>(local, wave_sums, &totals);
  const int g = totals.x;
  const int m = totals.y;
  if (!sorted) {
    for (int i = beg; i < end; ++i) {
      const int nt = tiles_for(cu[i + 1] - cu[i], block_m);
      block_offsets[i] = run.x;
      for (int t = 0; t < nt; ++t)
        if (run.x + t < grid_cap) grid_mapping[run.x + t] = i;
      run.x += nt;
    }
    if (tid == 0) block_offsets[num_seqs] = g;
    for (int f = g + tid; f < grid_cap; f += THREADS) grid_mapping[f] = -1;
    for (int f = tid; f < grid_cap; f += THREADS) tile_order[f] = f < g ? f : -1;
    return;
  }
  for (int i = beg; i < end; ++i) {
    bo_s[i] = run.x;
    block_offsets[i] = run.x;
    run.x += tiles_for(len_s[i], block_m);
    if (len_s[i] > 0) pos_s[run.y++] = i;
  }
  if (tid == 0) block_offsets[num_seqs] = g;
  __syncthreads();  // len_s, bo_s and pos_s complete

  // grid_mapping, one tile per thread: the owner of tile f is the last
  // sequence that starts at or before f (empty sequences start where the
  // next one does and own nothing).
  const int gw = min(g, grid_cap);
  for (int f = tid; f < grid_cap; f += THREADS) {
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
  // sequence at rank r < m.
  // Keys ((INT32_MAX - len) << 32 | i) sorted ascending: length descending,
  // equal lengths in index order.  A bitonic sort over p2 = max(64, 2^ceil(
  // log2 m)) keys (padding ~0 sorts last), kItems keys per thread in
  // registers, element e = it * THREADS + tid.  Each merge of blocks of k
  // keys compares e with its mirror e ^ (k - 1), then with e ^ j for j = k/4
  // down to 1, the smaller key always to the lower index.  Steps within 64
  // run in registers (wave_sort, wave_clean); longer ones exchange through
  // LDS, one barrier per step (two key buffers alternate).  Waves whose
  // elements all lie at or past p2 skip the work.
  int p2 = 64;
  while (p2 < m) p2 <<= 1;
  const unsigned lane = static_cast<unsigned>(tid & 63);
  const LaneSwap ls = lane_swap_roles(lane);
  unsigned long long r[kItems];
#pragma unroll
  for (int it = 0; it < kItems; ++it) {
    const int e = it * THREADS + tid;
    r[it] = ~0ull;
    if (e < m) {
      const int i = pos_s[e];
      r[it] = (static_cast<unsigned long long>(0x7fffffffu - static_cast<unsigned>(len_s[i])) << 32) |
              static_cast<unsigned>(i);
    }
    if (it * THREADS + (tid & ~63) < p2) r[it] = wave_sort(r[it], lane, ls);
  }
  int buf = 0;
  for (int k = 128; k <= p2; k <<= 1) {
    for (int j = k >> 1; j >= 64; j >>= 1) {
      const int mask = j == (k >> 1) ? k - 1 : j;  // the mirror opens the merge
      unsigned long long* kb = keys[buf];
#pragma unroll
      for (int it = 0; it < kItems; ++it) {
        const int e = it * THREADS + tid;
        if (e < p2) kb[e] = r[it];
      }
      __syncthreads();
#pragma unroll
      for (int it = 0; it < kItems; ++it) {
        const int e = it * THREADS + tid;
        if (e < p2) r[it] = keep(r[it], kb[e ^ mask], (e & j) == 0);
      }
      buf ^= 1;  // the next step writes the other buffer: no second barrier
    }
#pragma unroll
    for (int it = 0; it < kItems; ++it)
      if (it * THREADS + (tid & ~63) < p2) r[it] = wave_clean(r[it], lane, ls);
  }
#pragma unroll
  for (int it = 0; it < kItems; ++it) {
    const int e = it * THREADS + tid;
    if (e < m) order_s[e] = static_cast<int>(r[it] & 0xffffffffu);
  }
  __syncthreads();  // order_s complete; pos_s free again

  // 3. positions in the longest-first order (pos_s[r] = first slot of the
  // sequence at rank r), then one slot per thread: slot p belongs to the
  // last rank whose position is <= p and takes that sequence's tiles from
  // its last local tile down to tile 0.
  const int rper = (m + THREADS - 1) / THREADS;
  const int rbeg = min(m, tid * rper);
  const int rend = min(m, rbeg + rper);
  int2 rlocal = make_int2(0, 0);
  for (int r = rbeg; r < rend; ++r) rlocal.x += tiles_for(len_s[order_s[r]], block_m);
  int2 rtot;
  int pos = block_exclusive_scan2<kWaves>(rlocal, wave_sums, &rtot).x;
  for (int r = rbeg; r < rend; ++r) {
    pos_s[r] = pos;
    pos += tiles_for(len_s[order_s[r]], block_m);
  }
  __syncthreads();
  for (int p = tid; p < gw; p += THREADS) {
    int lo = 0, hi = m - 1;  // pos_s[0] = 0 <= p (p < gw implies m >= 1)
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (pos_s[mid] <= p) lo = mid; else hi = mid - 1;
    }
    const int i = order_s[lo];
    const int nt = tiles_for(len_s[i], block_m);
    tile_order[p] = bo_s[i] + nt - 1 - (p - pos_s[lo]);
  }
  for (int p = gw + tid; p < grid_cap; p += THREADS) tile_order[p] = -1;
}

}  // namespace

hipError_t launch_grid_build(const int32_t* cu_seqlens, int32_t num_seqs, int32_t block_m,
                             int32_t* block_offsets, int32_t* grid_mapping, int32_t* tile_order,
                             int64_t grid_cap, int32_t* task_counter, hipStream_t s, int32_t* zero,
                             int32_t zero_count) {
  const int zc = zero ? zero_count : 0;
  if (num_seqs <= kSmallSeqs)
    hipLaunchKernelGGL((grid_build_kernel<256, kSmallSeqs>), dim3(1), dim3(256), 0, s, cu_seqlens, num_seqs,
                       block_m, block_offsets, grid_mapping, tile_order, static_cast<int>(grid_cap), task_counter,
                       zero, zc);
  else
    hipLaunchKernelGGL((grid_build_kernel<1024, VLP_DEVICE_SORT_MAX_SEQS>), dim3(1), dim3(1024), 0, s,
                       cu_seqlens, num_seqs, block_m, block_offsets, grid_mapping, tile_order,
                       static_cast<int>(grid_cap), task_counter, zero, zc);
  return hipGetLastError();
}

}  // namespace vlp
