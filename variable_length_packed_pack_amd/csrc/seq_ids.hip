// Document ids -> cu_seqlens on the GPU.
//
// A packed sequence whose tokens carry document ids (the sample-id mask of
// one packed sequence) is the same attention problem as a batch of
// sequences, one per run of equal ids: a query may see exactly the keys of
// its own run.  This kernel turns the ids into that batch's cu_seqlens with
// a fixed capacity ("So you wanna CUDA Graph", "Terminology time": unused
// slots repeat the total, i.e. zero-length sequences, which the attention
// kernels skip), so the whole path runs without a host read ("DanLing
// NestedTensor" 3.3: varlen kernels consume the partitions' segment
// boundaries).
//
// One workgroup of 1024 threads walks the ids in chunks of 16 consecutive
// tokens per thread: boundary flags (token 0, or an id different from the
// previous token's), an exclusive scan of the per-thread counts, then every
// thread writes its run starts in order.  The run count goes to device
// memory; if it exceeds the capacity only the first max_seqs starts are
// written and the caller must treat cu_seqlens as invalid.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "vlp_internal.h"

namespace vlp {
namespace {

constexpr int kIdThreads = 1024;
constexpr int kIdWaves = kIdThreads / 64;
constexpr int kIdPer = 16;  // consecutive tokens per thread and chunk

__device__ int ids_exclusive_scan(int v, int* wave_sums, int* total) {
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
  for (int i = 0; i < kIdWaves; ++i) {
    const int x = wave_sums[i];
    base += i < w ? x : 0;
    tot += x;
  }
  *total = tot;
  __syncthreads();  // wave_sums is reused by the next chunk
  return base + incl - v;
}

__global__ __launch_bounds__(kIdThreads) void ids_to_cu_kernel(const int32_t* __restrict__ ids, int num_tokens,
                                                               int max_seqs, int32_t* __restrict__ cu,
                                                               int32_t* __restrict__ num_out) {
  __shared__ int wave_sums[kIdWaves];
  int running = 0;  // runs that start before this chunk (the same in every thread)
  for (int64_t base = 0; base < num_tokens; base += kIdThreads * kIdPer) {
    const int64_t t0 = base + static_cast<int64_t>(threadIdx.x) * kIdPer;
    int flags = 0, cnt = 0;
    if (t0 < num_tokens) {
      int prev = t0 == 0 ? 0 : ids[t0 - 1];
      const int n = static_cast<int>(min(static_cast<int64_t>(kIdPer), num_tokens - t0));
      for (int e = 0; e < n; ++e) {
        const int x = ids[t0 + e];
        if (t0 + e == 0 || x != prev) {
          flags |= 1 << e;
          ++cnt;
        }
        prev = x;
      }
    }
    int total;
    int p = running + ids_exclusive_scan(cnt, wave_sums, &total);
    for (int e = 0; e < kIdPer; ++e)
      if ((flags >> e) & 1) {
        if (p < max_seqs) cu[p] = static_cast<int32_t>(t0 + e);
        ++p;
      }
    running += total;
  }
  for (int i = min(running, max_seqs) + static_cast<int>(threadIdx.x); i <= max_seqs; i += kIdThreads)
    cu[i] = num_tokens;
  if (threadIdx.x == 0) *num_out = running;
}

}  // namespace

hipError_t launch_ids_to_cu(const int32_t* ids, int32_t num_tokens, int32_t max_seqs, int32_t* cu, int32_t* num_out,
                            hipStream_t s) {
  hipLaunchKernelGGL(ids_to_cu_kernel, dim3(1), dim3(kIdThreads), 0, s, ids, num_tokens, max_seqs, cu, num_out);
  return hipGetLastError();
}

}  // namespace vlp
