// Debug validation of device cu_seqlens contents (VLP_CHECK=1).
//
// The fast path never reads cu_seqlens on the host ("gigl.nn.packed_attention":
// the packed path needs no host syncs beyond the token count), so contents
// that break the contract -- cu[0] != 0, a decreasing step, a total beyond
// the rows of the buffer ("PyCoRa", "The Data Structure": offsets start at 0
// and the last one is the element count) -- give undefined results there.
// With VLP_CHECK=1 in the environment the entry points first run this check
// and wait for it, and refuse such contents with VLP_ERR_INVALID before any
// other kernel reads them.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "vlp_internal.h"

namespace vlp {
namespace {

// One workgroup; bit 0 of *bad: cu[0] != 0 or cu[num_seqs] > max_total;
// bit 1: a decreasing step; bit 2: an empty sequence where every sequence
// must be non-empty.  Only cu[0 .. num_seqs] is read.
__global__ __launch_bounds__(256) void cu_check_kernel(const int32_t* cu, int num_seqs, int64_t max_total,
                                                       int require_nonempty, int32_t* bad) {
  int flags = 0;
  if (threadIdx.x == 0 && (cu[0] != 0 || static_cast<int64_t>(cu[num_seqs]) > max_total)) flags |= 1;
  for (int i = threadIdx.x; i < num_seqs; i += blockDim.x) {
    const int32_t lo = cu[i], hi = cu[i + 1];
    if (hi < lo) flags |= 2;
    if (require_nonempty && hi == lo) flags |= 4;
  }
  if (flags) atomicOr(bad, flags);
}

}  // namespace

hipError_t check_cu_seqlens(const int32_t* cu, int32_t num_seqs, int64_t max_total, bool require_nonempty,
                            hipStream_t s, int32_t* flags) {
  *flags = 0;
  int32_t* bad = nullptr;
  hipError_t e = hipMalloc(&bad, sizeof(int32_t));
  if (e != hipSuccess) return e;
  e = hipMemsetAsync(bad, 0, sizeof(int32_t), s);
  if (e == hipSuccess) {
    hipLaunchKernelGGL(cu_check_kernel, dim3(1), dim3(256), 0, s, cu, num_seqs, max_total,
                       require_nonempty ? 1 : 0, bad);
    e = hipGetLastError();
  }
  if (e == hipSuccess) e = hipMemcpyAsync(flags, bad, sizeof(int32_t), hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  const hipError_t f = hipFree(bad);
  return e != hipSuccess ? e : f;
}

}  // namespace vlp
