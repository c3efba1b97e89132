// Launch templates of the tiled backward (see attn_bwd_mfma.h); each element
// type's translation unit instantiates them.
#pragma once

#include "attn_bwd_mfma.h"
#include "tile_config.h"

namespace vlp {

// Query rows per streamed block of the dK/dV kernel.
constexpr int kBwdBlockQ = 64;

template <typename Kernel>
hipError_t bwd_go(Kernel kernel, int threads, const BwdArgs& a, int64_t blocks, int32_t workers, hipStream_t s) {
  int64_t width = 0;
  const hipError_t e = launch_width(kernel, threads, blocks, workers, &width);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kernel, dim3(static_cast<unsigned>(width)), dim3(threads), 0, s, a);
  return hipGetLastError();
}

template <int DT, int D, bool CAUSAL>
hipError_t bwd_dq_go(const BwdArgs& a, int64_t blocks, int32_t workers, hipStream_t s) {
  constexpr int NW = tile_waves(DT, D);
  constexpr int BN = tile_block_n(DT, D);
  return workers == kStaticGrid
             ? bwd_go(attn_bwd_dq_h16<DT, D, NW, BN, CAUSAL, false>, NW * 64, a, blocks, workers, s)
             : bwd_go(attn_bwd_dq_h16<DT, D, NW, BN, CAUSAL, true>, NW * 64, a, blocks, workers, s);
}

template <int DT, int D, bool CAUSAL>
hipError_t bwd_dkdv_go(const BwdArgs& a, int64_t blocks, int32_t workers, hipStream_t s) {
  constexpr int NW = VLP_BWD_BLOCK_K / 32;  // key tiles of the key grid
  return workers == kStaticGrid
             ? bwd_go(attn_bwd_dkdv_h16<DT, D, NW, kBwdBlockQ, CAUSAL, false>, NW * 64, a, blocks, workers, s)
             : bwd_go(attn_bwd_dkdv_h16<DT, D, NW, kBwdBlockQ, CAUSAL, true>, NW * 64, a, blocks, workers, s);
}

template <int DT, bool DKDV>
hipError_t bwd_launch(const BwdArgs& a, int head_dim, bool causal, int64_t blocks, int32_t workers, hipStream_t s) {
  if (blocks <= 0) return hipSuccess;
#define VLP_BWD_CASE(D)                                                                     \
  case D:                                                                                   \
    if (DKDV)                                                                               \
      return causal ? bwd_dkdv_go<DT, D, true>(a, blocks, workers, s)                       \
                    : bwd_dkdv_go<DT, D, false>(a, blocks, workers, s);                     \
    return causal ? bwd_dq_go<DT, D, true>(a, blocks, workers, s)                           \
                  : bwd_dq_go<DT, D, false>(a, blocks, workers, s);
  switch (head_dim) {
    VLP_BWD_CASE(16)
    VLP_BWD_CASE(32)
    VLP_BWD_CASE(64)
    VLP_BWD_CASE(128)
    default: return hipErrorInvalidValue;
  }
#undef VLP_BWD_CASE
}

}  // namespace vlp
