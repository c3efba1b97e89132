// Launch templates of the tiled backward (see attn_bwd_mfma.h); each element
// type's translation unit instantiates them.
#pragma once

#include "attn_bwd_mfma.h"
#include "tile_config.h"

namespace vlp {

// Query rows per streamed block of the dK/dV kernel.
constexpr int kBwdBlockQ = 64;

template <int DT, int D, bool CAUSAL>
hipError_t bwd_dq_go(const BwdArgs& a, int64_t blocks, hipStream_t s) {
  constexpr int NW = tile_waves(DT, D);
  constexpr int BN = tile_block_n(DT, D);
  hipLaunchKernelGGL((attn_bwd_dq_h16<DT, D, NW, BN, CAUSAL>), dim3(static_cast<unsigned>(blocks)), dim3(NW * 64),
                     0, s, a);
  return hipGetLastError();
}

template <int DT, int D, bool CAUSAL>
hipError_t bwd_dkdv_go(const BwdArgs& a, int64_t blocks, hipStream_t s) {
  constexpr int NW = VLP_BWD_BLOCK_K / 32;  // key tiles of the key grid
  hipLaunchKernelGGL((attn_bwd_dkdv_h16<DT, D, NW, kBwdBlockQ, CAUSAL>), dim3(static_cast<unsigned>(blocks)),
                     dim3(NW * 64), 0, s, a);
  return hipGetLastError();
}

template <int DT, bool DKDV>
hipError_t bwd_launch(const BwdArgs& a, int head_dim, bool causal, int64_t blocks, hipStream_t s) {
  if (blocks <= 0) return hipSuccess;
#define VLP_BWD_CASE(D)                                                                             \
  case D:                                                                                           \
    if (DKDV) return causal ? bwd_dkdv_go<DT, D, true>(a, blocks, s) : bwd_dkdv_go<DT, D, false>(a, blocks, s); \
    return causal ? bwd_dq_go<DT, D, true>(a, blocks, s) : bwd_dq_go<DT, D, false>(a, blocks, s);
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
