// Tiled packed-attention backward, fp32 inputs: template instances.
#include "attn_bwd_f32.h"
#include "tile_config.h"

namespace vlp {
namespace {

template <int D, bool CAUSAL, bool DKDV>
hipError_t go(const BwdArgs& a, int64_t blocks, hipStream_t s) {
  constexpr int NW = tile_waves(VLP_FP32, D);
  constexpr int BN = tile_block_n(VLP_FP32, D);  // keys (dQ) or queries (dK/dV) per streamed block
  static_assert(32 * NW == VLP_BWD_BLOCK_K, "the dK/dV kernel covers one tile of the key grid");
  if (DKDV)
    hipLaunchKernelGGL((attn_bwd_dkdv_f32<D, NW, BN, CAUSAL>), dim3(static_cast<unsigned>(blocks)), dim3(NW * 64),
                       0, s, a);
  else
    hipLaunchKernelGGL((attn_bwd_dq_f32<D, NW, BN, CAUSAL>), dim3(static_cast<unsigned>(blocks)), dim3(NW * 64), 0,
                       s, a);
  return hipGetLastError();
}

template <bool DKDV>
hipError_t launch(const BwdArgs& a, int head_dim, bool causal, int64_t blocks, hipStream_t s) {
  if (blocks <= 0) return hipSuccess;
  switch (head_dim) {
    case 16: return causal ? go<16, true, DKDV>(a, blocks, s) : go<16, false, DKDV>(a, blocks, s);
    case 32: return causal ? go<32, true, DKDV>(a, blocks, s) : go<32, false, DKDV>(a, blocks, s);
    case 64: return causal ? go<64, true, DKDV>(a, blocks, s) : go<64, false, DKDV>(a, blocks, s);
    case 128: return causal ? go<128, true, DKDV>(a, blocks, s) : go<128, false, DKDV>(a, blocks, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_attn_bwd_dq_f32(const BwdArgs& a, int head_dim, bool causal, int64_t blocks, hipStream_t s) {
  return launch<false>(a, head_dim, causal, blocks, s);
}

hipError_t launch_attn_bwd_dkdv_f32(const BwdArgs& a, int head_dim, bool causal, int64_t blocks, hipStream_t s) {
  return launch<true>(a, head_dim, causal, blocks, s);
}

}  // namespace vlp
