// Tiled packed-attention backward, fp32 inputs: template instances.
#include "attn_bwd_f32.h"
#include "attn_bwd_launch.h"
#include "tile_config.h"

namespace vlp {
namespace {

template <int D, bool CAUSAL, bool DKDV>
hipError_t go(const BwdArgs& a, int64_t blocks, int32_t workers, hipStream_t s) {
  constexpr int NW = tile_waves(VLP_FP32, D);     // dQ: one tile of the forward's query grid
  constexpr int NWK = VLP_BWD_BLOCK_K / 32;        // dK/dV: one tile of the key grid
  constexpr int BN = tile_block_n(VLP_FP32, D);  // keys (dQ) or queries (dK/dV) per streamed block
  const bool stat = workers == kStaticGrid;
  if (DKDV)
    return stat ? bwd_go(attn_bwd_dkdv_f32<D, NWK, BN, CAUSAL, false>, NWK * 64, a, blocks, workers, s)
                : bwd_go(attn_bwd_dkdv_f32<D, NWK, BN, CAUSAL, true>, NWK * 64, a, blocks, workers, s);
  return stat ? bwd_go(attn_bwd_dq_f32<D, NW, BN, CAUSAL, false>, NW * 64, a, blocks, workers, s)
              : bwd_go(attn_bwd_dq_f32<D, NW, BN, CAUSAL, true>, NW * 64, a, blocks, workers, s);
}

template <bool DKDV>
hipError_t launch(const BwdArgs& a, int head_dim, bool causal, int64_t blocks, int32_t workers, hipStream_t s) {
  if (blocks <= 0) return hipSuccess;
  switch (head_dim) {
    case 16: return causal ? go<16, true, DKDV>(a, blocks, workers, s) : go<16, false, DKDV>(a, blocks, workers, s);
    case 32: return causal ? go<32, true, DKDV>(a, blocks, workers, s) : go<32, false, DKDV>(a, blocks, workers, s);
    case 64: return causal ? go<64, true, DKDV>(a, blocks, workers, s) : go<64, false, DKDV>(a, blocks, workers, s);
    case 128:
      return causal ? go<128, true, DKDV>(a, blocks, workers, s) : go<128, false, DKDV>(a, blocks, workers, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_attn_bwd_dq_f32(const BwdArgs& a, int head_dim, bool causal, int64_t blocks,
                                  int32_t workers, hipStream_t s) {
  return launch<false>(a, head_dim, causal, blocks, workers, s);
}

hipError_t launch_attn_bwd_dkdv_f32(const BwdArgs& a, int head_dim, bool causal, int64_t blocks,
                                  int32_t workers, hipStream_t s) {
  return launch<true>(a, head_dim, causal, blocks, workers, s);
}

}  // namespace vlp
