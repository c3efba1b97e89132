// Tile shapes of the tiled forward, shared by the host dispatcher and the
// kernel instantiations so both agree on block_m.
#pragma once

#include "../../include/vlp.h"

namespace vlp {

// Waves per workgroup (32 query rows each) and keys per inner step.  Four
// waves (128-row tiles) for 16-bit head dims 64 and 128 and for fp32 head
// dim 64: each K/V block in LDS then serves 128 query rows (D = 64: the
// encoder batch 8 % and the fp32 graph batch ~6 % faster than with 64-row
// tiles).  fp32 at D = 128 keeps two: four would not fit its registers.
constexpr int tile_waves(int dtype, int head_dim) {
  return dtype == VLP_FP32 ? (head_dim == 64 ? 4 : 2) : (head_dim >= 64 ? 4 : 2);
}
constexpr int tile_block_n(int dtype, int /*head_dim*/) { return dtype == VLP_FP32 ? 32 : 64; }
// 16-bit inputs at head dim 128 run the two-group forward (eight waves,
// 256-row tiles; attn_fwd_pingpong.h); the backward keeps tile_waves.
constexpr bool fwd_pingpong(int dtype, int head_dim) { return dtype != VLP_FP32 && head_dim == 128; }
// Query rows per tile of the forward kernels.
constexpr int fwd_block_m(int dtype, int head_dim) {
  return fwd_pingpong(dtype, head_dim) ? 256 : 32 * tile_waves(dtype, head_dim);
}
constexpr bool head_dim_built(int head_dim) {
  return head_dim == 16 || head_dim == 32 || head_dim == 64 || head_dim == 128;
}

}  // namespace vlp
