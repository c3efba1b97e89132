// Tile shapes of the tiled forward, shared by the host dispatcher and the
// kernel instantiations so both agree on block_m.
#pragma once

#include "../../include/vlp.h"

namespace vlp {

// Waves per workgroup (32 query rows each) and keys per inner step.  Four
// waves (128-row tiles) for 16-bit head dims 64 and 128: each K/V block in
// LDS then serves 128 query rows (the encoder batch, D = 64: 8 % faster than
// 64-row tiles).
constexpr int tile_waves(int dtype, int head_dim) {
  return dtype == VLP_FP32 ? 2 : (head_dim >= 64 ? 4 : 2);
}
constexpr int tile_block_n(int dtype, int /*head_dim*/) { return dtype == VLP_FP32 ? 32 : 64; }
constexpr bool head_dim_built(int head_dim) {
  return head_dim == 16 || head_dim == 32 || head_dim == 64 || head_dim == 128;
}

}  // namespace vlp
