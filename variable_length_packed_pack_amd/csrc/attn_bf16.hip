// Tiled packed-attention forward, bf16 inputs: template instances and launcher.
// The kernels are described in attn_fwd_mfma.h and (head dim 128)
// attn_fwd_pingpong.h.
#include "attn_fwd_mfma.h"
#include "attn_fwd_pingpong.h"
#include "tile_config.h"

namespace vlp {
namespace {

template <int D, bool CAUSAL>
hipError_t go(const AttnArgs& a, int64_t blocks, int32_t workers, hipStream_t s) {
  if constexpr (fwd_pingpong(VLP_BF16, D)) {
    constexpr int BN = tile_block_n(VLP_BF16, D);
    const auto kernel = workers == kStaticGrid ? attn_fwd_h16_pingpong<VLP_BF16, D, BN, CAUSAL, false>
                                               : attn_fwd_h16_pingpong<VLP_BF16, D, BN, CAUSAL, true>;
    int64_t width = 0;
    const hipError_t e = launch_width(kernel, 512, blocks, workers, &width);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kernel, dim3(static_cast<unsigned>(width)), dim3(512), 0, s, a);
    return hipGetLastError();
  } else {
    constexpr int NW = tile_waves(VLP_BF16, D);
    constexpr int BN = tile_block_n(VLP_BF16, D);
    const auto kernel = workers == kStaticGrid ? attn_fwd_h16<VLP_BF16, D, NW, BN, CAUSAL, false>
                                               : attn_fwd_h16<VLP_BF16, D, NW, BN, CAUSAL, true>;
    int64_t width = 0;
    const hipError_t e = launch_width(kernel, NW * 64, blocks, workers, &width);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kernel, dim3(static_cast<unsigned>(width)), dim3(NW * 64), 0, s, a);
    return hipGetLastError();
  }
}

template <int D>
hipError_t go_d(const AttnArgs& a, bool causal, int64_t blocks, int32_t workers, hipStream_t s) {
  return causal ? go<D, true>(a, blocks, workers, s) : go<D, false>(a, blocks, workers, s);
}

}  // namespace

hipError_t launch_attn_bf16(const AttnArgs& a, int head_dim, bool causal, int64_t blocks, int32_t workers,
                           hipStream_t s) {
  if (blocks <= 0) return hipSuccess;
  switch (head_dim) {
    case 16: return go_d<16>(a, causal, blocks, workers, s);
    case 32: return go_d<32>(a, causal, blocks, workers, s);
    case 64: return go_d<64>(a, causal, blocks, workers, s);
    case 128: return go_d<128>(a, causal, blocks, workers, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace vlp
