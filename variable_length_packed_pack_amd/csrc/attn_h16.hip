// Tiled packed-attention forward for 16-bit inputs (bf16 and fp16): template
// instances and launchers.  The kernels are described in attn_fwd_mfma.h and
// (head dim 128) attn_fwd_pingpong.h.
#include "attn_fwd_mfma.h"
#include "attn_fwd_pingpong.h"
#include "tile_config.h"

namespace vlp {
namespace {

template <int DT, int D, bool CAUSAL>
hipError_t go(const AttnArgs& a, int64_t blocks, int32_t workers, hipStream_t s) {
  if constexpr (fwd_pingpong(DT, D)) {
    constexpr int BN = tile_block_n(DT, D);
    const auto kernel = workers == kStaticGrid ? attn_fwd_h16_pingpong<DT, D, BN, CAUSAL, false>
                                               : attn_fwd_h16_pingpong<DT, D, BN, CAUSAL, true>;
    int64_t width = 0;
    const hipError_t e = launch_width(kernel, 512, blocks, workers, &width);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kernel, dim3(static_cast<unsigned>(width)), dim3(512), 0, s, a);
    return hipGetLastError();
  } else {
    constexpr int NW = tile_waves(DT, D);
    constexpr int BN = tile_block_n(DT, D);
    const auto kernel = workers == kStaticGrid ? attn_fwd_h16<DT, D, NW, BN, CAUSAL, false>
                                               : attn_fwd_h16<DT, D, NW, BN, CAUSAL, true>;
    int64_t width = 0;
    const hipError_t e = launch_width(kernel, NW * 64, blocks, workers, &width);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kernel, dim3(static_cast<unsigned>(width)), dim3(NW * 64), 0, s, a);
    return hipGetLastError();
  }
}

template <int DT, int D>
hipError_t go_d(const AttnArgs& a, bool causal, int64_t blocks, int32_t workers, hipStream_t s) {
  return causal ? go<DT, D, true>(a, blocks, workers, s) : go<DT, D, false>(a, blocks, workers, s);
}

template <int DT>
hipError_t launch_h16(const AttnArgs& a, int head_dim, bool causal, int64_t blocks, int32_t workers,
                      hipStream_t s) {
  if (blocks <= 0) return hipSuccess;
  switch (head_dim) {
    case 16: return go_d<DT, 16>(a, causal, blocks, workers, s);
    case 32: return go_d<DT, 32>(a, causal, blocks, workers, s);
    case 64: return go_d<DT, 64>(a, causal, blocks, workers, s);
    case 128: return go_d<DT, 128>(a, causal, blocks, workers, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_attn_bf16(const AttnArgs& a, int head_dim, bool causal, int64_t blocks, int32_t workers,
                           hipStream_t s) {
  return launch_h16<VLP_BF16>(a, head_dim, causal, blocks, workers, s);
}

hipError_t launch_attn_f16(const AttnArgs& a, int head_dim, bool causal, int64_t blocks, int32_t workers,
                          hipStream_t s) {
  return launch_h16<VLP_FP16>(a, head_dim, causal, blocks, workers, s);
}

}  // namespace vlp
