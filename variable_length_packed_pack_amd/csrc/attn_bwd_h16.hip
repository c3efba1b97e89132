// Tiled packed-attention backward for 16-bit inputs (bf16 and fp16): template
// instances.
#include "attn_bwd_launch.h"

namespace vlp {

hipError_t launch_attn_bwd_dq_bf16(const BwdArgs& a, int head_dim, bool causal, int64_t blocks,
                                   int32_t workers, hipStream_t s) {
  return bwd_launch<VLP_BF16, false>(a, head_dim, causal, blocks, workers, s);
}

hipError_t launch_attn_bwd_dkdv_bf16(const BwdArgs& a, int head_dim, bool causal, int64_t blocks,
                                   int32_t workers, hipStream_t s) {
  return bwd_launch<VLP_BF16, true>(a, head_dim, causal, blocks, workers, s);
}

hipError_t launch_attn_bwd_dq_f16(const BwdArgs& a, int head_dim, bool causal, int64_t blocks,
                                   int32_t workers, hipStream_t s) {
  return bwd_launch<VLP_FP16, false>(a, head_dim, causal, blocks, workers, s);
}

hipError_t launch_attn_bwd_dkdv_f16(const BwdArgs& a, int head_dim, bool causal, int64_t blocks,
                                   int32_t workers, hipStream_t s) {
  return bwd_launch<VLP_FP16, true>(a, head_dim, causal, blocks, workers, s);
}

}  // namespace vlp
