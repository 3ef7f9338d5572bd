// MFMA paged attention over 8-bit K/V codes, bf16 queries and outputs.
#include "attn_mfma_launch.h"

namespace pa {

hipError_t launch_attn_mfma_q_bf16(const AttnParams& p, const AttnPlan& plan, int kv_dtype,
                                  int head_dim, int page_size, int batch, hipStream_t stream) {
  return launch_attn_mfma_q_t<bf16_t>(p, plan, kv_dtype, head_dim, page_size, batch, stream);
}

}  // namespace pa
