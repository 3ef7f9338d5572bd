// MFMA paged attention kernels for bf16_t elements.
#include "attn_mfma_launch.h"

namespace pa {

hipError_t launch_attn_mfma_bf16(const AttnParams& p, const AttnPlan& plan, int head_dim,
                               int page_size, int batch, hipStream_t stream) {
  return launch_attn_mfma_t<bf16_t>(p, plan, head_dim, page_size, batch, stream);
}

}  // namespace pa
