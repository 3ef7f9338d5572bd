// Vector-ALU paged attention kernels for float elements.
#include "attn_valu_launch.h"

namespace pa {

hipError_t launch_attn_valu_f32(const AttnParams& p, const AttnPlan& plan, int head_dim,
                               int page_size, int batch, hipStream_t stream) {
  return launch_attn_valu_t<float>(p, plan, head_dim, page_size, batch, stream);
}

}  // namespace pa
