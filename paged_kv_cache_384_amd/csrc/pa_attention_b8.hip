// Decode attention kernels for KV blocks of 8 tokens (the template is in pa_attention.h).
#include "pa_attention.h"

namespace pa {

hipError_t launch_decode_attention_b8(DType dt, int head_dim, const DecodeArgs& a,
                                       hipStream_t stream) {
  return launch_attn_block<8>(dt, head_dim, a, stream);
}

hipError_t launch_decode_attention_shared_b8(DType dt, const DecodeArgs& a, hipStream_t stream) {
  return launch_attn_shared_block<8>(dt, a, stream);
}

}  // namespace pa
