// Decode attention kernels for KV blocks of 16 tokens (the template is in pa_attention.h).
#include "pa_attention.h"

namespace pa {

hipError_t launch_decode_attention_b16(DType dt, int head_dim, const DecodeArgs& a,
                                       hipStream_t stream) {
  return launch_attn_block<16>(dt, head_dim, a, stream);
}

hipError_t launch_decode_attention_shared_b16(DType dt, const DecodeArgs& a, hipStream_t stream) {
  return launch_attn_shared_block<16>(dt, a, stream);
}

}  // namespace pa
