// Decode attention kernels for KV blocks of 32 tokens (the template is in pa_attention.h).
#include "pa_attention.h"

namespace pa {

hipError_t launch_decode_attention_b32(DType dt, int head_dim, const DecodeArgs& a,
                                       hipStream_t stream) {
  return launch_attn_block<32>(dt, head_dim, a, stream);
}

hipError_t launch_decode_attention_shared_b32(DType dt, const DecodeArgs& a, hipStream_t stream) {
  return launch_attn_shared_block<32>(dt, a, stream);
}

}  // namespace pa
