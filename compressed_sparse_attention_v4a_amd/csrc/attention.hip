// Dispatch of the shared-KV MQA attention calls: the MFMA kernels for bf16 rows
// of 512 channels with heads in groups of 64, the general kernel otherwise (or
// when the general policy is forced).
#include "internal.h"

namespace v4a {

size_t attn_generic_workspace(const AttnArgs& a);
hipError_t launch_attention_generic(const AttnArgs& a, void* ws, hipStream_t s);
bool attn_mfma_supported(const AttnArgs& a);
size_t attn_mfma_workspace(const AttnArgs& a);
hipError_t launch_attention_mfma(const AttnArgs& a, void* ws, hipStream_t s);

static bool use_mfma(const AttnArgs& a, int policy) { return policy == 0 && attn_mfma_supported(a); }

size_t attn_workspace(const AttnArgs& a, int policy) {
  return use_mfma(a, policy) ? attn_mfma_workspace(a) : attn_generic_workspace(a);
}

hipError_t launch_attention(const AttnArgs& a, void* ws, int policy, hipStream_t s) {
  return use_mfma(a, policy) ? launch_attention_mfma(a, ws, s) : launch_attention_generic(a, ws, s);
}

}  // namespace v4a
