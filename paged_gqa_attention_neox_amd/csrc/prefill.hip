// Varlen causal prefill dispatch.  (The bf16 matrix-core kernel is added
// here; until then every shape runs the generic kernel.)
#include "kernels.h"

namespace qw {

hipError_t launch_prefill(const AttnArgs& a, hipStream_t stream) {
  return launch_attn_generic(a, stream);
}

}  // namespace qw
