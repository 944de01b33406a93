// moe.hip -- W4A16 routed MoE (placeholder until the kernels land).
#include "internal.h"

namespace nvfp4 {

size_t moe_workspace_bytes(int tokens, int experts, int top_k, int hidden, int inter) {
  (void)tokens; (void)experts; (void)top_k; (void)hidden; (void)inter;
  return 256;
}

hipError_t launch_moe(const MoeArgs& m, hipStream_t s) {
  (void)m; (void)s;
  return hipErrorNotSupported;
}

}  // namespace nvfp4
