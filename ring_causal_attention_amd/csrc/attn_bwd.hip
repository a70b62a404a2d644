// Blockwise attention backward for gfx950 (placeholder until the kernels land).
#include "common.hpp"
#include "kernels.hpp"

namespace lwm {
hipError_t launch_attn_bwd(const BwdParams& p, hipStream_t stream) {
  (void)p;
  (void)stream;
  return hipErrorNotSupported;
}
}  // namespace lwm
