// Back-to-back GEMM kernels (placeholder until the fused kernels land).
#include "cf_launch.h"

namespace cf {

bool b2b_supported(const B2bParams& p) {
  (void)p;
  return false;
}

hipError_t launch_b2b(const B2bParams& p, hipStream_t stream) {
  (void)p;
  (void)stream;
  return hipErrorNotSupported;
}

}  // namespace cf
