// Grouped GEMM for the MX format (e4m3 activations x e2m1 weights with UE8M0
// per-32 scales).  Not built yet: the launcher reports "not supported".
#include "device_common.h"
#include "internal.h"

namespace moe {

hipError_t launch_gemm_mx(const GemmParams& p, int epi, bool paired, int num_cus, hipStream_t stream) {
  (void)p; (void)epi; (void)paired; (void)num_cus; (void)stream;
  return hipErrorNotSupported;
}

}  // namespace moe
