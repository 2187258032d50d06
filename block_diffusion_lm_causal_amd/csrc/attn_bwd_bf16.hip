// Backward of block-causal / staircase attention (bf16, gfx950).
#include "bca_device.hpp"
#include "bca_kernels.hpp"

namespace bca {

hipError_t launch_bwd_bf16(const BwdArgs& a, int max_seqlen, hipStream_t stream) {
  (void)a; (void)max_seqlen; (void)stream;
  return hipErrorNotSupported;
}

}  // namespace bca
