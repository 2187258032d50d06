// Small device utilities of the bca library (gfx950): a word fill used to
// poison workspaces (BCA_POISON=1) without hipMemsetAsync, so that the fill
// may also be recorded into a captured graph.
#include "bca_kernels.hpp"

namespace bca {
namespace {

__global__ __launch_bounds__(256) void fill_u32_kernel(uint32_t* p, size_t n, uint32_t value) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) p[i] = value;
}

}  // namespace

hipError_t launch_fill_u32(void* p, size_t nwords, uint32_t value, hipStream_t stream) {
  if (nwords == 0) return hipSuccess;
  const size_t wgs = (nwords + 255) / 256;
  const unsigned grid = (unsigned)(wgs < 4096 ? wgs : 4096);
  hipLaunchKernelGGL(fill_u32_kernel, dim3(grid), dim3(256), 0, stream, static_cast<uint32_t*>(p),
                     nwords, value);
  return hipGetLastError();
}

}  // namespace bca
