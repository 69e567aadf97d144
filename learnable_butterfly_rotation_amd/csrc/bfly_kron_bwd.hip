// Set-up of the Kronecker backward: the transposed mixing factor in the
// caller's workspace.  The backward itself is composed from the mixing
// kernel and the butterfly backward: see bfly_kron_backward.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bfly {

__global__ void kron_bwd_setup_kernel(const float* __restrict__ mix, int m, float* __restrict__ mix_t) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < m * m) mix_t[(i % m) * m + i / m] = mix[i];
}

hipError_t launch_kron_bwd_setup(const float* mix, int m, float* mix_t, hipStream_t s) {
  hipLaunchKernelGGL(kron_bwd_setup_kernel, dim3((m * m + 255) / 256), dim3(256), 0, s, mix, m,
                     mix_t);
  return hipGetLastError();
}

}  // namespace bfly
