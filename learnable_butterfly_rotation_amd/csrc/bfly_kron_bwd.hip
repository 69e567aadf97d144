// Set-up of the Kronecker backward: the transposed mixing factor in the
// caller's workspace (and, for n_theta > 0, a zero angle set after it).  The
// backward itself is composed from the mixing kernel and the butterfly
// backward: see bfly_kron_backward.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bfly {

__global__ void kron_bwd_setup_kernel(const float* __restrict__ mix, int m, float* __restrict__ mix_t,
                                      float* __restrict__ theta0, int n_theta) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < m * m) mix_t[(i % m) * m + i / m] = mix[i];
  if (i < n_theta) theta0[i] = 0.f;
}

hipError_t launch_kron_bwd_setup(const float* mix, int m, float* mix_t, float* theta0, int n_theta,
                                 hipStream_t s) {
  const int count = n_theta > m * m ? n_theta : m * m;
  hipLaunchKernelGGL(kron_bwd_setup_kernel, dim3((count + 255) / 256), dim3(256), 0, s, mix, m,
                     mix_t, theta0, n_theta);
  return hipGetLastError();
}

}  // namespace bfly
