// The layer-output calibration step's own kernels (bfly_calib_w.hip).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bfly {

// Workgroup tiles of launch_gemm_f32 (also the number of sum-of-squares
// partials it writes).
int64_t gemm_f32_tiles(int64_t M, int32_t N);
// C[M][N] = alpha * A B with A row-major [M][K]; B row-major [N][K] when
// b_transposed (C = A B^T), else [K][N].  K % 16 == 0; every matrix below
// 4 GiB.  ss (optional): gemm_f32_tiles(M, N) partial sums of squares of C.
hipError_t launch_gemm_f32(const float* A, const float* B, bool b_transposed, float* C, int64_t M,
                           int32_t N, int32_t K, float alpha, float* ss, hipStream_t s);
// wr [out][n] <- (quantizer's value of wr) - wr, from the codes, scales
// (and zero points) bfly_forward_quant wrote for it.
hipError_t launch_quant_residual(float* wr, const uint8_t* codes, const uint16_t* scales,
                                 const uint16_t* zeros, int64_t out, int32_t n, int32_t bits,
                                 int32_t group, bool asym, hipStream_t s);
// g [count] += the uniformity term's gradient at xr (group maxima amax
// [count / group], log-bins lb [bins]).
hipError_t launch_kl_grad_add(const float* xr, const float* amax, const float* lb, float* g,
                              int64_t count, int32_t group, int32_t bins, float kl_scale,
                              hipStream_t s);
// loss[1] = sum(ss) / n_rec; loss[0] = loss[1] + lambda * loss[2].
hipError_t launch_weight_loss(const float* ss, int64_t nparts, double n_rec, float lambda_kl,
                              float* loss, hipStream_t s);

}  // namespace bfly
