// One calibration step for the angles: kernel parameters and launches.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bfly {

constexpr int CALIB_THREADS = 256;
constexpr int CALIB_EPT = 8;          // consecutive elements per thread
constexpr int CALIB_MAX_BINS = 32;
constexpr int CALIB_MAX_BLOCKS = 2048;

struct CalibLossParams {
  float* y;             // [rows][n]: Y = Q X in, dL/dY out (grad pass, in place)
  int64_t rows;
  int32_t n, group, bits, bins;
  float lambda_kl;
  float* partials;      // [blocks][bins + 1]: soft-histogram sums, squared error
  float* lb;            // [bins]: log(bins * p_b) of the smoothed histogram
  float* loss;          // [3]: total, reconstruction, KL
};

int calib_blocks(int64_t rows, int n);
hipError_t launch_calib_hist(const CalibLossParams& p, hipStream_t s);
hipError_t launch_calib_reduce(const CalibLossParams& p, hipStream_t s);
hipError_t launch_calib_grad(const CalibLossParams& p, hipStream_t s);
hipError_t launch_adam(float* theta, float* m, float* v, const float* g, int count, int step,
                       float lr, float beta1, float beta2, float eps, hipStream_t s);

}  // namespace bfly
