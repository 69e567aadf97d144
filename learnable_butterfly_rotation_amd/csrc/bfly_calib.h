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
  float* y;             // [rows][n]: Y = Q X
  float* amax;          // [rows][n / group]: the groups' max |y|, written by the histogram pass
  int64_t rows;
  int32_t n, group, bits, bins;
  float lambda_kl;
  float* partials;      // [blocks][bins + 1]: soft-histogram sums, squared error
  float* lb;            // [bins]: log(bins * p_b) of the smoothed histogram
  float* loss;          // [3]: total, reconstruction, KL
};

// Per-element quantities of the loss, shared by the histogram pass and the
// gradient (computed inside the backward kernel): the quantizer's value y^
// (symmetric absmax round to nearest even at the fp16 scale s; s == 0: 0)
// and the bin coordinate of u = y / a.
constexpr float kCalibSmooth = 1e-6f;

__device__ __forceinline__ float calib_fp16_rne(float v) {
  return (float)(_Float16)fminf(v, 65504.f);
}

__device__ __forceinline__ float calib_dequant(float y, float s, float qmax) {
  if (s == 0.f) return 0.f;
  const float q = fminf(fmaxf(rintf(y / s), -qmax), qmax);
  return q * s;
}

// lower centre j, fraction f, inside = not clamped
__device__ __forceinline__ void calib_bin(float u, int bins, int& j, float& f, bool& inside) {
  const float hb = 0.5f * (float)bins;  // 1 / h (exact for a power-of-two bin count)
  float t = fmaf(u, hb, hb - 0.5f);     // (u - c_0) / h
  inside = t >= 0.f && t <= (float)(bins - 1);
  t = fminf(fmaxf(t, 0.f), (float)(bins - 1));
  j = min((int)t, bins - 2);
  f = t - (float)j;
}

// dL/dy of one element, given its group max a (see bfly_calib.hip).  Inside
// the backward kernel, which is bound by its vector work, the two
// divisions become hardware reciprocals (1 ulp): a rounding or bin decision
// within an ulp of its boundary may then go the other way than in the
// histogram pass, which moves that element's gradient by one step.
__device__ __forceinline__ float calib_grad(float y, float a, float qmax, float inv_qmax, int bins,
                                            const float* lb, float two_n, float kl_scale) {
  const float s = calib_fp16_rne(a * inv_qmax);
  float yq = 0.f;
  if (s != 0.f) yq = fminf(fmaxf(rintf(y * __builtin_amdgcn_rcpf(s)), -qmax), qmax) * s;
  float g = two_n * (y - yq);
  if (a > 0.f) {
    const float inv_a = __builtin_amdgcn_rcpf(a);
    const float h_inv = 0.5f * (float)bins;
    float t = fmaf(y * inv_a, h_inv, h_inv - 0.5f);  // (u + 1) / h - 1/2
    if (t >= 0.f && t <= (float)(bins - 1)) {
      const int j = min((int)t, bins - 2);
      g = fmaf(kl_scale * inv_a, lb[j + 1] - lb[j], g);
    }
  }
  return g;
}

// What the backward kernel needs to form dL/dY itself from its recomputed Y.
struct CalibGradArgs {
  const float* amax;   // [rows][n / group]: the groups' max |y| (histogram pass)
  const float* lb;     // [bins]
  int32_t group, bits, bins;
  float two_n;         // 2 / N
  float kl_scale;      // lambda / (N (1 + bins 1e-6) h)
};

int calib_blocks(int64_t rows, int n);
hipError_t launch_calib_hist(const CalibLossParams& p, hipStream_t s);
hipError_t launch_calib_reduce(const CalibLossParams& p, hipStream_t s);
// The backward (pass 1 and 2) with dL/dY formed from its own Y; dx unused.
struct BwdParams;
hipError_t launch_backward_calib(const BwdParams& p, const CalibGradArgs& c, float* dtheta,
                                 hipStream_t s);
hipError_t launch_adam(float* theta, float* m, float* v, const float* g, int count, int step,
                       float lr, float beta1, float beta2, float eps, hipStream_t s);

}  // namespace bfly
