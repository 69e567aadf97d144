// Internal interface between the C-ABI layer (bfly_api.cpp) and the HIP
// kernels.  Not installed; callers use include/bfly.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace bfly {

// Output selector for the rotated rows.
enum YKind : int { Y_NONE = -1, Y_F32 = 0, Y_BF16 = 1 };

// The prepared coefficient table of a butterfly of length n = 2^L, in one
// device allocation (half = n/2 pairs per stage):
//   cs    float2 [L][half]    (cos t, sin t) of every angle (backward)
//   fg    float2 [L-1][half]  (beta, gamma): stages 0..L-2 in scaled form
//   flast float4 [half]       the last stage with the scales folded in
//   lift  float2 [L-1][half]  (p, u): stages 0..L-2 as three shears
//   last  float4 [half]       the last stage with the tracked signs folded in
//
// Scaled form (the "fast Givens" rotation): every element carries a scale
// sigma (1 on input) and the kernel stores w = x / sigma.  A rotation by t of
// the pair (i, j) becomes two fused multiply-adds on the stored values,
//   w_i <- w_i + beta w_j,  w_j <- w_j + gamma w_i  (both from the old values)
// with beta = -tan t * sigma_j / sigma_i, gamma = tan t * sigma_i / sigma_j,
// after which both scales are multiplied by cos t.  The last stage maps the
// stored values to the true outputs with the 2x2 matrix
// (c sigma_i, -s sigma_j, s sigma_i, c sigma_j).  Scales are tracked in fp64
// when the table is prepared.  Stored magnitudes grow like 1 / |sigma| (for
// angles drawn uniformly, 1/|sigma| reaches ~2^31 at n = 4096); a pair
// whose scales would fall below 2^-64 has beta set to NaN, and a forward
// launch that sees any NaN uses the three-shear form instead.
//
// Three-shear form: x += p y; y += u x; x += p y is the Givens rotation by
// an angle phi with |phi| <= pi/2 (p = -tan(phi/2), u = sin phi).  A
// rotation by t with |t| > pi/2 equals minus the rotation by t -+ pi; the
// minus is not applied but tracked as a sign on both elements, and a
// rotation of sign-carrying elements is again a rotation (by +-t).  The last
// stage maps the sign-carrying values straight to the true outputs.
//   eps   float [L-1][half]   the product of the signs the pair's two
//                             elements carry in the three-shear form (the
//                             backward's angle gradients are accumulated on
//                             signed values and multiplied by it at the end)
struct Table {
  const float2* cs;
  const float2* fg;
  const float4* flast;
  const float2* lift;
  const float4* last;
  const float* eps;
};

__host__ __device__ inline size_t table_bytes(int logn) {
  const size_t half = (size_t)1 << (logn - 1);
  return half * 8 * (size_t)(3 * logn + 2) + half * 4 * (size_t)(logn - 1);
}

__host__ __device__ inline Table table_at(const void* base, int logn) {
  const size_t half = (size_t)1 << (logn - 1);
  const char* b = static_cast<const char*>(base);
  Table t;
  t.cs = reinterpret_cast<const float2*>(b);
  t.fg = reinterpret_cast<const float2*>(b + half * 8 * logn);
  t.flast = reinterpret_cast<const float4*>(b + half * 8 * (2 * logn - 1));
  t.lift = reinterpret_cast<const float2*>(b + half * 8 * (2 * logn + 1));
  t.last = reinterpret_cast<const float4*>(b + half * 8 * (3 * logn));
  t.eps = reinterpret_cast<const float*>(b + half * 8 * (3 * logn + 2));
  return t;
}

// Everything one forward launch needs.  tab is the prepared table of the
// butterfly of length nb; mix is the m x m Kronecker factor (nullptr for a
// plain butterfly).
struct FwdParams {
  const void* x;
  void* y;
  uint8_t* codes;     // nullptr: no quantization
  uint16_t* scales;
  uint16_t* zeros;    // asymmetric mode only
  Table tab;
  const float* mix;
  int64_t rows;
  int32_t m;          // segments per row (1 = plain butterfly)
  int32_t lognb;      // log2 of the butterfly length
  int32_t x_bf16;     // 1: bf16 input, 0: fp32 input
  int32_t y_kind;     // YKind
  int32_t bits;       // 2 or 4 (ignored without codes)
  int32_t group;      // elements per quantization group
  int32_t asym;       // 1: asymmetric min-max, 0: symmetric absmax
};

struct BwdParams {
  const float* x;
  const float* g;
  float* y;           // optional
  float* dx;
  float* partials;    // [nblk][log2 n][n/2]
  Table tab;
  int64_t rows;
  int32_t logn;
  int32_t nblk;       // number of partial slots = grid size
};

// Kernel-launch helpers; each returns the hipError_t of the launch.
hipError_t launch_prepare(const float* theta, void* table, int logn, hipStream_t s);
hipError_t launch_forward(const FwdParams& p, hipStream_t s);
hipError_t launch_backward(const BwdParams& p, float* dtheta, hipStream_t s);

// Whether a forward instantiation exists for (lognb, m); validation uses it.
bool forward_supported(int lognb, int m);

// Grid size of the backward: a function of (rows, logn) only, so that the
// angle-gradient summation order never depends on the device.
int backward_blocks(int64_t rows, int logn);

}  // namespace bfly
