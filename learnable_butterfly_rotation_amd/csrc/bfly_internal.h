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
//   fgt   float4 [2(L+1)][n/8] the scaled form, in forward-thread order:
//                             row q of thread t holds what the forward
//                             kernel's thread t loads q-th, so that every
//                             load of a wave is one contiguous 1 KiB run.
//                             Rows 2s and 2s+1 (s < L-1): (beta, gamma) of
//                             the thread's pairs 0,1 and 2,3 of stage s;
//                             rows 2(L-1)+j: the last stage of its pair j
//                             with the scales folded in.  (Thread t of a
//                             forward phase with base bit b holds the eight
//                             elements whose bits b..b+2 vary; fwd_pair_slot
//                             gives the place of each pair.)
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
  const float4* fgt;
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
  t.fgt = reinterpret_cast<const float4*>(b + half * 8 * logn);
  t.lift = reinterpret_cast<const float2*>(b + half * 8 * (2 * logn + 1));
  t.last = reinterpret_cast<const float4*>(b + half * 8 * (3 * logn));
  t.eps = reinterpret_cast<const float*>(b + half * 8 * (3 * logn + 2));
  return t;
}

// Place of pair (s, p) in fgt: the forward kernel gives stage s to phase
// s / 3, whose base bit is b = min(3 (s / 3), L - 3); thread t holds the
// elements with t's bits below b, e at bits b..b+2 and t's other bits above,
// and its pair slot j is e without the pair bit s - b.  Returns the float4
// row (2s + j/2 for s < L-1, 2(L-1) + j for the last stage) times n/8 plus
// t, and sets j.
__host__ __device__ inline int64_t fwd_pair_slot(int s, int p, int logn, int& j) {
  const int i = ((p >> s) << (s + 1)) | (p & ((1 << s) - 1));  // lower element
  const int k = s / 3;
  const int b = (3 * k < logn - 3) ? 3 * k : logn - 3;
  const int e = (i >> b) & 7;
  const int t = (i & ((1 << b) - 1)) | ((i >> (b + 3)) << b);
  const int q = s - b;
  j = ((e >> (q + 1)) << q) | (e & ((1 << q) - 1));
  const int64_t T = (int64_t)1 << (logn - 3);
  const int row = s < logn - 1 ? 2 * s + (j >> 1) : 2 * (logn - 1) + j;
  return row * T + t;
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
