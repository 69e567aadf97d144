// Internal interface between the C-ABI layer (bfly_api.cpp) and the HIP
// kernels.  Not installed; callers use include/bfly.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace bfly {

// Output selector for the rotated rows.
enum YKind : int { Y_NONE = -1, Y_F32 = 0, Y_BF16 = 1 };

// Everything one forward launch needs.  cs is the prepared (cos, sin) table
// [log2 nb][nb/2]; mix is the m x m Kronecker factor (nullptr when m == 1).
struct FwdParams {
  const void* x;
  void* y;
  uint8_t* codes;     // nullptr: no quantization
  uint16_t* scales;
  uint16_t* zeros;    // asymmetric mode only
  const float2* cs;
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
  const float2* cs;
  int64_t rows;
  int32_t logn;
  int32_t nblk;       // number of partial slots = grid size
};

// Kernel-launch helpers; each returns the hipError_t of the launch.
hipError_t launch_prepare(const float* theta, float2* cs, int64_t count, hipStream_t s);
hipError_t launch_forward(const FwdParams& p, hipStream_t s);
hipError_t launch_backward(const BwdParams& p, float* dtheta, hipStream_t s);

// Whether a forward instantiation exists for (lognb, m); validation uses it.
bool forward_supported(int lognb, int m);

// Grid size of the backward: a function of (rows, logn) only, so that the
// angle-gradient summation order never depends on the device.
int backward_blocks(int64_t rows, int logn);

}  // namespace bfly
