// Quantized-weight matrix product: kernel parameters and launch.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bfly {

// y[r][o] = sum_k a[r][k] * w[o][k] for r < rows, o < n_out, with
// w[o][k] = scale[o][k / group] * (q[o][k] - zero[o][k / group]) from the
// packed codes (symmetric: two's-complement q, no zero point).
struct QgemmParams {
  const uint16_t* a;        // bf16 bits [rows][k]
  const uint8_t* codes;     // [n_out][k * bits / 8]
  const uint16_t* scales;   // fp16 bits [n_out][k / group]
  const uint16_t* zeros;    // fp16 bits [n_out][k / group], asymmetric only
  void* y;                  // [rows][n_out], fp32 or bf16
  int64_t rows;
  int32_t n_out, k, group, bits;
  bool asym, y_bf16;
};

// Tile sizes the launch requires: n_out % QG_BN == 0, k % QG_BK == 0,
// group % QG_BK == 0.
constexpr int QG_BM = 256, QG_BN = 128, QG_BK = 64;
// At most this many rows take the few-row kernel (a workgroup per 16 weight
// rows, codes decoded in registers, 16 activation rows per workgroup row)
// instead of the 256 x 128 MFMA tiles.
constexpr int QG_GEMV_ROWS = 64;

hipError_t launch_qgemm(const QgemmParams& p, hipStream_t s);

}  // namespace bfly
