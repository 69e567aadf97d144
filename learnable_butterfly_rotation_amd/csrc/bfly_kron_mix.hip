// The mixing step of wide Kronecker composites, v = (O kron I) x: for every
// row and every column b of the nb-long segments,
//   v[a*nb + b] = sum_a' O[a][a'] x[a'*nb + b]       (fp32 out).
// Since (O kron B) = (I kron B)(O kron I), the caller then runs the plain
// butterfly (and its fused quantizer) on the rows * m segments of v.
//
// One thread per pair of adjacent columns of one row: it loads the pair from
// all m segments (coalesced across the wave), then forms the outputs eight
// segments at a time from O^T in LDS (16-byte broadcast reads).  m is padded
// to MB, a multiple of 8 (the padding reads zeros and stores nothing).
#include "bfly_common.h"

namespace bfly {

struct KronMixParams {
  const void* x;   // [rows][m * nb], fp32 or bf16
  float* v;        // [rows][m * nb]
  const float* mix;  // O, [m][m]
  int64_t rows;
  int32_t m, nb;
};

namespace {

template <int MB, bool XBF16>
__global__ __launch_bounds__(256) void kron_mix_kernel(const KronMixParams P) {
  __shared__ __align__(16) float omt[MB * MB];  // O^T, zero-padded
  const int m = P.m, nb = P.nb, half = nb >> 1;
  for (int i = threadIdx.x; i < MB * MB; i += 256) {
    const int a2 = i / MB, a = i - a2 * MB;
    omt[i] = (a < m && a2 < m) ? P.mix[a * m + a2] : 0.f;
  }
  __syncthreads();
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  // half >= 128: the 64 lanes of a wave share one row
  const int64_t row0 = gid / half;
  const int64_t row = ((int64_t)__builtin_amdgcn_readfirstlane((int)(row0 >> 32)) << 32) |
                      (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)row0);
  if (row >= P.rows) return;
  const int cp = (int)(gid - row * half);
  const int n = m * nb;
  constexpr int ESZ = XBF16 ? 2 : 4;
  const auto rx = buffer_range(static_cast<const char*>(P.x) + row * n * ESZ, (int64_t)n * ESZ);
  const auto rv = buffer_range(P.v + row * n, (int64_t)n * 4);

  float xv[MB][2];
#pragma unroll
  for (int a2 = 0; a2 < MB; ++a2) {
    const uint32_t e = (uint32_t)(a2 * nb + 2 * cp);  // past the row for a2 >= m: reads 0
    if (XBF16) {
      const uint32_t w = buf_ld4(rx, e * 2);
      xv[a2][0] = bf16_lo(w);
      xv[a2][1] = bf16_hi(w);
    } else {
      const uint32_t lo = buf_ld4(rx, e * 4), hi = buf_ld4(rx, e * 4 + 4);
      xv[a2][0] = __uint_as_float(lo);
      xv[a2][1] = __uint_as_float(hi);
    }
  }
#pragma unroll
  for (int ab = 0; ab < MB / 8; ++ab) {
    float acc[8][2];
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j][0] = acc[j][1] = 0.f;
#pragma unroll
    for (int a2 = 0; a2 < MB; ++a2) {
      const float4 o0 = *reinterpret_cast<const float4*>(&omt[a2 * MB + ab * 8]);
      const float4 o1 = *reinterpret_cast<const float4*>(&omt[a2 * MB + ab * 8 + 4]);
      const float o[8] = {o0.x, o0.y, o0.z, o0.w, o1.x, o1.y, o1.z, o1.w};
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        acc[j][0] = fmaf(o[j], xv[a2][0], acc[j][0]);
        acc[j][1] = fmaf(o[j], xv[a2][1], acc[j][1]);
      }
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {  // segments past m fall outside the row's range
      const uint32_t e = (uint32_t)((ab * 8 + j) * nb + 2 * cp);
      buf_st4(rv, e * 4, __float_as_uint(acc[j][0]));
      buf_st4(rv, e * 4 + 4, __float_as_uint(acc[j][1]));
    }
  }
}

template <int MB>
hipError_t launch_mb(const KronMixParams& p, bool xbf16, hipStream_t s) {
  const int64_t threads = p.rows * (p.nb / 2);
  const int64_t blocks = (threads + 255) / 256;
  if (xbf16)
    hipLaunchKernelGGL((kron_mix_kernel<MB, true>), dim3((unsigned)blocks), dim3(256), 0, s, p);
  else
    hipLaunchKernelGGL((kron_mix_kernel<MB, false>), dim3((unsigned)blocks), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace

// m in [2, 64], nb a power of two in [256, 4096], m * nb <= 65536.
hipError_t launch_kron_mix(const void* x, bool xbf16, float* v, const float* mix, int64_t rows,
                           int m, int nb, hipStream_t s) {
  KronMixParams p{x, v, mix, rows, m, nb};
  switch ((m + 7) / 8) {
    case 1: return launch_mb<8>(p, xbf16, s);
    case 2: return launch_mb<16>(p, xbf16, s);
    case 3: return launch_mb<24>(p, xbf16, s);
    case 4: return launch_mb<32>(p, xbf16, s);
    case 5: return launch_mb<40>(p, xbf16, s);
    case 6: return launch_mb<48>(p, xbf16, s);
    case 7: return launch_mb<56>(p, xbf16, s);
    case 8: return launch_mb<64>(p, xbf16, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace bfly
