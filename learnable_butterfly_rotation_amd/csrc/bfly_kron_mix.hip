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

// bf16 input: the same product on the matrix cores.  Per row, V (m x nb) =
// O (m x m) X (m x nb) is a small dense product; v_mfma_f32_32x32x16_bf16
// tiles it with O as the A operand (rows and k padded with zeros to MT x 32
// and KS x 16) and X as the B operand.  O is split into three bf16 parts,
// o = o1 + o2 + o3 (each the rounded remainder of the previous ones; for
// normal fp32 entries the sum is exact), so every product of a part with a
// bf16 input is exact and the sums are fp32, as in the kernel above; the
// small parts are added first.
//
// One wave per (row, block of 64 columns).  Lane l loads, for its 8 values
// of k (j = 16 ks + 8 (l / 32) + t), the bf16 pair at columns 2 (l % 32) and
// 2 (l % 32) + 1: lanes 0..31 read 128 contiguous bytes per segment.  The low
// halves form the B operand of the even columns, the high halves that of the
// odd columns (two v_perm_b32 per pair of k), so the two output tiles hold
// columns 2c and 2c + 1 of the same lane and each output row is stored as
// 8-byte pairs, 256 contiguous bytes per half-wave.  Segments past m read
// zeros and rows past m are not stored (both outside the row's range).  The
// grid is persistent; each wave keeps O's parts in registers and has PD
// items' loads in flight.
typedef __bf16 mix_bf16x8_t __attribute__((ext_vector_type(8)));
typedef float mix_f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t mix_u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t mix_u32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ mix_bf16x8_t mix_frag(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  const mix_u32x4_t v = {a, b, c, d};
  return __builtin_bit_cast(mix_bf16x8_t, v);
}

template <int MT, int KS>
__global__ __launch_bounds__(256) void kron_mix_mfma_kernel(const KronMixParams P) {
  constexpr int PD = KS <= 3 ? 2 : 1;  // items in flight per wave (registers)
  const int lane = threadIdx.x & 63, col = lane & 31, kh = lane >> 5;
  const int m = P.m, nb = P.nb;
  const uint32_t n = (uint32_t)(m * nb);
  const int lgblk = __builtin_ctz((unsigned)nb) - 6;  // 64-column blocks per row: 2^lgblk
  const int64_t nitems = P.rows << lgblk;
  const int64_t stride = (int64_t)gridDim.x * 4;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  int64_t item = (int64_t)blockIdx.x * 4 + wave;

  // A operand: the three parts of O, zero outside m x m
  mix_bf16x8_t a[3][MT][KS];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      uint32_t w[3][4];
      const int i = 32 * mt + col;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int j = 16 * ks + 8 * kh + 2 * u;
        const float o0 = (i < m && j < m) ? P.mix[i * m + j] : 0.f;
        const float o1 = (i < m && j + 1 < m) ? P.mix[i * m + j + 1] : 0.f;
        const uint32_t p1 = pack_bf16(o0, o1);
        const float r0 = o0 - bf16_lo(p1), r1 = o1 - bf16_hi(p1);  // exact
        const uint32_t p2 = pack_bf16(r0, r1);
        const uint32_t p3 = pack_bf16(r0 - bf16_lo(p2), r1 - bf16_hi(p2));
        w[0][u] = p1;
        w[1][u] = p2;
        w[2][u] = p3;
      }
#pragma unroll
      for (int q = 0; q < 3; ++q) a[q][mt][ks] = mix_frag(w[q][0], w[q][1], w[q][2], w[q][3]);
    }

  const char* xb = static_cast<const char*>(P.x);
  auto load = [&](int64_t it, uint32_t (&d)[KS][8]) {
    const int64_t row = it >> lgblk;
    const uint32_t c0 = (uint32_t)(it & ((1 << lgblk) - 1)) * 64u + 2u * col;
    const auto rx = buffer_range32(xb + row * n * 2, it < nitems ? n * 2u : 0u);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int t = 0; t < 8; ++t)
        d[ks][t] = buf_ld4(rx, ((uint32_t)(16 * ks + 8 * kh + t) * (uint32_t)nb + c0) * 2u);
  };

  uint32_t d[PD][KS][8];
#pragma unroll
  for (int s = 0; s < PD; ++s) load(item + s * stride, d[s]);
  for (; item < nitems; item += PD * stride) {
#pragma unroll
    for (int s = 0; s < PD; ++s) {
      const int64_t it = item + s * stride;
      mix_bf16x8_t b[KS][2];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        uint32_t lo[4], hi[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          lo[u] = __builtin_amdgcn_perm(d[s][ks][2 * u + 1], d[s][ks][2 * u], 0x05040100u);
          hi[u] = __builtin_amdgcn_perm(d[s][ks][2 * u + 1], d[s][ks][2 * u], 0x07060302u);
        }
        b[ks][0] = mix_frag(lo[0], lo[1], lo[2], lo[3]);
        b[ks][1] = mix_frag(hi[0], hi[1], hi[2], hi[3]);
      }
      // the refill of slot s goes out once its values are repacked
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int h = 0; h < 2; ++h) asm volatile("" : "+v"(b[ks][h])::"memory");
      load(it + PD * stride, d[s]);
      mix_f32x16_t acc[MT][2];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[mt][h][r] = 0.f;
#pragma unroll
      for (int q = 2; q >= 0; --q)
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
          for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int h = 0; h < 2; ++h)
              acc[mt][h] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[q][mt][ks], b[ks][h],
                                                                  acc[mt][h], 0, 0, 0);
      const int64_t row = it >> lgblk;
      const uint32_t c0 = (uint32_t)(it & ((1 << lgblk) - 1)) * 64u + 2u * col;
      const auto rv = buffer_range32(P.v + row * n, it < nitems ? n * 4u : 0u);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const uint32_t i = (uint32_t)(32 * mt + 8 * (r >> 2) + 4 * kh + (r & 3));
          const mix_u32x2_t pr = {__float_as_uint(acc[mt][0][r]), __float_as_uint(acc[mt][1][r])};
          __builtin_amdgcn_raw_buffer_store_b64(pr, rv, (int)((i * (uint32_t)nb + c0) * 4u), 0, 0);
        }
    }
  }
}

template <int MT, int KS>
hipError_t launch_mfma(const KronMixParams& p, hipStream_t s) {
  auto kern = kron_mix_mfma_kernel<MT, KS>;
  int cus = 0, per_cu = 0;  // resident workgroups on the device
  const hipError_t e = kernel_setup(reinterpret_cast<const void*>(kern), 256, 0, &per_cu, &cus);
  if (e != hipSuccess) return e;
  const int cap = per_cu * cus;
  const int64_t items = p.rows * (p.nb / 64);
  const int64_t want = (items + 3) / 4;
  const int blocks = (int)(want < cap ? want : cap);
  hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(256), 0, s, p);
  return hipGetLastError();
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
  if (rows == 0) return hipSuccess;
  if (xbf16) {
    if (m <= 16) return launch_mfma<1, 1>(p, s);
    if (m <= 32) return launch_mfma<1, 2>(p, s);
    if (m <= 48) return launch_mfma<2, 3>(p, s);
    return launch_mfma<2, 4>(p, s);
  }
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
