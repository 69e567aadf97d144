// Wide Kronecker composites y = (O kron B(theta_b)) x in ONE pass, for
// segments of nb = 256 and bf16 rows (the 11008 = 43 x 256 width of the
// LLaMA-2-7B MLP; duidaima.com write-up of ButterflyQuant, section
// "butterfly": Kronecker composites for widths that are not powers of two).
// The two-pass path (the mix into an fp32 workspace, then the butterfly)
// moves each row's bytes three times over; here one workgroup takes one row
// at a time:
//   1. the mix V (m x 256) = O (m x m) X (m x 256) on the matrix cores
//      (v_mfma_f32_32x32x16_bf16), O split into three bf16 parts so that
//      every product with a bf16 input is exact and the sums are fp32 (the
//      arithmetic of the two-pass mix); wave w computes the rows 32 (w / 4)
//      .. of V at the 64 columns 64 (w % 4) .., loading its X columns itself
//      (one row ahead) and writing its V tile into LDS;
//   2. after one barrier, 16 teams of 32 threads (half a wave each) take the
//      m segments of V in turn: thread t holds elements 8t .. 8t + 7, the
//      8 Givens stages run as plain rotations, stages 0..2 inside the
//      thread's registers and stages 3..7 with the partner lane's values
//      (DPP for lane masks 1 and 2, ds_swizzle for 4, 8 and 16); then the
//      bf16 (or fp32) output and the group quantizer of the fused forward
//      kernel, stored straight to HBM.
// V is double-buffered in LDS (2 x 64 x 260 floats), so one barrier per row
// separates the mix of row r + 1 from the reads of row r's segments.  O's
// three parts sit in LDS too (each wave reads its A operands per row): in
// registers they would push the kernel past 256 VGPRs beside the butterfly's
// coefficients.
#include "bfly_fwd_kernel.h"

namespace bfly {
namespace {

constexpr int KF_NB = 256;                  // segment length (8 stages)
constexpr int KF_L = 8;
constexpr int KF_THREADS = 512;             // 8 waves: 2 x 4 mix tiles, 16 butterfly teams
constexpr int KF_TEAMS = KF_THREADS / 32;
constexpr int KF_VS = KF_NB + 4;            // LDS words per V row (bank offset between rows)
constexpr int KF_VBUF = 64 * KF_VS;         // one V buffer: up to 64 segments
constexpr int KF_OS = 64 + 8;              // bf16 per row of an O part (16-byte reads spread over banks)
constexpr int KF_OPART = 64 * KF_OS;        // one part: up to 64 x 64
constexpr size_t KF_LDS = 2 * KF_VBUF * sizeof(float) + 3 * KF_OPART * sizeof(uint16_t);

typedef __bf16 kf_bf16x8_t __attribute__((ext_vector_type(8)));
typedef float kf_f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t kf_u32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ kf_bf16x8_t kf_frag(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  const kf_u32x4_t v = {a, b, c, d};
  return __builtin_bit_cast(kf_bf16x8_t, v);
}

// The partner's value at lane distance 2^k (k = 0..4) within 32 lanes.
template <int K>
__device__ __forceinline__ float kf_partner(float v) {
  if constexpr (K == 0) return dpp<DPP_XOR1>(v);
  else if constexpr (K == 1) return dpp<DPP_XOR2>(v);
  else  // bit mode: and 0x1F, xor (1 << K) within each group of 32 lanes
    return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), ((1 << K) << 10) | 0x1F));
}

template <int K>
__device__ __forceinline__ void kf_lane_stage(float (&w)[8], const float2 (&k)[8]) {
  float p[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) p[e] = kf_partner<K>(w[e]);
  // lower element: c w - s partner; upper: c w + s partner (k.y holds -s or +s)
#pragma unroll
  for (int e = 0; e < 8; ++e) w[e] = fmaf(k[e].y, p[e], k[e].x * w[e]);
}

template <int KS, int YK>
__global__ __launch_bounds__(KF_THREADS) void kron_fused_kernel(const KronFusedParams P) {
  extern __shared__ float4 kf_lds_raw[];
  float* const vbuf = reinterpret_cast<float*>(kf_lds_raw);
  const int tid = threadIdx.x, lane = tid & 63, col = lane & 31, kh = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int mt = wave >> 2, blk = wave & 3;  // mix tile: V rows 32 mt.., columns 64 blk..
  const int team = tid >> 5, t = tid & 31;   // butterfly team and thread
  const int m = P.m;
  const uint32_t n = (uint32_t)(m * KF_NB);

  // O's three bf16 parts into LDS, zero outside m x m: o = o1 + o2 + o3,
  // each the rounded remainder of the ones before (exact for normal fp32)
  uint16_t* const opart = reinterpret_cast<uint16_t*>(vbuf + 2 * KF_VBUF);
  for (int k = tid; k < 64 * 32; k += KF_THREADS) {  // pairs of entries (i, j), (i, j + 1)
    const int i = k >> 5, j = 2 * (k & 31);
    const float o0 = (i < m && j < m) ? P.mix[i * m + j] : 0.f;
    const float o1 = (i < m && j + 1 < m) ? P.mix[i * m + j + 1] : 0.f;
    const uint32_t p1 = pack_bf16(o0, o1);
    const float r0 = o0 - bf16_lo(p1), r1 = o1 - bf16_hi(p1);
    const uint32_t p2 = pack_bf16(r0, r1);
    const uint32_t p3 = pack_bf16(r0 - bf16_lo(p2), r1 - bf16_hi(p2));
    *reinterpret_cast<uint32_t*>(opart + 0 * KF_OPART + i * KF_OS + j) = p1;
    *reinterpret_cast<uint32_t*>(opart + 1 * KF_OPART + i * KF_OS + j) = p2;
    *reinterpret_cast<uint32_t*>(opart + 2 * KF_OPART + i * KF_OS + j) = p3;
  }
  __syncthreads();

  // Butterfly coefficients (cos, sin) of the pairs this thread rotates:
  // stages 0..2 by register pair, stages 3..7 by element with the sign of
  // sin folded in (the element is the pair's lower or upper one).
  float2 rc[3][4], lc[KF_L - 3][8];
#pragma unroll
  for (int s = 0; s < 3; ++s)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      rc[s][j] = P.cs[s * (KF_NB / 2) + pair_rank(8 * t + pair_lo(j, s), s)];
#pragma unroll
  for (int s = 3; s < KF_L; ++s)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int i = 8 * t + e;
      const float2 q = P.cs[s * (KF_NB / 2) + pair_rank(i & ~(1 << s), s)];
      lc[s - 3][e] = make_float2(q.x, ((i >> s) & 1) ? q.y : -q.y);
    }

  // the quantizer's fixed parameters
  const bool quant = P.codes != nullptr;
  const int bits = P.bits, group = quant ? P.group : 8;
  const bool asym = P.asym != 0;
  const int gt = group / 8;
  const float top = asym ? (float)((1 << bits) - 1) : (float)((1 << (bits - 1)) - 1);
  const float inv_top = 1.0f / top;
  const uint32_t ngr = quant ? n / (uint32_t)group : 0u;
  const bool scale_lane = quant && (t & (gt - 1)) == 0;

  // X columns of this wave's block for row r: lane l holds, for its 8 values
  // of k (segment 16 ks + 8 kh + u), the bf16 pair at columns
  // 64 blk + 2 col, + 1 (segments past m fall outside the row's range)
  const char* xb = static_cast<const char*>(P.x);
  auto load = [&](int64_t r, uint32_t (&d)[KS][8]) {
    const auto rx = buffer_range32(xb + r * (int64_t)n * 2, r < P.rows ? n * 2u : 0u);
    const uint32_t c0 = (uint32_t)(64 * blk + 2 * col);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int u = 0; u < 8; ++u)
        d[ks][u] = buf_ld4(rx, ((uint32_t)(16 * ks + 8 * kh + u) * KF_NB + c0) * 2u);
  };

  uint32_t d[KS][8];
  int64_t r = blockIdx.x;
  load(r, d);
  int buf = 0;
  for (; r < P.rows; r += gridDim.x, buf ^= 1) {
    float* const V = vbuf + buf * KF_VBUF;
    // 1. the mix on the matrix cores (the next row's loads go out once the
    // operands are repacked)
    kf_bf16x8_t b[KS][2];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      uint32_t lo[4], hi[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        lo[u] = __builtin_amdgcn_perm(d[ks][2 * u + 1], d[ks][2 * u], 0x05040100u);
        hi[u] = __builtin_amdgcn_perm(d[ks][2 * u + 1], d[ks][2 * u], 0x07060302u);
      }
      b[ks][0] = kf_frag(lo[0], lo[1], lo[2], lo[3]);
      b[ks][1] = kf_frag(hi[0], hi[1], hi[2], hi[3]);
    }
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int h = 0; h < 2; ++h) asm volatile("" : "+v"(b[ks][h])::"memory");
    load(r + gridDim.x, d);
    kf_f32x16_t acc[2];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[h][e] = 0.f;
#pragma unroll
    for (int q = 2; q >= 0; --q)  // the small parts first
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        // A operand: O part q, row 32 mt + col, k = 16 ks + 8 kh .. + 7
        const uint4 av = *reinterpret_cast<const uint4*>(opart + q * KF_OPART + (32 * mt + col) * KF_OS +
                                                         16 * ks + 8 * kh);
        const kf_bf16x8_t a = kf_frag(av.x, av.y, av.z, av.w);
#pragma unroll
        for (int h = 0; h < 2; ++h)
          acc[h] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b[ks][h], acc[h], 0, 0, 0);
      }
    // V rows 32 mt + 8 (e / 4) + 4 kh + e % 4, columns 64 blk + 2 col + h
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int i = 32 * mt + 8 * (e >> 2) + 4 * kh + (e & 3);
      *reinterpret_cast<float2*>(V + i * KF_VS + 64 * blk + 2 * col) = make_float2(acc[0][e], acc[1][e]);
    }
    __syncthreads();

    // 2. the butterfly on each segment, then the outputs
    const auto ry = buffer_range32(static_cast<uint16_t*>(P.y) + (YK == Y_BF16 ? r * (int64_t)n : 0),
                                   YK == Y_BF16 ? n * 2u : 0u);
    const auto ry4 = buffer_range32(static_cast<float*>(P.y) + (YK == Y_F32 ? r * (int64_t)n : 0),
                                    YK == Y_F32 ? n * 4u : 0u);
    const auto rcod = buffer_range32(P.codes + (quant ? r * (int64_t)(n * (uint32_t)bits / 8) : 0),
                                   quant ? n * (uint32_t)bits / 8 : 0u);
    const auto rs = buffer_range32(P.scales + (quant ? r * (int64_t)ngr : 0), ngr * 2u);
    const auto rz = buffer_range32(P.zeros + (quant && asym ? r * (int64_t)ngr : 0), asym ? ngr * 2u : 0u);
    for (int sa = team; sa < m; sa += KF_TEAMS) {
      float w[8];
      {
        const float4 q0 = *reinterpret_cast<const float4*>(V + sa * KF_VS + 8 * t);
        const float4 q1 = *reinterpret_cast<const float4*>(V + sa * KF_VS + 8 * t + 4);
        w[0] = q0.x; w[1] = q0.y; w[2] = q0.z; w[3] = q0.w;
        w[4] = q1.x; w[5] = q1.y; w[6] = q1.z; w[7] = q1.w;
      }
#pragma unroll
      for (int s = 0; s < 3; ++s)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int lo = pair_lo(j, s), hi = lo | (1 << s);
          const float u = w[lo], v = w[hi];
          w[lo] = fmaf(rc[s][j].x, u, -(rc[s][j].y * v));
          w[hi] = fmaf(rc[s][j].y, u, rc[s][j].x * v);
        }
      kf_lane_stage<0>(w, lc[0]);
      kf_lane_stage<1>(w, lc[1]);
      kf_lane_stage<2>(w, lc[2]);
      kf_lane_stage<3>(w, lc[3]);
      kf_lane_stage<4>(w, lc[4]);
      const uint32_t el = (uint32_t)(sa * KF_NB + 8 * t);  // element of the row
      if (YK == Y_BF16) {
        buf_st16<kNonTemporal>(ry, el * 2,
                               make_uint4(pack_bf16(w[0], w[1]), pack_bf16(w[2], w[3]),
                                          pack_bf16(w[4], w[5]), pack_bf16(w[6], w[7])));
      } else if (YK == Y_F32) {
        buf_st16<kNonTemporal>(ry4, el * 4,
                               make_uint4(__float_as_uint(w[0]), __float_as_uint(w[1]),
                                          __float_as_uint(w[2]), __float_as_uint(w[3])));
        buf_st16<kNonTemporal>(ry4, el * 4 + 16,
                               make_uint4(__float_as_uint(w[4]), __float_as_uint(w[5]),
                                          __float_as_uint(w[6]), __float_as_uint(w[7])));
      }
      if (quant) {  // uniform: every lane of an active team quantizes
        const QParams qp = quant_params(w, gt, asym, inv_top, top);
        quant_clamp(w, qp);
        const uint32_t packed = quant_pack(w, qp, bits, asym);
        if (bits == 4) buf_st4<kNonTemporal>(rcod, el / 2, packed);
        else buf_st2<kNonTemporal>(rcod, el / 4, (uint16_t)packed);
        const uint32_t off = scale_lane ? 2 * (el / (uint32_t)group) : kOutOfRange;
        buf_st2<kNonTemporal>(rs, off, (uint16_t)(qp.sz & 0xFFFFu));
        if (asym) buf_st2<kNonTemporal>(rz, off, (uint16_t)(qp.sz >> 16));
      }
    }
  }
}

template <int KS, int YK>
hipError_t launch_kf(const KronFusedParams& p, hipStream_t s) {
  auto kern = kron_fused_kernel<KS, YK>;
  int per_cu = 0, num_cu = 0;
  const hipError_t e = kernel_setup(reinterpret_cast<const void*>(kern), KF_THREADS, KF_LDS,
                                    &per_cu, &num_cu);
  if (e != hipSuccess) return e;
  const int64_t cap = (int64_t)per_cu * num_cu;
  const int grid = (int)(p.rows < cap ? p.rows : cap);
  hipLaunchKernelGGL(kern, dim3(grid), dim3(KF_THREADS), KF_LDS, s, p);
  return hipGetLastError();
}

template <int KS>
hipError_t launch_kf_ks(const KronFusedParams& p, hipStream_t s) {
  if (p.y == nullptr) return launch_kf<KS, Y_NONE>(p, s);
  return p.y_bf16 ? launch_kf<KS, Y_BF16>(p, s) : launch_kf<KS, Y_F32>(p, s);
}

}  // namespace

bool kron_fused_supported(int m, int nb, bool xbf16) { return xbf16 && nb == KF_NB && m >= 2 && m <= 64; }

hipError_t launch_kron_fused(const KronFusedParams& p, hipStream_t s) {
  if (p.rows == 0) return hipSuccess;
  switch ((p.m + 15) / 16) {
    case 1: return launch_kf_ks<1>(p, s);
    case 2: return launch_kf_ks<2>(p, s);
    case 3: return launch_kf_ks<3>(p, s);
    default: return launch_kf_ks<4>(p, s);
  }
}

}  // namespace bfly
