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
//      m segments of V in turn: each thread holds 8 consecutive elements,
//      the 8 Givens stages run in the forward kernel's scaled two-FMA form
//      (stages 0..2 in registers, 3..6 as DPP multiply-adds on mapped lane
//      bits, stage 7 across half-waves through ds_swizzle), with plain
//      rotations as the fallback the table can ask for; then the bf16 (or
//      fp32) output and the group quantizer of the fused forward kernel,
//      stored straight to HBM.
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

// Lane layout of a butterfly team (32 lanes, half a wave): lane t holds the
// 8 consecutive elements i(e) = e + 8 c + 128 h, e = 0..7, with c =
// dpp_unmix(t & 15) and h = t >> 4.  Element bits 3..6 sit on the lane bits
// through the map lane = XOR of (1, 2, 7, 15) over the set bits of c, so a
// stage on element bit 3 + j pairs lane t with t ^ (1, 2, 7, 15)[j]: quad
// permutes, half-row mirror and row mirror, all DPP operands of one
// multiply-add (the forward kernel's phase A).  Element bit 7 pairs lane t
// with t ^ 16 (ds_swizzle).  Groups of 2^k consecutive elements stay on
// aligned runs of consecutive lanes, so the quantizer's reductions hold.
__device__ __forceinline__ int kf_elem0(int t) { return 8 * dpp_unmix(t & 15) + 128 * (t >> 4); }

__device__ __forceinline__ float kf_swap16(float v) {  // the value of lane t ^ 16
  return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), (16 << 10) | 0x1F));
}

// The partner value on element bit 3 + J (plain form).
template <int J>
__device__ __forceinline__ float kf_partner(float v) {
  if constexpr (J == 0) return dpp<DPP_XOR1>(v);
  else if constexpr (J == 1) return dpp<DPP_XOR2>(v);
  else if constexpr (J == 2) return dpp<DPP_HALF_MIRROR>(v);
  else if constexpr (J == 3) return dpp<DPP_MIRROR>(v);
  else return kf_swap16(v);
}

// Coefficients of one team thread.
//   scaled ("fast Givens") form, read from the table's forward layout by
//   element: stages 0..2 (beta, gamma) per register pair, stages 3..6 one
//   per element (its own coefficient: the DPP multiply-add adds it times the
//   partner's old value), stage 7 (own, cross) per element from the last
//   stage's 2x2 matrix (c s_i, -s s_j, s s_i, c s_j);
//   plain form (the fallback when the table marks the scaled form unusable):
//   (cos, sin) of each pair, read from the table's cs at every use (a rare
//   path; in registers the two forms' sets would not fit beside each other).
struct KfFast {
  float b[3][4], g[3][4], k[4][8], own[8], cross[8];
};
struct KfPlain {
  const float2* cs;
  int base;  // this thread's first element
};

__device__ __forceinline__ bool kf_load_fast(KfFast& C, const float* fgt, int t) {
  const int base = kf_elem0(t);
  bool nan_seen = false;
  auto fin = [&](float v) {
    nan_seen |= (__float_as_uint(v) & 0x7fffffffu) > 0x7f800000u;  // bit test (no NaN arithmetic)
    return v;
  };
#pragma unroll
  for (int s = 0; s < 3; ++s)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int lo = base + pair_lo(j, s);
      C.b[s][j] = fin(fgt[fwd_coef_index(s, lo, KF_L)]);
      C.g[s][j] = fin(fgt[fwd_coef_index(s, lo | (1 << s), KF_L)]);
    }
#pragma unroll
  for (int s = 3; s < KF_L - 1; ++s)
#pragma unroll
    for (int e = 0; e < 8; ++e) C.k[s - 3][e] = fin(fgt[fwd_coef_index(s, base + e, KF_L)]);
  const bool upper = (t >> 4) & 1;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float4 q = *reinterpret_cast<const float4*>(fgt + fwd_last_index((base + e) & ~128, KF_L));
    C.own[e] = upper ? q.w : q.x;
    C.cross[e] = upper ? q.z : q.y;
  }
  return nan_seen;
}


// The 8 stages of one segment (w: this thread's 8 values, true values out).
__device__ __forceinline__ void kf_segment(float (&w)[8], const KfFast& C) {
#pragma unroll
  for (int s = 0; s < 3; ++s)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int lo = pair_lo(j, s), hi = lo | (1 << s);
      rotate<true>(w[lo], w[hi], C.b[s][j], C.g[s][j]);
    }
#pragma unroll
  for (int j = 0; j < 4; ++j) BFLY_DPP_SWITCH(j, BFLY_LANE_FMA8_IP, w, C.k[j])
  float p[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) p[e] = kf_swap16(w[e]);
#pragma unroll
  for (int e = 0; e < 8; ++e) w[e] = fmaf(C.cross[e], p[e], C.own[e] * w[e]);
}

// Lane stage 3 + J in the plain form: lower element c w - s partner, upper
// c w + s partner.
template <int J>
__device__ __forceinline__ void kf_plain_lane(float (&w)[8], const KfPlain& C) {
  constexpr int s = 3 + J;
  float p[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) p[e] = kf_partner<J>(w[e]);
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int i = C.base + e;
    const float2 q = C.cs[s * (KF_NB / 2) + pair_rank(i & ~(1 << s), s)];
    w[e] = fmaf(((i >> s) & 1) ? q.y : -q.y, p[e], q.x * w[e]);
  }
}

__device__ __forceinline__ void kf_segment(float (&w)[8], const KfPlain& C) {
#pragma unroll
  for (int s = 0; s < 3; ++s)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int lo = pair_lo(j, s), hi = lo | (1 << s);
      const float2 q = C.cs[s * (KF_NB / 2) + pair_rank(C.base + lo, s)];
      const float u = w[lo], v = w[hi];
      w[lo] = fmaf(q.x, u, -(q.y * v));
      w[hi] = fmaf(q.y, u, q.x * v);
    }
  kf_plain_lane<0>(w, C);
  kf_plain_lane<1>(w, C);
  kf_plain_lane<2>(w, C);
  kf_plain_lane<3>(w, C);
  kf_plain_lane<4>(w, C);
}

// The row loop over rows blockIdx.x, + gridDim.x, ... below nrun: one
// barrier per row, then the next row's mix (matrix cores, into the other LDS
// buffer) alongside this row's segments (vector units).  QM fixes the two common quantizer formats
// at compile time (no group-size branches).
template <int KS, int YK, int QM, class Coef>
__device__ __forceinline__ void kf_rows(const KronFusedParams& P, float* vbuf, const uint16_t* opart,
                                        const Coef& C, int64_t nrun) {
  const int tid = threadIdx.x, lane = tid & 63, col = lane & 31, kh = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int mt = wave >> 2, blk = wave & 3;  // mix tile: V rows 32 mt.., columns 64 blk..
  const int team = tid >> 5, t = tid & 31;   // butterfly team and thread
  const int m = P.m;
  const uint32_t n = (uint32_t)(m * KF_NB);
  const int e0 = kf_elem0(t);                // this thread's first element of a segment

  constexpr bool QUANT = QM != Q_NONE;
  constexpr bool FIXED = QM == Q_S4G128 || QM == Q_A2G128;
  const int bits = QM == Q_S4G128 ? 4 : (QM == Q_A2G128 ? 2 : P.bits);
  const bool asym = QM == Q_A2G128 || (QM == Q_ANY && P.asym != 0);
  const int group = FIXED ? 128 : (QUANT ? P.group : 8);
  const int gt = group / 8;
  const float top = asym ? (float)((1 << bits) - 1) : (float)((1 << (bits - 1)) - 1);
  const float inv_top = 1.0f / top;
  const uint32_t ngr = QUANT ? n / (uint32_t)group : 0u;
  const bool scale_lane = QUANT && (t & (gt - 1)) == 0;

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

  // the mix of one row from the X words in d (on the matrix cores): the
  // MFMAs are issued here, their results written to V by mix_store
  kf_f32x16_t acc[2];
  // this wave's A operands (O's parts at rows 32 mt + col), the same for
  // every row: held in registers up to KS = 3 (m <= 48; four k steps would
  // spill), read from LDS at each use above that
  constexpr bool AREG = KS <= 3;
  kf_bf16x8_t aop[3][AREG ? KS : 1];
  auto a_frag = [&](int q, int ks) {
    const uint4 av = *reinterpret_cast<const uint4*>(opart + q * KF_OPART + (32 * mt + col) * KF_OS +
                                                     16 * ks + 8 * kh);
    return kf_frag(av.x, av.y, av.z, av.w);
  };
  if constexpr (AREG) {
#pragma unroll
    for (int q = 0; q < 3; ++q)
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) aop[q][ks] = a_frag(q, ks);
  }
  auto mix_issue = [&](const uint32_t (&dd)[KS][8]) {
    kf_bf16x8_t b[KS][2];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      uint32_t lo[4], hi[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        lo[u] = __builtin_amdgcn_perm(dd[ks][2 * u + 1], dd[ks][2 * u], 0x05040100u);
        hi[u] = __builtin_amdgcn_perm(dd[ks][2 * u + 1], dd[ks][2 * u], 0x07060302u);
      }
      b[ks][0] = kf_frag(lo[0], lo[1], lo[2], lo[3]);
      b[ks][1] = kf_frag(hi[0], hi[1], hi[2], hi[3]);
    }
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[h][e] = 0.f;
#pragma unroll
    for (int q = 2; q >= 0; --q)  // the small parts first
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        // A operand: O part q, row 32 mt + col, k = 16 ks + 8 kh .. + 7
        const kf_bf16x8_t aq = AREG ? aop[q][AREG ? ks : 0] : a_frag(q, ks);
#pragma unroll
        for (int h = 0; h < 2; ++h)
          acc[h] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aq, b[ks][h], acc[h], 0, 0, 0);
      }
  };
  // V rows 32 mt + 8 (e / 4) + 4 kh + e % 4, columns 64 blk + 2 col + h
  auto mix_store = [&](float* Vw) {
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int i = 32 * mt + 8 * (e >> 2) + 4 * kh + (e & 3);
      *reinterpret_cast<float2*>(Vw + i * KF_VS + 64 * blk + 2 * col) = make_float2(acc[0][e], acc[1][e]);
    }
  };

  // Software pipeline over rows: the mix of the next row runs on the matrix
  // cores while this row's butterfly runs on the vector units.  Row r's V
  // sits in buffer buf; the next row's goes to the other one, last read by
  // the row before r (finished by every wave at this iteration's barrier).
  uint32_t d[KS][8];
  int64_t r = blockIdx.x;
  load(r, d);
  int buf = 0;
  if (r < nrun) {
    mix_issue(d);
    load(r + gridDim.x, d);
    mix_store(vbuf);
  }
  for (; r < nrun; r += gridDim.x, buf ^= 1) {
    float* const V = vbuf + buf * KF_VBUF;
    __syncthreads();  // V of row r is complete; the other buffer is free
    const bool next = r + gridDim.x < nrun;
    if (next) {
      mix_issue(d);
      load(r + 2 * gridDim.x, d);
    }

    // 2. the butterfly on each segment, then the outputs
    const auto ry = buffer_range32(static_cast<uint16_t*>(P.y) + (YK == Y_BF16 ? r * (int64_t)n : 0),
                                   YK == Y_BF16 ? n * 2u : 0u);
    const auto ry4 = buffer_range32(static_cast<float*>(P.y) + (YK == Y_F32 ? r * (int64_t)n : 0),
                                    YK == Y_F32 ? n * 4u : 0u);
    const auto rcod = buffer_range32(P.codes + (QUANT ? r * (int64_t)(n * (uint32_t)bits / 8) : 0),
                                     QUANT ? n * (uint32_t)bits / 8 : 0u);
    const auto rs = buffer_range32(P.scales + (QUANT ? r * (int64_t)ngr : 0), ngr * 2u);
    const auto rz = buffer_range32(P.zeros + (QUANT && asym ? r * (int64_t)ngr : 0), asym ? ngr * 2u : 0u);
    for (int sa = team; sa < m; sa += KF_TEAMS) {
      float w[8];
      {
        const float4 q0 = *reinterpret_cast<const float4*>(V + sa * KF_VS + e0);
        const float4 q1 = *reinterpret_cast<const float4*>(V + sa * KF_VS + e0 + 4);
        w[0] = q0.x; w[1] = q0.y; w[2] = q0.z; w[3] = q0.w;
        w[4] = q1.x; w[5] = q1.y; w[6] = q1.z; w[7] = q1.w;
      }
      kf_segment(w, C);
      const uint32_t el = (uint32_t)(sa * KF_NB + e0);  // element of the row
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
      if (QUANT) {  // every lane of an active team quantizes
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
    if (next) mix_store(vbuf + (buf ^ 1) * KF_VBUF);
  }
}

template <int KS, int YK, int QM>
__global__ __launch_bounds__(KF_THREADS) void kron_fused_kernel(const KronFusedParams P) {
  extern __shared__ float4 kf_lds_raw[];
  float* const vbuf = reinterpret_cast<float*>(kf_lds_raw);
  const int tid = threadIdx.x, t = tid & 31;
  const int m = P.m;
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
  // The scaled form unless the table marks it unusable (a NaN anywhere:
  // every team covers every pair, so all workgroups decide alike).
  KfFast F;
  const bool nan_seen = kf_load_fast(F, P.fgt, t);
  constexpr int NW = KF_THREADS / 64;
  __shared__ int nan_wave[NW];
  if ((tid & 63) == 0) nan_wave[tid >> 6] = __builtin_amdgcn_ballot_w64(nan_seen) != 0;
  __syncthreads();
  int seen = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) seen |= nan_wave[w];
  const bool usable = __builtin_amdgcn_readfirstlane(seen) == 0;
  // The two forms run as consecutive loops (one of them empty), not as the
  // two arms of a branch: the register allocator then never holds both
  // loops' state at once.
  kf_rows<KS, YK, QM>(P, vbuf, opart, F, usable ? P.rows : 0);
  KfPlain C;
  C.cs = P.cs;
  C.base = kf_elem0(t);
  kf_rows<KS, YK, (QM == Q_NONE ? Q_NONE : Q_ANY)>(P, vbuf, opart, C, usable ? 0 : P.rows);
}

template <int KS, int YK, int QM>
hipError_t launch_kf(const KronFusedParams& p, hipStream_t s) {
  auto kern = kron_fused_kernel<KS, YK, QM>;
  int per_cu = 0, num_cu = 0;
  const hipError_t e = kernel_setup(reinterpret_cast<const void*>(kern), KF_THREADS, KF_LDS,
                                    &per_cu, &num_cu);
  if (e != hipSuccess) return e;
  const int64_t cap = (int64_t)per_cu * num_cu;
  const int grid = (int)(p.rows < cap ? p.rows : cap);
  hipLaunchKernelGGL(kern, dim3(grid), dim3(KF_THREADS), KF_LDS, s, p);
  return hipGetLastError();
}

template <int KS, int YK>
hipError_t launch_kf_q(const KronFusedParams& p, hipStream_t s) {
  if (p.codes == nullptr) return launch_kf<KS, YK, Q_NONE>(p, s);
  if (p.group == 128 && p.bits == 4 && !p.asym) return launch_kf<KS, YK, Q_S4G128>(p, s);
  if (p.group == 128 && p.bits == 2 && p.asym) return launch_kf<KS, YK, Q_A2G128>(p, s);
  return launch_kf<KS, YK, Q_ANY>(p, s);
}

template <int KS>
hipError_t launch_kf_ks(const KronFusedParams& p, hipStream_t s) {
  if (p.y == nullptr) return launch_kf_q<KS, Y_NONE>(p, s);
  return p.y_bf16 ? launch_kf_q<KS, Y_BF16>(p, s) : launch_kf_q<KS, Y_F32>(p, s);
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
