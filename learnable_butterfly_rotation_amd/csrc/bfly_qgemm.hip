// Quantized-weight matrix product on the matrix cores: y = a w^T with w's
// rows stored as 2- or 4-bit group codes, the consumer of the rotated and
// quantized weights (ButterflyQuant abstract: W x = (W Q^T)(Q x) with 2-bit
// weights; the ButterflyQuant write-up, section "training and results":
// W2A16, bf16 activations against 2-bit weights).
//
// Exactness: a code minus its zero point is a small integer (|v| <= 15),
// exact in bf16, and a bf16 activation times it is exact in fp32.  So the
// MFMA sums sum_k a[r][k] * (q[o][k] - z) over one quantization group in
// fp32 with only the accumulation rounding, and the group's fp16 scale is
// applied afterwards: y += s[o][g] * P_g.  No weight value is rounded to
// bf16; the result is as accurate as an fp32 dot product.
//
// Workgroup: 512 threads (8 waves, 4 along rows x 2 along outputs), a
// 256 x 128 output tile, k in chunks of 64.  Per chunk the activations
// (256 x 64 bf16) and the decoded weights (128 x 64 bf16) go through LDS,
// double-buffered, one barrier per chunk; each wave runs 2 x 2
// v_mfma_f32_32x32x16_bf16 tiles (64 x 64 outputs).  Each weight code is
// decoded once per workgroup (by one thread) and then read by the four
// waves of its output columns.
#include <type_traits>

#include "bfly_common.h"
#include "bfly_qgemm.h"

namespace bfly {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr int QROW = QG_BK * 2 + 16;  // LDS bytes per tile row: 64 bf16 + 16 (banks)

// Tile shape for BM rows x QG_BN outputs: BM / 64 x 2 waves of 64 x 64.
template <int BM>
struct QTile {
  static constexpr int THREADS = 2 * BM;
  static constexpr int WMC = BM / 64;                  // waves along the rows
  static constexpr int A_BYTES = BM * QROW;
  static constexpr int B_BYTES = QG_BN * QROW;
  static constexpr int S_OFF = 2 * (A_BYTES + B_BYTES);  // the chunks' scales, fp16 [2][QG_BN]
  static constexpr int LDS = S_OFF + 2 * QG_BN * 2;
  static constexpr int TPR = THREADS / QG_BN;          // threads per weight row (decode)
  static constexpr int CPT = QG_BK / TPR;              // codes per thread per chunk
};

__device__ __forceinline__ uint4 lds_ld16(const uint8_t* p) {
  return *reinterpret_cast<const uint4*>(p);
}
__device__ __forceinline__ void lds_st16(uint8_t* p, uint4 v) { *reinterpret_cast<uint4*>(p) = v; }

__device__ __forceinline__ float half_to_float(uint16_t h) {
  return (float)__builtin_bit_cast(_Float16, h);
}

// Two small integers given as floats -> their bf16 patterns (the high
// halves, exact) in one word, lo in the low half.
__device__ __forceinline__ uint32_t pack_exact(float lo, float hi) {
  return __builtin_amdgcn_perm(__float_as_uint(hi), __float_as_uint(lo), 0x07060302u);
}

template <int B>
__device__ __forceinline__ float ubyte(uint32_t m) {
  return (float)((m >> (8 * B)) & 0xFFu);
}

// 16 codes of BITS bits (element e of the chunk in bits [BITS*e, ...) of
// the little-endian words x[]) minus z, as 8 words of bf16 pairs (elements
// 2i, 2i+1).  Symmetric codes arrive with their sign bit flipped (offset
// binary) and z = 2^(BITS-1).
template <int BITS>
__device__ __forceinline__ void decode16(const uint32_t (&x)[BITS / 2], float z, uint32_t (&w)[8]) {
  float f[16];
  if (BITS == 2) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t m = (x[0] >> (2 * j)) & 0x03030303u;  // elements j, j+4, j+8, j+12
      f[j] = ubyte<0>(m) - z;
      f[j + 4] = ubyte<1>(m) - z;
      f[j + 8] = ubyte<2>(m) - z;
      f[j + 12] = ubyte<3>(m) - z;
    }
  } else {
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const uint32_t m = (x[h] >> (4 * j)) & 0x0F0F0F0Fu;  // elements j, j+2, j+4, j+6
        f[8 * h + j] = ubyte<0>(m) - z;
        f[8 * h + j + 2] = ubyte<1>(m) - z;
        f[8 * h + j + 4] = ubyte<2>(m) - z;
        f[8 * h + j + 6] = ubyte<3>(m) - z;
      }
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) w[i] = pack_exact(f[2 * i], f[2 * i + 1]);
}

template <int BM, int BITS, bool ASYM, bool YBF16>
__global__ __launch_bounds__(QTile<BM>::THREADS, BM == 128 ? 2 : 1) void qgemm_kernel(
    const QgemmParams P) {
  using T = QTile<BM>;
  constexpr int QA_BYTES = T::A_BYTES, QB_BYTES = T::B_BYTES, QS_OFF = T::S_OFF;
  constexpr int TPR = T::TPR, CPT = T::CPT;
  extern __shared__ __align__(16) uint8_t smem[];
  const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
  const int wm = wv % T::WMC, wn = wv / T::WMC;
  const int K = P.k, N = P.n_out, G = P.group;
  const int NT = N / QG_BN;

  // Tile order: workgroups are dealt round-robin to the 8 XCDs; renumber so
  // that each XCD runs a contiguous range of tiles, outputs fastest: the
  // workgroups an XCD runs together share their activation rows in its L2.
  const uint32_t nblk = gridDim.x, b = blockIdx.x;
  const uint32_t per = nblk >> 3, rem = nblk & 7, xcd = b & 7;
  const uint32_t logical = xcd * per + (xcd < rem ? xcd : rem) + (b >> 3);
  const int mt = (int)(logical / (uint32_t)NT);
  const int nt = (int)(logical - (uint32_t)mt * (uint32_t)NT);
  const int64_t m0 = (int64_t)mt * BM;
  const int n0 = nt * QG_BN;
  const int mrows = group_rows(P.rows, mt, BM);

  constexpr int CB = CPT * BITS / 8;  // code bytes per thread per chunk
  constexpr int NW = CB / 4;          // ... as 32-bit words
  const int KB = K * BITS / 8;  // code bytes per weight row
  const int NG = K / G;         // groups per weight row
  const auto ra = buffer_range32(P.a + m0 * K, (uint32_t)mrows * (uint32_t)K * 2u);
  const auto rc = buffer_range32(P.codes + (int64_t)n0 * KB, (uint32_t)(QG_BN * KB));
  const auto rs = buffer_range32(P.scales + (int64_t)n0 * NG, (uint32_t)(QG_BN * NG * 2));
  const auto rz = buffer_range32(ASYM ? P.zeros + (int64_t)n0 * NG : P.scales,
                                 ASYM ? (uint32_t)(QG_BN * NG * 2) : 0u);

  // loads of one chunk: activations 4 x 16 B per thread (rows t/8 + BM/4 i),
  // codes of one weight row (t / TPR), elements CPT (t % TPR) .. + CPT-1
  const int arow = t >> 3, akc = t & 7;
  const uint32_t a_off = (uint32_t)(arow * K + akc * 8) * 2u;
  const uint32_t a_step = (uint32_t)(BM / 4 * K) * 2u;
  const int cn = t / TPR, cq = t % TPR;
  const uint32_t c_off = (uint32_t)(cn * KB + cq * CB);
  // Register prefetch two chunks deep: slot c % 2 holds chunk c from its
  // loads until its LDS stash one iteration before its compute, so a load
  // has about two chunks of matrix work to arrive.
  uint4 ar[2][4];
  uint32_t cr[2][NW];
  // fp16 bits (converted where used, so no load is waited for early): the
  // chunk's zero point (for the decode) and its group's scale of the weight
  // row t / 4 (stashed to LDS with the chunk, read back by the lanes of its
  // output column after the chunk's matrix work)
  uint16_t zr[2] = {0, 0};
  uint16_t sr[2] = {0, 0};
  // this lane's two output columns (C layout of the 32 x 32 tiles: lane l
  // holds column l % 32)
  const int col0 = wn * 64 + (lane & 31);
  auto issue = [&](auto slot_c, int c) {
    constexpr int SL = decltype(slot_c)::value;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      ar[SL][i] = buf_ld16(ra, a_off + i * a_step + (uint32_t)c * (QG_BK * 2));
    const uint32_t off = c_off + (uint32_t)c * (QG_BK * BITS / 8);
    if (NW == 1) {
      cr[SL][0] = buf_ld4(rc, off);
    } else if (NW == 2) {
      const u32x2_t v = __builtin_amdgcn_raw_buffer_load_b64(rc, (int)off, 0, 0);
      cr[SL][0] = v.x;
      cr[SL][NW - 1] = v.y;
    } else {
      const uint4 v = buf_ld16(rc, off);
      cr[SL][0] = v.x;
      cr[SL][1 % NW] = v.y;
      cr[SL][2 % NW] = v.z;
      cr[SL][3 % NW] = v.w;
    }
    const int g = c * QG_BK / G;
    if (ASYM) zr[SL] = __builtin_amdgcn_raw_buffer_load_b16(rz, (int)((cn * NG + g) * 2), 0, 0);
    sr[SL] = __builtin_amdgcn_raw_buffer_load_b16(rs, (int)((cn * NG + g) * 2), 0, 0);
  };
  auto stash = [&](auto slot_c, int bi) {
    constexpr int SL = decltype(slot_c)::value;
    uint8_t* Ab = smem + bi * QA_BYTES;
    uint8_t* Bb = smem + 2 * QA_BYTES + bi * QB_BYTES;
#pragma unroll
    for (int i = 0; i < 4; ++i) lds_st16(Ab + (arow + BM / 4 * i) * QROW + akc * 16, ar[SL][i]);
    const float z = ASYM ? half_to_float(zr[SL]) : (float)(1 << (BITS - 1));
#pragma unroll
    for (int u = 0; u < CPT / 16; ++u) {  // 16 codes at a time
      uint32_t x[BITS / 2];
#pragma unroll
      for (int h = 0; h < BITS / 2; ++h) {
        const uint32_t v = cr[SL][u * (BITS / 2) + h];
        x[h] = ASYM ? v : v ^ (BITS == 2 ? 0xAAAAAAAAu : 0x88888888u);
      }
      uint32_t w[8];
      decode16<BITS>(x, z, w);
      uint8_t* dst = Bb + cn * QROW + cq * (CPT * 2) + u * 32;
      lds_st16(dst, make_uint4(w[0], w[1], w[2], w[3]));
      lds_st16(dst + 16, make_uint4(w[4], w[5], w[6], w[7]));
    }
    if (cq == 0) *reinterpret_cast<uint16_t*>(smem + QS_OFF + bi * (QG_BN * 2) + cn * 2) = sr[SL];
  };

  f32x16_t Y[2][2], Pg[2][2];
  const f32x16_t zero = {};
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) Y[i][j] = zero;


  const int nch = K / QG_BK, cpg = G / QG_BK;
  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  issue(S0(), 0);
  issue(S1(), 1);
  stash(S0(), 0);
  __syncthreads();
  // chunk c: its slot and LDS buffer are c % 2 (SL)
  auto body = [&](auto slot_c, int c) {
    constexpr int SL = decltype(slot_c)::value;
    using Next = std::integral_constant<int, SL ^ 1>;
    const bool gfirst = (c % cpg) == 0, glast = (c % cpg) == cpg - 1;
    // Unconditional (a conditional load makes the waits below conservative
    // and drains the prefetch): past the last chunk the offsets only reach
    // other rows' data or fall outside the ranges, and nothing uses them.
    issue(slot_c, c + 2);
    const uint8_t* Ab = smem + SL * QA_BYTES + (wm * 64 + (lane & 31)) * QROW + (lane >> 5) * 16;
    const uint8_t* Bb = smem + 2 * QA_BYTES + SL * QB_BYTES + col0 * QROW + (lane >> 5) * 16;
#pragma unroll
    for (int kk = 0; kk < QG_BK / 16; ++kk) {
      bf16x8_t af[2], bfr[2];
#pragma unroll
      for (int i = 0; i < 2; ++i)
        af[i] = __builtin_bit_cast(bf16x8_t, lds_ld16(Ab + 32 * i * QROW + kk * 32));
#pragma unroll
      for (int j = 0; j < 2; ++j)
        bfr[j] = __builtin_bit_cast(bf16x8_t, lds_ld16(Bb + 32 * j * QROW + kk * 32));
      if (kk == 0 && gfirst) {
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j)
            Pg[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], zero, 0, 0, 0);
      } else {
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j)
            Pg[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], Pg[i][j], 0, 0, 0);
      }
    }
    if (glast) {
      const uint16_t* sl = reinterpret_cast<const uint16_t*>(smem + QS_OFF + SL * (QG_BN * 2));
      const float s_now[2] = {half_to_float(sl[col0]), half_to_float(sl[col0 + 32])};
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            Y[i][j][r] = fmaf(s_now[j], Pg[i][j][r], Y[i][j][r]);
    }
    stash(Next(), SL ^ 1);  // past the last chunk: into the idle buffer, unread
    __syncthreads();
  };
  int c = 0;
  for (; c + 1 < nch; c += 2) {
    body(S0(), c);
    body(S1(), c + 1);
  }
  if (c < nch) body(S0(), c);

  // store: register r of tile (i, j) is row 8 (r / 4) + 4 (lane / 32) + r % 4
  // of the tile, column lane % 32; rows past the end fall outside the range
  constexpr int YSZ = YBF16 ? 2 : 4;
  const auto ry = buffer_range32(static_cast<char*>(P.y) + m0 * N * YSZ,
                                 (uint32_t)mrows * (uint32_t)N * YSZ);
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = wm * 64 + 32 * i + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        const uint32_t off = (uint32_t)(row * N + n0 + col0 + 32 * j) * YSZ;
        if (YBF16) buf_st2(ry, off, (uint16_t)pack_bf16(Y[i][j][r], 0.f));
        else buf_st4(ry, off, __float_as_uint(Y[i][j][r]));
      }
}

// Few rows (decode time: one to a few dozen tokens): the product is bound by
// reading and decoding the codes once, and MFMA tiles of 256 rows would be
// mostly padding.  One wave per QV_OPW weight rows; lane l takes QV_KU
// consecutive codes per step (k = QV_KU l + 64 QV_KU i, inside one group:
// group >= 64); with QV_KU = 64 a row of 4096 codes is one step with every
// load in flight at once.  The codes are decoded to
// exact bf16 pairs as above; for each of the MR activation rows the 64-term
// sum is formed with v_dot2c_f32_bf16 (exact products), scaled by the
// group's scale and accumulated in fp32.  The 64 lanes' sums are then added
// by an xor-shuffle tree (fixed order) and lane m * QV_OPW + r stores y[m][r].
constexpr int QV_OPW = 4;   // weight rows per wave

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

template <int BITS, bool ASYM, bool YBF16, int MR, int QV_KU>
__global__ __launch_bounds__(256) void qgemv_kernel(const QgemmParams P) {
  static_assert(MR * QV_OPW <= 64, "one lane per output");
  constexpr int NW = QV_KU * BITS / 32;  // code words per lane per row and step
  const int lane = threadIdx.x & 63;
  const int o0 = (blockIdx.x * 4 + (threadIdx.x >> 6)) * QV_OPW;  // n_out % 16 == 0
  const int K = P.k, G = P.group, N = P.n_out, NG = K / G;
  const int KB = K * BITS / 8;
  const int64_t m0 = (int64_t)blockIdx.y * MR;
  const int mrows = group_rows(P.rows, blockIdx.y, MR);
  const auto ra = buffer_range32(P.a + m0 * K, (uint32_t)mrows * (uint32_t)K * 2u);
  const auto rc = buffer_range32(P.codes + (int64_t)o0 * KB, (uint32_t)(QV_OPW * KB));
  const auto rs = buffer_range32(P.scales + (int64_t)o0 * NG, (uint32_t)(QV_OPW * NG * 2));
  const auto rz = buffer_range32(ASYM ? P.zeros + (int64_t)o0 * NG : P.scales,
                                 ASYM ? (uint32_t)(QV_OPW * NG * 2) : 0u);
  float acc[MR][QV_OPW];
#pragma unroll
  for (int m = 0; m < MR; ++m)
#pragma unroll
    for (int r = 0; r < QV_OPW; ++r) acc[m][r] = 0.f;
  for (int k0 = lane * QV_KU; k0 < K; k0 += 64 * QV_KU) {
    const int g = k0 / G;
    uint32_t cw[QV_OPW][NW];
    uint16_t sb[QV_OPW], zb[QV_OPW];
#pragma unroll
    for (int r = 0; r < QV_OPW; ++r) {
      const uint32_t off = (uint32_t)(r * KB + k0 * BITS / 8);
      if (NW == 1) {
        cw[r][0] = buf_ld4(rc, off);
      } else if (NW == 2) {
        const u32x2_t v = __builtin_amdgcn_raw_buffer_load_b64(rc, (int)off, 0, 0);
        cw[r][0] = v.x;
        cw[r][NW - 1] = v.y;
      } else {
#pragma unroll
        for (int h = 0; h < NW / 4; ++h) {
          const uint4 v = buf_ld16(rc, off + 16 * h);
          cw[r][4 * h] = v.x;
          cw[r][(4 * h + 1) % NW] = v.y;
          cw[r][(4 * h + 2) % NW] = v.z;
          cw[r][(4 * h + 3) % NW] = v.w;
        }
      }
      const uint32_t so = (uint32_t)((r * NG + g) * 2);
      sb[r] = __builtin_amdgcn_raw_buffer_load_b16(rs, (int)so, 0, 0);
      zb[r] = ASYM ? __builtin_amdgcn_raw_buffer_load_b16(rz, (int)so, 0, 0) : (uint16_t)0;
    }
    if constexpr (BITS == 2 && MR == 1) {
      // One activation row, 2-bit codes: decode through a byte permute.  The
      // four values q - z of the row's group are bf16 entries of an 8-byte
      // table (exact small integers); codes i and i + 8 of a 16-code word sit
      // 16 bits apart, so one shift and mask put them in the two halves of
      // t, t * 0x202 + 0x01000100 is the byte selector of their table
      // entries, and v_perm_b32 gives the pair (w_i, w_i+8).  The activations
      // are re-paired the same way once, for all the weight rows.
      uint32_t pa[QV_KU / 2];
      {
        const uint32_t ao = (uint32_t)k0 * 2u;
#pragma unroll
        for (int u = 0; u < QV_KU / 16; ++u) {
          const uint4 v0 = buf_ld16(ra, ao + 32 * u), v1 = buf_ld16(ra, ao + 32 * u + 16);
          const uint32_t av[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
#pragma unroll
          for (int i = 0; i < 8; ++i)
            pa[8 * u + i] = __builtin_amdgcn_perm(av[4 + i / 2], av[i / 2],
                                                  (i & 1) ? 0x07060302u : 0x05040100u);
        }
      }
#pragma unroll
      for (int r = 0; r < QV_OPW; ++r) {
        uint32_t lut_lo, lut_hi;
        if (ASYM) {
          const float z = half_to_float(zb[r]);
          lut_lo = pack_exact(-z, 1.f - z);
          lut_hi = pack_exact(2.f - z, 3.f - z);
        } else {  // two's complement: 0, 1, -2, -1
          lut_lo = 0x3F800000u;  // (0, 1)
          lut_hi = 0xBF80C000u;              // (-2, -1)
        }
        float part = 0.f;
#pragma unroll
        for (int u = 0; u < QV_KU / 16; ++u) {
          const uint32_t x = cw[r][u];
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const uint32_t tq = (x >> (2 * i)) & 0x00030003u;
            const uint32_t w = __builtin_amdgcn_perm(lut_hi, lut_lo, tq * 0x202u + 0x01000100u);
            part = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pa[8 * u + i]),
                                                   __builtin_bit_cast(bf16x2_t, w), part, false);
          }
        }
        acc[0][r] = fmaf(half_to_float(sb[r]), part, acc[0][r]);
      }
      continue;
    }
    // one weight row at a time (its 32 decoded words), against every
    // activation row (re-read from the cache for each weight row)
#pragma unroll
    for (int r = 0; r < QV_OPW; ++r) {
      const float z = ASYM ? half_to_float(zb[r]) : (float)(1 << (BITS - 1));
      uint32_t w[QV_KU / 2];
#pragma unroll
      for (int u = 0; u < QV_KU / 16; ++u) {
        uint32_t x[BITS / 2];
#pragma unroll
        for (int h = 0; h < BITS / 2; ++h) {
          const uint32_t v = cw[r][u * (BITS / 2) + h];
          x[h] = ASYM ? v : v ^ (BITS == 2 ? 0xAAAAAAAAu : 0x88888888u);
        }
        uint32_t wu[8];
        decode16<BITS>(x, z, wu);
#pragma unroll
        for (int i = 0; i < 8; ++i) w[8 * u + i] = wu[i];
      }
      const float sr = half_to_float(sb[r]);
#pragma unroll
      for (int m = 0; m < MR; ++m) {
        const uint32_t ao = (uint32_t)(m * K + k0) * 2u;
        float part = 0.f;
#pragma unroll
        for (int q = 0; q < QV_KU / 8; ++q) {
          const uint4 v = buf_ld16(ra, ao + 16 * q);
          const uint32_t av[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
          for (int i = 0; i < 4; ++i)
            part = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, av[i]),
                                                   __builtin_bit_cast(bf16x2_t, w[4 * q + i]),
                                                   part, false);
        }
        acc[m][r] = fmaf(sr, part, acc[m][r]);
      }
    }
  }
  // lane sums, fixed-order tree; every lane ends with every total
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1)
#pragma unroll
    for (int m = 0; m < MR; ++m)
#pragma unroll
      for (int r = 0; r < QV_OPW; ++r) acc[m][r] += __shfl_xor(acc[m][r], off, 64);
  float mine = 0.f;
#pragma unroll
  for (int m = 0; m < MR; ++m)
#pragma unroll
    for (int r = 0; r < QV_OPW; ++r)
      if (lane == m * QV_OPW + r) mine = acc[m][r];
  if (lane < MR * QV_OPW) {  // rows past the end fall outside the range
    constexpr int YSZ = YBF16 ? 2 : 4;
    const auto ry = buffer_range32(static_cast<char*>(P.y) + m0 * N * YSZ,
                                   (uint32_t)mrows * (uint32_t)N * YSZ);
    const uint32_t off = (uint32_t)((lane / QV_OPW) * N + o0 + lane % QV_OPW) * YSZ;
    if (YBF16) buf_st2(ry, off, (uint16_t)pack_bf16(mine, 0.f));
    else buf_st4(ry, off, __float_as_uint(mine));
  }
}

template <int BITS, bool ASYM, bool YBF16, int MR, int KU>
hipError_t launch_gemv(const QgemmParams& p, hipStream_t s) {
  const dim3 grid((unsigned)(p.n_out / (4 * QV_OPW)), (unsigned)((p.rows + MR - 1) / MR));
  hipLaunchKernelGGL((qgemv_kernel<BITS, ASYM, YBF16, MR, KU>), grid, dim3(256), 0, s, p);
  return hipGetLastError();
}

template <int BITS, bool ASYM, bool YBF16>
hipError_t launch_one(const QgemmParams& p, hipStream_t s) {
  if (p.rows <= QG_GEMV_ROWS) {
    // one row: 64 codes per lane (a 4096-code row in one step, the decode
    // dominates); more rows: 16 per lane, the dot products dominate
    if (p.rows == 1) return launch_gemv<BITS, ASYM, YBF16, 1, 64>(p, s);
    if (p.rows <= 4) return launch_gemv<BITS, ASYM, YBF16, 4, 16>(p, s);
    return launch_gemv<BITS, ASYM, YBF16, 16, 16>(p, s);
  }
  constexpr int BM = QG_BM;
  using T = QTile<BM>;
  const void* fn = reinterpret_cast<const void*>(qgemm_kernel<BM, BITS, ASYM, YBF16>);
  const hipError_t lds_ok = kernel_setup(fn, T::THREADS, T::LDS, nullptr, nullptr);
  if (lds_ok != hipSuccess) return lds_ok;
  const int64_t mt = (p.rows + BM - 1) / BM;
  const int64_t blocks = mt * (p.n_out / QG_BN);
  hipLaunchKernelGGL((qgemm_kernel<BM, BITS, ASYM, YBF16>), dim3((unsigned)blocks),
                     dim3(T::THREADS), T::LDS, s, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_qgemm(const QgemmParams& p, hipStream_t s) {
  if (p.rows == 0) return hipSuccess;
  if (p.bits == 2) {
    if (p.asym) return p.y_bf16 ? launch_one<2, true, true>(p, s) : launch_one<2, true, false>(p, s);
    return p.y_bf16 ? launch_one<2, false, true>(p, s) : launch_one<2, false, false>(p, s);
  }
  if (p.asym) return p.y_bf16 ? launch_one<4, true, true>(p, s) : launch_one<4, true, false>(p, s);
  return p.y_bf16 ? launch_one<4, false, true>(p, s) : launch_one<4, false, false>(p, s);
}

}  // namespace bfly
