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
#include <algorithm>
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

// Few rows on the matrix cores.  Codes are decoded by the chip's format
// converters: a 2-bit code masked into a nibble is the fp4 (e2m1) number
// q / 2, a 4-bit code masked into a byte the fp8 (e4m3) number q 2^-9, and
// v_cvt_scalef32_pk_bf16_fp4 / _fp8 with the scale 2 (2^9) give two of
// them as the bf16 pair of the integers q, exactly.  Masking a 16-code word
// (2-bit) into its even and odd nibbles, or an 8-code word (4-bit) into its
// even and odd bytes, gives the pairs (q0, q2) (q1, q3) (q4, q6) (q5, q7) of
// every eight codes: 11 vector operations per 16 two-bit codes.  Symmetric
// codes have their sign bit flipped in the same masking (offset binary,
// z = 2^(bits-1)).
// The products run on v_mfma_f32_16x16x32_bf16: up to 16 activation rows
// are A (rows past the end read as zero, or repeat the last row), 16 weight
// rows are B; lane l holds eight k of block l / 16 of row l % 16 in both
// operands (the activations re-paired to the codes' pair order), and
// C[4 (l / 16) + i][l % 16].
// Zero points: per group the codes give C = sum a q, a second product
// against ones gives S = sum a, and the group adds s (C - z S).  Each
// product a q is exact; the sums are fp32.
// Work split: a workgroup per 16 weight rows with one wave per 1024 codes
// of k (up to MAXW waves; each takes a run of whole groups, in passes of
// 1024), the waves' sums added through LDS in fixed order.  A wave reads
// its codes in segments of 256 per row: lane l loads 16 (4-bit: 32)
// contiguous bytes of row l % 16, four lanes 64 (128) contiguous bytes.  A
// 4 x 4 transpose of dwords across the four 16-lane rows
// (v_permlane32_swap, then v_permlane16_swap) leaves lane l with codes
// 16 (l / 16) .. + 15 (4-bit: 8 (l / 16) .. + 7 and 32 + 8 (l / 16) .. + 7)
// of each 64-code chunk, so that the 32 codes of a step lie in one chunk,
// inside one group.  Each wave stages the scales and zero points of its
// groups, and (up to four rows) its activations, in its own part of LDS:
// those loads are issued before the codes, so waiting for them leaves the
// codes in flight (loads complete in issue order), and no workgroup
// barrier comes before the k loop.
constexpr int QV_PASS = 16;       // 64-code chunks per wave and pass (1024 codes)
constexpr int QV_LDS_ROWS = 4;    // activation rows staged in LDS at most
constexpr int QV_AW = 4;          // chunks of activations in flight (rows read from memory)
// waves per workgroup at most (the launch bound: more waves leave fewer
// registers per lane)
__host__ __device__ constexpr int qv_maxw(int bits, int q, int ni) {
  return (bits == 2 && q >= 2 && ni <= 2) ? 16 : 8;
}

template <int SEL>
__device__ __forceinline__ uint32_t fp4_pair(uint32_t v) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(v, 2.0f, SEL));
}
template <bool HI>
__device__ __forceinline__ uint32_t fp8_pair(uint32_t v) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v, 512.0f, HI));
}

// Activations (a0 .. a7) of one step in the codes' pair order:
// (a0, a2) (a1, a3) (a4, a6) (a5, a7).
__device__ __forceinline__ bf16x8_t pair_order(uint4 w) {
  u32x4_t r;
  r.x = __builtin_amdgcn_perm(w.y, w.x, 0x05040100u);
  r.y = __builtin_amdgcn_perm(w.y, w.x, 0x07060302u);
  r.z = __builtin_amdgcn_perm(w.w, w.z, 0x05040100u);
  r.w = __builtin_amdgcn_perm(w.w, w.z, 0x07060302u);
  return __builtin_bit_cast(bf16x8_t, r);
}

// After the call v[d] of lane-row r (lanes 16 r .. 16 r + 15) holds what
// v[r] of lane-row d held.
__device__ __forceinline__ void transpose4_rows(uint32_t& v0, uint32_t& v1, uint32_t& v2,
                                                uint32_t& v3) {
  const auto p0 = __builtin_amdgcn_permlane32_swap(v0, v2, false, false);
  const auto p1 = __builtin_amdgcn_permlane32_swap(v1, v3, false, false);
  const auto q0 = __builtin_amdgcn_permlane16_swap(p0[0], p1[0], false, false);
  const auto q1 = __builtin_amdgcn_permlane16_swap(p0[1], p1[1], false, false);
  v0 = q0[0];
  v1 = q0[1];
  v2 = q1[0];
  v3 = q1[1];
}

// Calls f(integral_constant<int, i>) for i = I .. COUNT-1, in order.
template <int I, int COUNT, class F>
__device__ __forceinline__ void static_for_from(F&& f) {
  if constexpr (I < COUNT) {
    f(std::integral_constant<int, I>());
    static_for_from<I + 1, COUNT>(f);
  }
}

// Q: 64-code chunks per group (group / 64); NI: rows of C used per lane;
// AL: activations staged in LDS (at most QV_LDS_ROWS rows) or read from
// memory; MAXW: waves per workgroup at most.  Workgroup (x, y) takes the
// weight rows 16 x .. + 15 and the activation rows 16 y .. + 15.
template <int BITS, int Q, int NI, bool AL, int MAXW>
__global__ __launch_bounds__(64 * MAXW) void qmv_kernel(const QgemmParams P) {
  typedef float f32x4_t __attribute__((ext_vector_type(4)));
  static_assert(QV_PASS % Q == 0, "shape");
  constexpr int MT = 1;
  constexpr int LPS = BITS / 2;       // b128 loads per lane and 256-code segment
  constexpr int GP = QV_PASS / Q;     // groups per pass
  constexpr int RS = GP >= 4 ? GP / 4 : 1;  // scale (zero) halves staged per lane and pass
  const int nw = (int)(blockDim.x >> 6);
  const int tid = (int)threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar control
  const int n = lane & 15, j = lane >> 4;
  const int o0 = blockIdx.x * 16;
  const int K = P.k, N = P.n_out, NG = K / (64 * Q);
  const int KB = K * BITS / 8;
  const int mrows = group_rows(P.rows, blockIdx.y, 16);  // at most QV_LDS_ROWS with AL
  const uint16_t* A = P.a + (int64_t)blockIdx.y * 16 * P.k;
  const bool asym = P.asym;
  const int gpw = (NG + nw - 1) / nw;
  const int gbeg = min(NG, wave * gpw);
  const int T = (min(NG, gbeg + gpw) - gbeg) * Q;  // chunks of this wave
  // LDS: per wave [scales, zeros: 16 x GP fp16] [activations (AL): mrows x 1024
  // bf16]; after the k loop, the waves' sums [nw][16 MT][16] fp32
  extern __shared__ __align__(16) uint8_t qv_lds[];
  constexpr int WSZ = 64 * GP;
  const int wbytes = WSZ + (AL ? mrows * 2048 : 0);
  uint16_t* ls = reinterpret_cast<uint16_t*>(qv_lds + wave * wbytes);
  uint16_t* lz = ls + 16 * GP;
  uint8_t* la = qv_lds + wave * wbytes + WSZ;

  const uint32_t szbytes = (uint32_t)(32 * NG);
  const auto rs = buffer_range32(P.scales + (int64_t)o0 * NG, szbytes);
  const auto rz = buffer_range32(asym ? P.zeros + (int64_t)o0 * NG : P.scales, asym ? szbytes : 0u);
  const auto ra = buffer_range32(A, (uint32_t)mrows * (uint32_t)K * 2u);
  const uint32_t cl = (uint32_t)(n * KB + j * 16 * LPS);  // lane part of a code offset
  const uint32_t kx = asym ? 0u : (BITS == 2 ? 0xAAAAAAAAu : 0x88888888u);  // sign flip

  uint16_t sst[RS], zst[RS];
  uint4 ast[AL ? (NI == 1 ? 2 : 2 * QV_LDS_ROWS) : 1];
  uint32_t cw[4][4 * LPS];
  // the loads of a pass starting at chunk c0 (group gbeg + c0 / Q), in the
  // order they are used: scales and zeros, activations, codes
  auto issue = [&](const int c0) {
    const int g0 = gbeg + c0 / Q;
#pragma unroll
    for (int r = 0; r < RS; ++r) {
      const int gl = j + 4 * r;  // this lane's group of the pass
      const bool ok = gl < GP && c0 + gl * Q < T;
      const uint32_t off = ok ? (uint32_t)(2 * (n * NG + g0 + gl)) : 0xFFFFFFF0u;
      sst[r] = __builtin_amdgcn_raw_buffer_load_b16(rs, (int)off, 0, 0);
      zst[r] = __builtin_amdgcn_raw_buffer_load_b16(rz, (int)off, 0, 0);
    }
    if constexpr (AL && NI == 1) {
      // one row: lane l takes elements 8 l and 8 (l + 64) of the pass's 1024
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int e = 64 * c0 + 8 * (lane + 64 * h);
        const uint32_t off = e < 64 * T ? (uint32_t)(2 * (64 * Q * gbeg + e)) : 0xFFFFFFF0u;
        ast[h] = buf_ld16(ra, off);
      }
    } else if constexpr (AL) {
      // rows 0 .. 3 (zero past the end) x the pass's 1024 codes: lane l
      // takes 32 bytes of row l / 16
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int e = 64 * c0 + 16 * (lane & 15) + 8 * h;  // element of the wave's k run
        const bool ok = (lane >> 4) < mrows && e < 64 * T;
        const uint32_t off = ok ? (uint32_t)(2 * ((lane >> 4) * K + 64 * Q * gbeg + e)) : 0xFFFFFFF0u;
        ast[h] = buf_ld16(ra, off);
      }
#pragma unroll
      for (int h = 2; h < 2 * QV_LDS_ROWS; ++h) {
        // pieces 2 .. 7: the same rows, the next 256 elements each
        const int e = 64 * c0 + 256 * (h / 2) + 16 * (lane & 15) + 8 * (h & 1);
        const bool ok = (lane >> 4) < mrows && e < 64 * T;
        const uint32_t off = ok ? (uint32_t)(2 * ((lane >> 4) * K + 64 * Q * gbeg + e)) : 0xFFFFFFF0u;
        ast[h] = buf_ld16(ra, off);
      }
    }
    static_for_from<0, 4>([&](auto sc) {
      constexpr int sg = decltype(sc)::value;
      const bool live = c0 + 4 * sg < T;
      // all of the offset in the range-checked (vector) part: a segment
      // may run past the end of the row (its chunks past T are not used)
      const auto rc = buffer_range32(P.codes + (int64_t)o0 * KB, live ? (uint32_t)(16 * KB) : 0u);
      const uint32_t su = live ? (uint32_t)((64 * Q * gbeg + 64 * (c0 + 4 * sg)) * BITS / 8) : 0u;
#pragma unroll
      for (int h = 0; h < LPS; ++h) {
        const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(rc, (int)(cl + su + 16u * h), 0, 0);
        cw[sg][4 * h + 0] = v.x;
        cw[sg][4 * h + 1] = v.y;
        cw[sg][4 * h + 2] = v.z;
        cw[sg][4 * h + 3] = v.w;
      }
    });
  };
  // staged values into this wave's LDS (waits for them, not for the codes)
  auto stage = [&]() {
#pragma unroll
    for (int r = 0; r < RS; ++r) {
      const int gl = j + 4 * r;
      if (gl < GP) {
        ls[n * GP + gl] = sst[r];
        lz[n * GP + gl] = zst[r];
      }
    }
    if constexpr (AL && NI == 1) {
#pragma unroll
      for (int h = 0; h < 2; ++h)
        *reinterpret_cast<bf16x8_t*>(la + 16 * (lane + 64 * h)) = pair_order(ast[h]);
    } else if constexpr (AL) {
      // piece h of lane l: row l / 16, elements 256 (h / 2) + 16 (l % 16) + 8 (h % 2),
      // stored in the codes' pair order (re-paired once here, not per step)
      if ((lane >> 4) < mrows) {
#pragma unroll
        for (int h = 0; h < 2 * QV_LDS_ROWS; ++h)
          *reinterpret_cast<bf16x8_t*>(la + 2 * ((lane >> 4) * 1024 + 256 * (h / 2) +
                                                 16 * (lane & 15) + 8 * (h & 1))) = pair_order(ast[h]);
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  };

  // activations read from memory (MT tiles of 16 rows), QV_AW chunks ahead
  const int arow = AL ? min(n, mrows - 1) : n;
  const int ak0 = BITS == 2 ? 16 * j : 8 * j;  // lane's elements of a chunk's steps
  const int ak1 = ak0 + (BITS == 2 ? 8 : 32);
  uint4 aw[AL ? 1 : QV_AW][MT][2];
  auto issue_a = [&](const int t, auto slot_c) {
    if constexpr (!AL) {
      constexpr int sl = decltype(slot_c)::value;
      const bool live = t < T;
      const auto ral = buffer_range32(A, live ? (uint32_t)mrows * (uint32_t)K * 2u : 0u);
      const int kc = 64 * Q * gbeg + 64 * t;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const int e = (arow + 16 * mt) * K + kc;
        aw[sl][mt][0] = buf_ld16(ral, (uint32_t)(2 * (e + ak0)));
        aw[sl][mt][1] = buf_ld16(ral, (uint32_t)(2 * (e + ak1)));
      }
    }
  };
  const u32x4_t ones_w = {0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};
  const bf16x8_t ones = __builtin_bit_cast(bf16x8_t, ones_w);
  const f32x4_t zero4 = {0.f, 0.f, 0.f, 0.f};
  // two sets of group sums (even and odd groups), so that a group's
  // scaling can overlap the next group's products
  f32x4_t C[2][MT], S[2][MT], acc[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) acc[mt] = zero4;
  const float zsym = (float)(1 << (BITS - 1));
  const uint8_t* la_lane = la + 2 * (arow * 1024 + ak0);

  auto pass = [&](const int c0) {
    static_for_from<0, QV_AW>([&](auto pc) { issue_a(c0 + (int)decltype(pc)::value, pc); });
    static_for_from<0, 4>([&](auto sc) {
      constexpr int sg = decltype(sc)::value;
      uint32_t y[4 * LPS];
#pragma unroll
      for (int w = 0; w < 4 * LPS; ++w) y[w] = cw[sg][w];
      if (c0 + 4 * sg >= T) return;
      transpose4_rows(y[0], y[1], y[2], y[3]);
      if constexpr (LPS == 2) transpose4_rows(y[4], y[5], y[6], y[7]);
      static_for_from<0, 4>([&](auto dc) {
        constexpr int d = decltype(dc)::value;
        constexpr int tl = 4 * sg + d;       // chunk within the pass
        constexpr int gl = tl / Q, ps = gl & 1;  // group within the pass, its set of sums
        const int t = c0 + tl;
        uint4 ar[MT][2];
        if constexpr (!AL) {
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) {
            ar[mt][0] = aw[tl % QV_AW][mt][0];
            ar[mt][1] = aw[tl % QV_AW][mt][1];
          }
          if constexpr (tl + QV_AW < QV_PASS) issue_a(t + QV_AW, std::integral_constant<int, tl % QV_AW>());
        }
        if (t >= T) return;
        u32x4_t b[2];
        if constexpr (BITS == 2) {
          const uint32_t x = y[d], xs = x >> 2;
          const uint32_t lo = (x ^ kx) & 0x33333333u, hi = (xs ^ (kx >> 2)) & 0x33333333u;
          b[0] = u32x4_t{fp4_pair<0>(lo), fp4_pair<0>(hi), fp4_pair<1>(lo), fp4_pair<1>(hi)};
          b[1] = u32x4_t{fp4_pair<2>(lo), fp4_pair<2>(hi), fp4_pair<3>(lo), fp4_pair<3>(hi)};
        } else {
#pragma unroll
          for (int w = 0; w < 2; ++w) {
            const uint32_t x = y[d + 4 * w], xs = x >> 4;
            const uint32_t lo = (x ^ kx) & 0x0F0F0F0Fu, hi = (xs ^ (kx >> 4)) & 0x0F0F0F0Fu;
            b[w] = u32x4_t{fp8_pair<false>(lo), fp8_pair<false>(hi), fp8_pair<true>(lo),
                           fp8_pair<true>(hi)};
          }
        }
        bf16x8_t a[MT][2];
        if constexpr (AL) {
          a[0][0] = *reinterpret_cast<const bf16x8_t*>(la_lane + 128 * tl);
          a[0][1] = *reinterpret_cast<const bf16x8_t*>(la_lane + 128 * tl + 2 * (ak1 - ak0));
        } else {
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) {
            a[mt][0] = pair_order(ar[mt][0]);
            a[mt][1] = pair_order(ar[mt][1]);
          }
        }
        const bf16x8_t b0 = __builtin_bit_cast(bf16x8_t, b[0]);
        const bf16x8_t b1 = __builtin_bit_cast(bf16x8_t, b[1]);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          C[ps][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[mt][0], b0, tl % Q == 0 ? zero4 : C[ps][mt], 0, 0, 0);
          S[ps][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[mt][0], ones, tl % Q == 0 ? zero4 : S[ps][mt], 0, 0, 0);
          C[ps][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[mt][1], b1, C[ps][mt], 0, 0, 0);
          S[ps][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[mt][1], ones, S[ps][mt], 0, 0, 0);
        }
        if constexpr (tl % Q == Q - 1) {  // the group's last chunk: add s (C - z S)
          const float sc = half_to_float(ls[n * GP + gl]);
          const float z = asym ? half_to_float(lz[n * GP + gl]) : zsym;
#pragma unroll
          for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int i = 0; i < NI; ++i)
              acc[mt][i] = fmaf(sc, fmaf(-z, S[ps][mt][i], C[ps][mt][i]), acc[mt][i]);
        }
      });
    });
  };
  // One pass (k up to 1024 per wave): straight code, no loop, so that the
  // compiler tracks every load in flight exactly.  Longer runs loop.
  issue(0);
  stage();
  if (T <= QV_PASS) {
    pass(0);
  } else {
    pass(0);
    for (int c0 = QV_PASS; c0 < T; c0 += QV_PASS) {
      issue(c0);
      stage();
      pass(c0);
    }
  }

  // --- the waves' sums, added in wave order ---
  __syncthreads();  // every wave is done with its staged values
  float* red = reinterpret_cast<float*>(qv_lds);  // [nw][16 MT][16]
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int i = 0; i < NI; ++i) red[(wave * MT * 16 + mt * 16 + 4 * j + i) * 16 + n] = acc[mt][i];
  __syncthreads();
  const int ysz = P.y_bf16 ? 2 : 4;
  const auto ry = buffer_range32(static_cast<char*>(P.y) + (int64_t)blockIdx.y * 16 * N * ysz,
                                 (uint32_t)mrows * (uint32_t)N * (uint32_t)ysz);
  for (int e = tid; e < MT * 256; e += 64 * nw) {
    const int m = e >> 4, c = e & 15;
    if (m < mrows) {
      float v = red[m * 16 + c];
      for (int w = 1; w < nw; ++w) v += red[(w * MT * 16 + m) * 16 + c];
      const uint32_t off = (uint32_t)(m * N + o0 + c) * (uint32_t)ysz;
      if (P.y_bf16) buf_st2(ry, off, (uint16_t)pack_bf16(v, 0.f));
      else buf_st4(ry, off, __float_as_uint(v));
    }
  }
}

template <int BITS, int Q, int NI, bool AL>
hipError_t launch_mv(const QgemmParams& p, hipStream_t s) {
  constexpr int MT = 1;
  constexpr int MAXW = qv_maxw(BITS, Q, NI);
  constexpr int GP = QV_PASS / Q;
  const int nw = std::min(MAXW, (p.k + 1023) / 1024);
  const size_t wbytes = (size_t)64 * GP + (AL ? (size_t)p.rows * 2048 : 0);
  const size_t lds = std::max((size_t)nw * wbytes, (size_t)nw * MT * 1024);
  const void* fn = reinterpret_cast<const void*>(qmv_kernel<BITS, Q, NI, AL, MAXW>);
  const hipError_t e = allow_lds(fn, lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((qmv_kernel<BITS, Q, NI, AL, MAXW>),
                     dim3((unsigned)(p.n_out / 16), (unsigned)((p.rows + 15) / 16)), dim3(64 * nw),
                     lds, s, p);
  return hipGetLastError();
}

template <int BITS, int Q>
hipError_t launch_mv_rows(const QgemmParams& p, hipStream_t s) {
  if (p.rows == 1) return launch_mv<BITS, Q, 1, true>(p, s);
  if (p.rows == 2) return launch_mv<BITS, Q, 2, true>(p, s);
  if (p.rows <= QV_LDS_ROWS) return launch_mv<BITS, Q, 4, true>(p, s);
  return launch_mv<BITS, Q, 4, false>(p, s);  // 16 rows per workgroup row
}

template <int BITS>
hipError_t launch_mv_group(const QgemmParams& p, hipStream_t s) {
  switch (p.group) {
    case 64: return launch_mv_rows<BITS, 1>(p, s);
    case 128: return launch_mv_rows<BITS, 2>(p, s);
    case 256: return launch_mv_rows<BITS, 4>(p, s);
    default: return launch_mv_rows<BITS, 8>(p, s);
  }
}

template <int BITS, bool ASYM, bool YBF16>
hipError_t launch_one(const QgemmParams& p, hipStream_t s) {
  if (p.rows <= QG_GEMV_ROWS) return launch_mv_group<BITS>(p, s);
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
