// Forward butterfly (plain and Kronecker composite) fused with per-group
// round-to-nearest quantization.  Included by the instantiation units.
//
// Per row of n = M * NB elements (M = 1: plain butterfly of length NB):
//   load (bf16 or fp32, 16-byte vectors) -> L = log2 NB Givens stages on each
//   of the M segments -> [M > 1: mix the segments with the M x M factor,
//   column by column] -> store y (bf16 / fp32 / none) -> group max/min ->
//   fp16 scale (and zero) -> codes, packed, stored.
//
// The coefficients of every pair a thread rotates stay in its VGPRs for all
// the rows it processes (8 per stage, 16 for the last), so after the
// prologue the only HBM traffic is the rows themselves.  A stage needs both
// elements of each pair in one thread's registers, or in two lanes one DPP
// operand connects: the scaled form runs in two phases (register bits plus
// lane-mapped bits, see FwdPlan) with two LDS transposes per row; the
// three-shear fallback runs in register-only phases of 3 bits, transposed
// through LDS between them.  Workgroup transposes are double-buffered, one
// barrier each.  The grid is persistent: each workgroup walks row groups
// with stride gridDim.x and prefetches the next group's input while
// computing.
#pragma once

#include <hip/hip_ext.h>

#include "bfly_common.h"

namespace bfly {

// RPT rows per thread: the same (cos, sin) registers serve RPT rows at once,
// halving the barriers and coefficient traffic per row and doubling the
// independent work between barriers.
template <int LOGNB, int M, int RPT>
struct FwdShape {
  static constexpr int LOGE = 3;
  static constexpr int NB = 1 << LOGNB;
  static constexpr int E = 1 << LOGE;
  static constexpr int T = NB >> LOGE;             // threads per row team
  static constexpr int LOGT = ilog2c(T);
  static constexpr int N = M * NB;                 // row length
  static constexpr int SEGS = RPT * M;             // segments a thread carries
  static constexpr int SEGW = lds_words(NB);       // padded LDS words per segment
  static constexpr int L = LOGNB;
  static constexpr int NPH = (L + LOGE - 1) / LOGE;  // register phases
  static constexpr int R_THREADS = (256 / T) > 0 ? (256 / T) : 1;
  static constexpr int R_LDS = (8192 / (SEGS * NB)) > 0 ? (8192 / (SEGS * NB)) : 1;
  static constexpr int R = R_THREADS < R_LDS ? R_THREADS : R_LDS;  // teams per workgroup
  static constexpr int NT = T * R;                 // threads per workgroup
  static constexpr int ROWS_PER_PASS = R * RPT;
  // Row groups whose input is in flight ahead of the one being computed
  // (each slot holds SEGS segments of the input in registers).  Measured at
  // n = 4096: two slots of one segment beat one (the load of the next group
  // is issued a full group earlier) and three (more registers, no gain); with
  // two segments (two rows per thread) one slot beats two and three (more
  // requests in flight lower the streaming rate), and three or four rows per
  // thread are slower than two.
  static constexpr int PD = SEGS == 1 ? 2 : 1;
  static constexpr int BUFW = R * SEGS * SEGW;     // words per LDS buffer
  // LDS addressing of the transpose into phase k (see LdsMode).
  static constexpr int id_transpose(int k) {
    return local_transpose(k) ? LDS_PAD
           : same_lane_bits(phase_base(k - 1, L, LOGE), k < NPH ? phase_base(k, L, LOGE) : 0) ? LDS_ID
           : (k == NPH && phase_base(k - 1, L, LOGE) >= 9) ? LDS_P512
           : LDS_PAD;
  }
  static_assert(lds_index(NB - 1, LDS_P512) < SEGW && lds_index(NB - 1, LDS_ID) < SEGW,
                "every addressing stays inside a segment's words");
  static constexpr bool local_transpose(int k) {   // transpose into phase k (k = NPH: back to 0)
    return wave_local(phase_base(k - 1, L, LOGE), k < NPH ? phase_base(k, L, LOGE) : 0, LOGT);
  }
  // Workgroup transposes before the last one (its buffer parity).
  static constexpr int final_gidx() {
    int g = 0;
    for (int k = 1; k < NPH; ++k) g += local_transpose(k) ? 0 : 1;
    return g;
  }
  static constexpr bool any_global() {
    for (int k = 1; k <= NPH; ++k)
      if (!local_transpose(k)) return true;
    return false;
  }
  // one buffer for wave-local transposes, two alternating ones for the rest
  static constexpr size_t LDS_BYTES = (any_global() ? 3ull : 1ull) * BUFW * sizeof(float);

  // The scaled form's two-phase plan (lane-mapped stages through DPP; see
  // FwdPlan): transposes A -> B and B -> A, wave-local when a team fits in
  // one wave.  LDS word of element i (lds2):
  //   i + 4 (i >> 5) + PADB (i >> 7) + PADE (i >> (L-3)).
  // The LDS serves 32 lanes of a 4-byte access, or 8 of a 16-byte one, per
  // pass over 32 banks.  Layout A's 16-byte accesses (8 elements per lane,
  // 8 lanes at element bits 3..5) need the 4 words per 32; layout B's 4-byte
  // accesses (32 lanes: element bits 0.. plus the lane-mapped bits SA..,
  // 128 apart) need lane-mapped blocks an odd multiple of 8 (DB = 2) or of 4
  // (DB = 3) banks apart, hence PADB; PADE makes the step between layout B's
  // registers a multiple of 64 words so register pairs share one
  // ds_read2st64 / ds_write2st64 (from n = 1024 on; smaller rows transpose
  // within a wave and keep their buffer small).  No pad depends on bits that vary within
  // one pass, except as stated, so every pass meets 32 distinct banks.
  static constexpr FwdPlan PL = fwd_plan(L);
  static constexpr bool TWO = PL.SA < L;
  static constexpr bool LOCAL2 = T <= 64;
  static constexpr int PADB = PL.DB == 2 ? 8 : (PL.DB == 3 ? 4 : 0);
  static constexpr int RSTEP0 = (1 << (L - 3)) + 4 * ((1 << (L - 3)) >> 5) + PADB * ((1 << (L - 3)) >> 7);
  static constexpr int PADE = (L >= 10) ? (64 - RSTEP0 % 64) % 64 : 0;
  static constexpr int lds2w(int i) {
    return i + 4 * (i >> 5) + PADB * (i >> 7) + PADE * (i >> (L - 3));
  }
  static constexpr int SEGW2 = (lds2w(NB - 1) + 4) & ~3;
  static constexpr int BUF2W = R * SEGS * SEGW2;
  static_assert((TWO ? (LOCAL2 ? 1 : 2) * BUF2W : 0) * sizeof(float) <= LDS_BYTES,
                "the two-phase buffers fit the allocation of the three-shear form");
};

// LDS word of element i in the two-phase transposes.
template <class S>
__device__ __forceinline__ constexpr int lds2(int i) { return S::lds2w(i); }

// A lane-mapped stage of the scaled form on a thread's 8 registers: each
// lane adds k_e times its partner lane's register e (the partner reached by
// the DPP control; every lane reads the old values).  One v_fmac_f32_dpp per
// element, as in inline assembly: the compiler does not fold a DPP move into
// a multiply-add.  s_nop 1 first: a DPP operand must not have been written
// by a VALU instruction in the two issue slots before (within the block each
// source was last written a full stage earlier).
#define BFLY_DPP_OP(I, D, S, K, CTRL) \
  "v_fmac_f32_dpp %" #D ", %" #S ", %" #K " " CTRL " row_mask:0xf bank_mask:0xf\n"
// In place: register e's own DPP source is register e.
#define BFLY_LANE_FMA8_IP(CTRL, V, K)                                                            \
  asm("s_nop 1\n" BFLY_DPP_OP(0, 0, 0, 8, CTRL) BFLY_DPP_OP(1, 1, 1, 9, CTRL)                   \
          BFLY_DPP_OP(2, 2, 2, 10, CTRL) BFLY_DPP_OP(3, 3, 3, 11, CTRL)                           \
              BFLY_DPP_OP(4, 4, 4, 12, CTRL) BFLY_DPP_OP(5, 5, 5, 13, CTRL)                       \
                  BFLY_DPP_OP(6, 6, 6, 14, CTRL) BFLY_DPP_OP(7, 7, 7, 15, CTRL)                   \
      : "+v"(V[0]), "+v"(V[1]), "+v"(V[2]), "+v"(V[3]), "+v"(V[4]), "+v"(V[5]), "+v"(V[6]),     \
        "+v"(V[7])                                                                                \
      : "v"(K[0]), "v"(K[1]), "v"(K[2]), "v"(K[3]), "v"(K[4]), "v"(K[5]), "v"(K[6]), "v"(K[7]))
// Into separate accumulators.
#define BFLY_LANE_FMA8_ACC(CTRL, ACC, SRC, K)                                                    \
  asm("s_nop 1\n" BFLY_DPP_OP(0, 0, 8, 16, CTRL) BFLY_DPP_OP(1, 1, 9, 17, CTRL)                 \
          BFLY_DPP_OP(2, 2, 10, 18, CTRL) BFLY_DPP_OP(3, 3, 11, 19, CTRL)                         \
              BFLY_DPP_OP(4, 4, 12, 20, CTRL) BFLY_DPP_OP(5, 5, 13, 21, CTRL)                     \
                  BFLY_DPP_OP(6, 6, 14, 22, CTRL) BFLY_DPP_OP(7, 7, 15, 23, CTRL)                 \
      : "+v"(ACC[0]), "+v"(ACC[1]), "+v"(ACC[2]), "+v"(ACC[3]), "+v"(ACC[4]), "+v"(ACC[5]),     \
        "+v"(ACC[6]), "+v"(ACC[7])                                                                \
      : "v"(SRC[0]), "v"(SRC[1]), "v"(SRC[2]), "v"(SRC[3]), "v"(SRC[4]), "v"(SRC[5]),           \
        "v"(SRC[6]), "v"(SRC[7]), "v"(K[0]), "v"(K[1]), "v"(K[2]), "v"(K[3]), "v"(K[4]),         \
        "v"(K[5]), "v"(K[6]), "v"(K[7]))
// The DPP control of lane-map mask j: j = 0, 1: quad permutes (lane ^ 1,
// lane ^ 2); j = 2: half-row mirror (lane ^ 7); j = 3: row mirror (lane ^ 15).
#define BFLY_DPP_SWITCH(J, MACRO, ...)                          \
  switch (J) {                                                  \
    case 0: MACRO("quad_perm:[1,0,3,2]", __VA_ARGS__); break;    \
    case 1: MACRO("quad_perm:[2,3,0,1]", __VA_ARGS__); break;    \
    case 2: MACRO("row_half_mirror", __VA_ARGS__); break;        \
    default: MACRO("row_mirror", __VA_ARGS__); break;            \
  }

// A lane-mapped stage s < L-1, on lane-map bit j.
__device__ __forceinline__ void lane_stage(int j, float (&v)[8], const float (&c0)[4],
                                           const float (&c1)[4]) {
  float k[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) k[e] = (e & 1) ? c1[e >> 1] : c0[e >> 1];
  BFLY_DPP_SWITCH(j, BFLY_LANE_FMA8_IP, v, k)
}
// The last stage on a lane-mapped bit: y_e = a_e w_e + b_e w_partner, with
// last[h] = (a_2h, b_2h, a_2h+1, b_2h+1).
__device__ __forceinline__ void lane_last(int j, float (&v)[8], const float4 (&last)[4]) {
  float acc[8], b[8];
#pragma unroll
  for (int h = 0; h < 4; ++h) {
    acc[2 * h] = last[h].x * v[2 * h];
    acc[2 * h + 1] = last[h].z * v[2 * h + 1];
    b[2 * h] = last[h].y;
    b[2 * h + 1] = last[h].w;
  }
  BFLY_DPP_SWITCH(j, BFLY_LANE_FMA8_ACC, acc, v, b)
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] = acc[e];
}

// One of stages 0..L-2 on the pair (a, b): two fused multiply-adds on the
// stored values in the scaled form (c0 = beta, c1 = gamma), else three
// shears (c0 = p, c1 = u).
template <bool FAST>
__device__ __forceinline__ void rotate(float& a, float& b, float c0, float c1) {
  if (FAST) {
    const float a0 = a;
    a = fmaf(c0, b, a);
    b = fmaf(c1, a0, b);
  } else {
    shear3(a, b, c0, c1);
  }
}


// Cross-lane max/min over the `gt` consecutive lanes of a quantization group
// (gt a power of two <= 64).  Within a 16-lane DPP row: xor-1 and xor-2 quad
// permutes, then the half-row mirror (lane l <-> 7 - l) joins the two quads
// of a half-row and the row mirror (l <-> 15 - l) the two halves; wider
// groups use bpermute.
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
constexpr int DPP_XOR1 = 0xB1;         // quad_perm [1,0,3,2]
constexpr int DPP_XOR2 = 0x4E;         // quad_perm [2,3,0,1]
constexpr int DPP_HALF_MIRROR = 0x141;
constexpr int DPP_MIRROR = 0x140;

__device__ __forceinline__ float group_max(float v, int gt) {
  if (gt >= 2) v = fmaxf(v, dpp<DPP_XOR1>(v));
  if (gt >= 4) v = fmaxf(v, dpp<DPP_XOR2>(v));
  if (gt >= 8) v = fmaxf(v, dpp<DPP_HALF_MIRROR>(v));
  if (gt >= 16) v = fmaxf(v, dpp<DPP_MIRROR>(v));
  if (gt >= 32) v = fmaxf(v, __shfl_xor(v, 16));
  if (gt >= 64) v = fmaxf(v, __shfl_xor(v, 32));
  return v;
}
__device__ __forceinline__ float group_min(float v, int gt) {
  if (gt >= 2) v = fminf(v, dpp<DPP_XOR1>(v));
  if (gt >= 4) v = fminf(v, dpp<DPP_XOR2>(v));
  if (gt >= 8) v = fminf(v, dpp<DPP_HALF_MIRROR>(v));
  if (gt >= 16) v = fminf(v, dpp<DPP_MIRROR>(v));
  if (gt >= 32) v = fminf(v, __shfl_xor(v, 16));
  if (gt >= 64) v = fminf(v, __shfl_xor(v, 32));
  return v;
}

// Quantization of the E = 8 consecutive values one thread holds (part of a
// group spread over gt = group/8 consecutive lanes), in two steps: the
// group's parameters, then the codes.
//
// Scale: s16 = fp16(absmax / qmax) or fp16((max - min) / levels), the
// quotient taken as a product with the fp32 reciprocal of the constant (it
// can differ from the correctly rounded quotient only within 2 fp32 ulps of
// an fp16 rounding midpoint).  Codes: q = rne(y * r) with r = 1/s16 (one
// Newton step on the hardware reciprocal), computed as
// fma(y, r, 1.5*2^23 + bias): the exact product is rounded once, to an
// integer, ties to even, and the low bits of the result's encoding are
// q + bias.  Clamping y to [qlo*s16, qhi*s16] (products exact in fp32) is the
// same as clamping q afterwards.  The clamp changes a code only when some
// y * r of the group rounds outside [qlo, qhi].  With the symmetric scale
// that needs a scale that lost precision (fp16 subnormal, or saturated at
// 65504): near_edge flags a group within 1/4 of that (room to spare for the
// fp32 rounding of the extremes' products), and callers may skip the clamp
// where no group is.  With the asymmetric one the zero point's own rounding
// can push the top code one past qhi as well, and near_edge fires for about
// half the groups: callers clamp those always.
struct QParams {
  float r, clo, chi, z;
  uint32_t sz;  // fp16 scale bits (low half), zero-point bits (high half)
  bool near_edge;
};
__device__ __forceinline__ QParams quant_params(const float (&v)[8], int gt, bool asym, float inv_top,
                                                float top) {
  float lo, hi;
  if (asym) {
    lo = fminf(fminf(fminf(v[0], v[1]), fminf(v[2], v[3])), fminf(fminf(v[4], v[5]), fminf(v[6], v[7])));
    hi = fmaxf(fmaxf(fmaxf(v[0], v[1]), fmaxf(v[2], v[3])), fmaxf(fmaxf(v[4], v[5]), fmaxf(v[6], v[7])));
    lo = group_min(lo, gt);
    hi = group_max(hi, gt);
  } else {
    // a chain the compiler maps onto three-input maxima (4 instructions)
    hi = fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fabsf(v[2]));
    hi = fmaxf(fmaxf(hi, fabsf(v[3])), fabsf(v[4]));
    hi = fmaxf(fmaxf(hi, fabsf(v[5])), fabsf(v[6]));
    hi = fmaxf(hi, fabsf(v[7]));
    hi = group_max(hi, gt);
    lo = 0.f;
  }
  const float s_pre = fminf((hi - lo) * inv_top, 65504.f);  // saturate to the largest finite fp16
  const _Float16 s16 = (_Float16)s_pre;
  const float sc = (float)s16;
  QParams q;
  // Branch-free: a zero scale (all-zero group, or max = min) selects r = 0,
  // so every code, the zero point and both bounds come out zero.
  q.r = __builtin_amdgcn_rcpf(sc);
  q.r = fmaf(fmaf(-sc, q.r, 1.0f), q.r, q.r);
  q.r = sc != 0.f ? q.r : 0.f;
  q.z = asym ? __builtin_amdgcn_fmed3f(rintf(-lo * q.r), 0.f, top) : 0.f;
  q.clo = asym ? -q.z * sc : -top * sc;
  q.chi = (top - q.z) * sc;
  q.sz = (uint32_t)__builtin_bit_cast(uint16_t, s16) |
         ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)q.z) << 16);
  // z and top are small integers: the bounds are exact.
  q.near_edge = hi * q.r > (top - q.z) + 0.25f || lo * q.r < -q.z - 0.25f;
  return q;
}
__device__ __forceinline__ void quant_clamp(float (&v)[8], const QParams& q) {
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] = __builtin_amdgcn_fmed3f(v[e], q.clo, q.chi);
}
// The packed codes of v, already clamped (or known not to need it).
__device__ __forceinline__ uint32_t quant_pack(const float (&v)[8], const QParams& q, int bits, bool asym) {
  uint32_t packed;
  if (!asym && bits == 4) {
    // biased nibbles q + 8 in 1..15, two per byte, then two's complement by ^8
    uint32_t f[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) f[e] = __float_as_uint(fmaf(v[e], q.r, 12582920.0f));
    const uint32_t p0 = (f[1] << 4) | f[0], p1 = (f[3] << 4) | f[2];
    const uint32_t p2 = (f[5] << 4) | f[4], p3 = (f[7] << 4) | f[6];
    const uint32_t w01 = __builtin_amdgcn_perm(p1, p0, 0x0C0C0400u);  // [p0.b0, p1.b0, 0, 0]
    const uint32_t w23 = __builtin_amdgcn_perm(p3, p2, 0x04000C0Cu);  // [0, 0, p2.b0, p3.b0]
    packed = (w01 | w23) ^ 0x88888888u;
  } else if (asym) {
    // The bits of fma(y, r, 1.5*2^23) are 0x4B400000 + q as an integer, so
    // sum_e (q_e + z) << (bits*e), whose fields cannot carry once the codes
    // are clamped to [0, 2^bits - 1], is sum_e bits_e << (bits*e) plus one
    // constant per group, in wrapping 32-bit arithmetic.
    // z in every field: z * 0x5555 or z * 0x1111 (twice) is exact in fp32
    const uint32_t rep = bits == 2 ? 0x5555u : 0x11111111u;  // sum_e 2^(bits*e)
    const uint32_t zr = (uint32_t)(q.z * (bits == 2 ? 21845.0f : 4369.0f));
    const uint32_t zrep = bits == 2 ? zr : (zr | (zr << 16));
    // Horner form, one v_lshl_add_u32 per element (the compiler otherwise
    // splits the sum into separate shifts and three-input adds)
    packed = __float_as_uint(fmaf(v[7], q.r, 12582912.0f));
#pragma unroll
    for (int e = 6; e >= 0; --e) {
      const uint32_t f = __float_as_uint(fmaf(v[e], q.r, 12582912.0f));
      if (bits == 2)  // the only asymmetric widths are 2 and 4
        asm("v_lshl_add_u32 %0, %1, 2, %2" : "=v"(packed) : "v"(packed), "v"(f));
      else
        asm("v_lshl_add_u32 %0, %1, 4, %2" : "=v"(packed) : "v"(packed), "v"(f));
    }
    packed += zrep - 0x4B400000u * rep;
  } else {
    const uint32_t off = (uint32_t)q.z - 0x4B400000u;
    const uint32_t mask = (1u << bits) - 1u;
    packed = 0;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float f = fmaf(v[e], q.r, 12582912.0f);
      packed |= ((__float_as_uint(f) + off) & mask) << (bits * e);
    }
  }
  return packed;
}

// Output / quantizer variants of the row loop, fixed at compile time so the
// loop carries no mode branches.
// Q_S4G128 and Q_A2G128 fix the two common formats (symmetric INT4 and
// asymmetric INT2, groups of 128) at compile time, so the group reductions
// are straight-line code the scheduler can interleave with the rotations;
// Q_ANY reads bits, group and mode at run time.
enum QMode : int { Q_NONE = 0, Q_S4G128 = 1, Q_A2G128 = 2, Q_ANY = 3 };

// Number of workgroup-wide (non wave-local) transposes in one row.
template <class S>
__host__ __device__ constexpr int global_transposes() {
  int g = 0;
  for (int k = 1; k <= S::NPH; ++k) g += S::local_transpose(k) ? 0 : 1;
  return g;
}

// The coefficients of every pair one thread rotates, for either form.
template <class S>
struct Coeffs {
  float c0[S::L - 1][S::E / 2];
  float c1[S::L - 1][S::E / 2];
  float4 last[S::E / 2];
};

// The persistent row loop for one (input, output, quantizer) variant.
// Input registers of one row group: SEGS segments of 16-byte vectors.
template <class S, bool XBF16>
struct InRegs {
  static constexpr int RAW = XBF16 ? S::E / 8 : S::E / 4;  // 16-byte vectors per segment
  uint4 r[S::PD][S::SEGS][RAW];
};

// Issue the loads of row group grp into prefetch slot d, through a buffer
// resource covering exactly the group's valid rows (none past the end).
// elem0: the element of the thread's register 0 within its row segment.
// Non-temporal: every input line is read once (-0.7 us at n = 4096, 8192
// rows).  XS: rows lie XS * n elements apart (XS = 2: one half of each row of
// twice the length).
template <class S, bool XBF16, int XS = 1>
__device__ __forceinline__ void load_group(const FwdParams& P, const int64_t rows, const int64_t grp,
                                           InRegs<S, XBF16>& in, const int d, const int team,
                                           const int elem0) {
  constexpr int N = S::N, NB = S::NB, RPP = S::ROWS_PER_PASS;
  constexpr int RPT = S::ROWS_PER_PASS / S::R, M = S::SEGS / RPT;
  constexpr int RAW = InRegs<S, XBF16>::RAW, ESZ = XBF16 ? 2 : 4;
  constexpr int LD = XS * N;  // row stride in elements
  const uint32_t valid = (uint32_t)group_rows(rows, grp, RPP);
  const auto rs = buffer_range32(reinterpret_cast<const char*>(P.x) + grp * ((int64_t)RPP * LD) * ESZ,
                                 valid * (uint32_t)(LD * ESZ));
  const int thr_elem = team * RPT * LD + elem0;
#pragma unroll
  for (int rr = 0; rr < RPT; ++rr)
#pragma unroll
    for (int a = 0; a < M; ++a)
#pragma unroll
      for (int c = 0; c < RAW; ++c)
        in.r[d][rr * M + a][c] =
            buf_ld16<kNonTemporal>(rs, (uint32_t)(thr_elem + rr * LD + a * NB) * ESZ + 16 * c);
}

// PRE: the caller has already issued the prologue's loads (slot d holds row
// group blockIdx.x + d * gridDim.x), before its own set-up work.
// CHECK: the coefficients are still arriving.  The block's first row group
// runs before anything waits for all of them (each phase waits for its own
// stages' loads only); then the coefficients are checked for the NaN marker
// of an unusable scaled form.  If any workgroup thread saw one, the loop
// stops after that group (whose stored outputs are garbage) and returns
// false, and the caller must redo every row.  The early stop only shortens
// the loop: a separate exit path would put the two forms' loops on two arms
// of a branch, where the register allocator does far worse.
template <class S, bool XBF16, int YK, int QM, bool FAST, bool PRE, bool CHECK, int XS = 1>
__device__ __forceinline__ bool row_loop(const FwdParams& P, const int64_t rows, float* lds, int team,
                                         int t, const Coeffs<S>& C, InRegs<S, XBF16>& in) {
  constexpr int LOGE = S::LOGE, E = S::E, NB = S::NB, N = S::N, M = S::SEGS / (S::ROWS_PER_PASS / S::R);
  constexpr int RPT = S::ROWS_PER_PASS / S::R;
  constexpr int SEGS = S::SEGS, SEGW = S::SEGW, BUFW = S::BUFW, RPP = S::ROWS_PER_PASS;
  constexpr int L = S::L, NPH = S::NPH;
  constexpr int RAW = XBF16 ? E / 8 : E / 4;  // 16-byte vectors per segment
  constexpr bool QUANT = QM != Q_NONE;
  constexpr int LD = XS * N;  // row stride of x and y in elements
  static_assert(XS == 1 || (!QUANT && M == 1), "strided rows: plain butterfly, rows only");
  static_assert(global_transposes<S>() % 2 == 0, "buffer alternation assumes an even count");

  float* const lbuf = lds + team * (SEGS * SEGW);          // wave-local transposes
  float* const gbuf0 = lds + BUFW + team * (SEGS * SEGW);  // workgroup transposes
  float* const gbuf1 = lds + 2 * BUFW + team * (SEGS * SEGW);

  const int64_t ngrp = (rows + RPP - 1) / RPP;
  constexpr bool FIXED = QM == Q_S4G128 || QM == Q_A2G128;
  const int bits = QM == Q_S4G128 ? 4 : (QM == Q_A2G128 ? 2 : P.bits);
  const bool asym = QM == Q_A2G128 || (QM == Q_ANY && P.asym != 0);
  const int group = FIXED ? 128 : P.group;
  const int gt = QUANT ? group / E : 1;
  const int lg_group = QUANT ? 31 - __builtin_clz(group) : 0;
  const float top = asym ? (float)((1 << bits) - 1) : (float)((1 << (bits - 1)) - 1);
  const float inv_top = 1.0f / top;
  const int ngroups_row = QUANT ? N >> lg_group : 0;

  // Memory: every row group gets buffer resources covering exactly its valid
  // rows (bases and sizes uniform across the workgroup, in scalar
  // registers); each thread adds fixed 32-bit offsets.  Rows past the end,
  // groups past the end and lanes with nothing to store fall outside the
  // ranges, so no memory instruction sits under a branch and the compiler
  // can keep every prefetch in flight.
  constexpr int64_t GRP_ELEMS = (int64_t)RPP * LD;
  // Element of the thread's register 0 within a row segment: the two-phase
  // plan's layout A for the scaled form, register-contiguous blocks for the
  // three-shear form.
  const int elem0 = FAST ? fwd_elem_a(t, 0, S::PL) : t * E;
  const int thr_elem = team * RPT * LD + elem0;  // element offset of (team, t) in a group

  constexpr int PD = S::PD;
  auto& cur = in.r;
  auto load = [&](int64_t grp, int d) { load_group<S, XBF16, XS>(P, rows, grp, in, d, team, elem0); };

  // The previous row group's outputs: bf16 rows, codes and scales (and, for
  // fp32 output, its rows), stored only once the next group's input has
  // arrived, so the wait for that input never has to wait for freshly issued
  // stores as well.  Non-temporal: every output line is written once
  // (measured at n = 4096: 36.0 -> 34.3 us for 8192 rows).
  uint32_t held_y[SEGS][E / 2], held_c[SEGS], held_sz[SEGS];
#pragma unroll
  for (int sg = 0; sg < SEGS; ++sg) {
#pragma unroll
    for (int k = 0; k < E / 2; ++k) held_y[sg][k] = 0u;
    held_c[sg] = held_sz[sg] = 0u;
  }
  int64_t held_grp = -1;
  const bool scale_lane = QUANT && (t & (gt - 1)) == 0;
  auto flush = [&](const float (&w)[SEGS][E]) {
    if (YK == Y_NONE && !QUANT) return;
    const int64_t hg = held_grp;
    const uint32_t vr = (uint32_t)group_rows(rows, hg, RPP);  // at most RPP rows: 32-bit sizes
    const auto ry = buffer_range32(reinterpret_cast<const uint16_t*>(P.y) + hg * GRP_ELEMS, vr * (LD * 2));
    const auto ry4 = buffer_range32(reinterpret_cast<const float*>(P.y) + hg * GRP_ELEMS, vr * (LD * 4));
    const auto rc = buffer_range32(P.codes + hg * (GRP_ELEMS * bits / 8), vr * (uint32_t)(N * bits / 8));
    const auto rsc = buffer_range32(P.scales + hg * RPP * ngroups_row, vr * (uint32_t)(ngroups_row * 2));
    const auto rz = buffer_range32(P.zeros + hg * RPP * ngroups_row, vr * (uint32_t)(ngroups_row * 2));
#pragma unroll
    for (int rr = 0; rr < RPT; ++rr)
#pragma unroll
      for (int a = 0; a < M; ++a) {
        const int sg = rr * M + a;
        const uint32_t el = (uint32_t)(thr_elem + rr * LD + a * NB);
        if (YK == Y_BF16) {
#pragma unroll
          for (int c = 0; c < E / 8; ++c)
            buf_st16<kNonTemporal>(ry, el * 2 + 16 * c,
                     make_uint4(held_y[sg][4 * c], held_y[sg][4 * c + 1], held_y[sg][4 * c + 2],
                                held_y[sg][4 * c + 3]));
        } else if (YK == Y_F32) {
#pragma unroll
          for (int c = 0; c < E / 4; ++c)
            buf_st16<kNonTemporal>(ry4, el * 4 + 16 * c,
                     make_uint4(__float_as_uint(w[sg][4 * c]), __float_as_uint(w[sg][4 * c + 1]),
                                __float_as_uint(w[sg][4 * c + 2]), __float_as_uint(w[sg][4 * c + 3])));
        }
        if (QUANT) {
          if (bits == 4) buf_st4<kNonTemporal>(rc, el / 2, held_c[sg]);
          else buf_st2<kNonTemporal>(rc, el / 4, (uint16_t)held_c[sg]);
          const uint32_t gi = (uint32_t)((team * RPT + rr) * ngroups_row + ((a * NB + elem0) >> lg_group));
          const uint32_t off = scale_lane ? 2 * gi : kOutOfRange;
          buf_st2<kNonTemporal>(rsc, off, (uint16_t)held_sz[sg]);
          if (asym) buf_st2<kNonTemporal>(rz, off, (uint16_t)(held_sz[sg] >> 16));
        }
      }
  };

  // The M x M factor, read once into scalar registers (uniform values; the
  // compiler cannot prove the matrix unaliased by the outputs, and would
  // otherwise reload it into vector registers for every row group).
  float mixs[M > 1 ? M * M : 1];
#pragma unroll
  for (int i = 0; i < (M > 1 ? M * M : 1); ++i)
    mixs[i] = M > 1 ? __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(P.mix[i]))) : 0.f;
  const int64_t G = gridDim.x;

  // The last transpose of a row group leaves its rows in layout 0 in this
  // buffer; the next slot (or the epilogue) reads them there.
  float* const fin_buf = S::local_transpose(NPH) ? lbuf : ((S::final_gidx() & 1) ? gbuf1 : gbuf0);
  // Two-phase plan (scaled form): A -> B through abuf, B -> A through bbuf
  // (the same buffer when a team is one wave's: its LDS accesses stay in
  // order).  One-phase rows keep their results in registers (fin).
  constexpr int SEGW2 = S::SEGW2;
  float* const abuf = lds + team * (SEGS * SEGW2);
  float* const bbuf = S::LOCAL2 ? abuf : lds + S::BUF2W + team * (SEGS * SEGW2);
  const int ea = lds2<S>(elem0);
  const int eb = lds2<S>(fwd_elem_b(t, 0, S::PL));
  float fin[SEGS][E];
#pragma unroll
  for (int sg = 0; sg < SEGS; ++sg)
#pragma unroll
    for (int e = 0; e < E; ++e) fin[sg][e] = 0.f;
  auto get_a = [&](const float* buf, float (&x)[E]) {
    const float4 q0 = *reinterpret_cast<const float4*>(buf + ea);
    const float4 q1 = *reinterpret_cast<const float4*>(buf + ea + 4);
    x[0] = q0.x; x[1] = q0.y; x[2] = q0.z; x[3] = q0.w;
    x[4] = q1.x; x[5] = q1.y; x[6] = q1.z; x[7] = q1.w;
  };
  auto put_a = [&](float* buf, const float (&x)[E]) {
    *reinterpret_cast<float4*>(buf + ea) = make_float4(x[0], x[1], x[2], x[3]);
    *reinterpret_cast<float4*>(buf + ea + 4) = make_float4(x[4], x[5], x[6], x[7]);
  };
  auto get_b = [&](const float* buf, float (&x)[E]) {
#pragma unroll
    for (int e = 0; e < E; ++e) x[e] = buf[eb + lds2<S>(e << (L - 3))];
  };
  auto put_b = [&](float* buf, const float (&x)[E]) {
#pragma unroll
    for (int e = 0; e < E; ++e) buf[eb + lds2<S>(e << (L - 3))] = x[e];
  };
  auto sync2 = [&]() {
    if (S::LOCAL2) wave_lds_sync();
    else __syncthreads();
  };
  auto read_final = [&](float (&w)[SEGS][E]) {
    if (FAST) {
      if (S::TWO) {
#pragma unroll
        for (int sg = 0; sg < SEGS; ++sg) get_a(bbuf + sg * SEGW2, w[sg]);
        if (S::LOCAL2) wave_lds_sync();
      } else {
#pragma unroll
        for (int sg = 0; sg < SEGS; ++sg)
#pragma unroll
          for (int e = 0; e < E; ++e) w[sg][e] = fin[sg][e];
      }
      return;
    }
#pragma unroll
    for (int sg = 0; sg < SEGS; ++sg)
      lds_get1<LOGE, SEGW>(fin_buf + sg * SEGW, w[sg], t, 0, S::id_transpose(NPH));
    if (S::local_transpose(NPH)) wave_lds_sync();
  };
  // Scaled form, two-phase plan: the stages of phase A and of phase B.
  auto phase_a = [&](float (&x)[E]) {
#pragma unroll
    for (int s = 0; s < 3; ++s)
#pragma unroll
      for (int j = 0; j < E / 2; ++j) {
        const int lo = pair_lo(j, s), hi = lo | (1 << s);
        rotate<true>(x[lo], x[hi], C.c0[s][j], C.c1[s][j]);
      }
#pragma unroll
    for (int s = 3; s < S::PL.SA; ++s) {
      if (s < L - 1) lane_stage(s - 3, x, C.c0[s], C.c1[s]);
      else lane_last(s - 3, x, C.last);
    }
  };
  auto phase_b = [&](float (&x)[E]) {
#pragma unroll
    for (int s = S::PL.SA; s < L - 3; ++s) lane_stage(s - S::PL.SA, x, C.c0[s], C.c1[s]);
#pragma unroll
    for (int s = (S::PL.SA > L - 3 ? S::PL.SA : L - 3); s < L; ++s) {
      const int q = s - (L - 3);
#pragma unroll
      for (int j = 0; j < E / 2; ++j) {
        const int lo = pair_lo(j, q), hi = lo | (1 << q);
        if (s < L - 1) rotate<true>(x[lo], x[hi], C.c0[s][j], C.c1[s][j]);
        else last2x2(x[lo], x[hi], C.last[j]);
      }
    }
  };
  // Everything the previous group still needs before its stores: the
  // Kronecker mix, bf16 packing and quantization.
  auto finish = [&](float (&w)[SEGS][E]) {
    if (M > 1) {  // Kronecker mix across a row's segments, column by column
#pragma unroll
      for (int rr = 0; rr < RPT; ++rr)
#pragma unroll
        for (int e = 0; e < E; ++e) {
          float mw[M];
#pragma unroll
          for (int a = 0; a < M; ++a) {
            float acc = mixs[a * M] * w[rr * M][e];
#pragma unroll
            for (int a2 = 1; a2 < M; ++a2) acc = fmaf(mixs[a * M + a2], w[rr * M + a2][e], acc);
            mw[a] = acc;
          }
#pragma unroll
          for (int a = 0; a < M; ++a) w[rr * M + a][e] = mw[a];
        }
    }
    if (YK == Y_BF16) {
#pragma unroll
      for (int sg = 0; sg < SEGS; ++sg)
#pragma unroll
        for (int k = 0; k < E / 2; ++k) {
          held_y[sg][k] = pack_bf16(w[sg][2 * k], w[sg][2 * k + 1]);
          // packed here, so the unclamped values die before the clamp below
          asm volatile("" : "+v"(held_y[sg][k]));
        }
    }
    if (QUANT) {
      QParams qp[SEGS];
      bool near_edge = false;
#pragma unroll
      for (int sg = 0; sg < SEGS; ++sg) {
        qp[sg] = quant_params(w[sg], gt, asym, inv_top, top);
        near_edge |= qp[sg].near_edge;
        held_sz[sg] = qp[sg].sz;
      }
      if (YK == Y_F32) {  // the rows are stored as they are: clamp copies
#pragma unroll
        for (int sg = 0; sg < SEGS; ++sg) {
          float c[E];
#pragma unroll
          for (int e = 0; e < E; ++e) c[e] = w[sg][e];
          quant_clamp(c, qp[sg]);
          held_c[sg] = quant_pack(c, qp[sg], bits, asym);
        }
      } else {  // one wave-uniform test for every segment, the clamp in place
        // (asymmetric groups put an extreme past the test's margin in about
        // half the cases, so a wave of them always clamps)
        if (asym || __builtin_amdgcn_ballot_w64(near_edge) != 0) {
#pragma unroll
          for (int sg = 0; sg < SEGS; ++sg) quant_clamp(w[sg], qp[sg]);
        }
#pragma unroll
        for (int sg = 0; sg < SEGS; ++sg) held_c[sg] = quant_pack(w[sg], qp[sg], bits, asym);
      }
    }
  };

  // One row group through the whole path, from prefetch slot d (a
  // compile-time index once the callers' loops are unrolled).
  auto slot = [&](const int64_t grp, const int d) __attribute__((always_inline)) {
    // The previous group's rows come out of LDS first: their read latency is
    // covered by this group's unpacking and first register phase, and their
    // finishing work (quantization above all) interleaves with that phase.
    // (On the first pass this reads whatever the buffer holds; its stores
    // fall in empty ranges.)
    float w[SEGS][E];
    read_final(w);
    float v[SEGS][E];
#pragma unroll
    for (int sg = 0; sg < SEGS; ++sg) {
      if (XBF16) {
#pragma unroll
        for (int c = 0; c < RAW; ++c) {
          const uint32_t u[4] = {cur[d][sg][c].x, cur[d][sg][c].y, cur[d][sg][c].z, cur[d][sg][c].w};
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            v[sg][8 * c + 2 * k] = bf16_lo(u[k]);
            v[sg][8 * c + 2 * k + 1] = bf16_hi(u[k]);
          }
        }
      } else {
#pragma unroll
        for (int c = 0; c < RAW; ++c) {
          v[sg][4 * c] = __uint_as_float(cur[d][sg][c].x);
          v[sg][4 * c + 1] = __uint_as_float(cur[d][sg][c].y);
          v[sg][4 * c + 2] = __uint_as_float(cur[d][sg][c].z);
          v[sg][4 * c + 3] = __uint_as_float(cur[d][sg][c].w);
        }
      }
    }
    // Slot d is free once unpacked, and its refill should reuse its
    // registers.  Pinning the unpacked values here (an empty asm that the
    // load cannot cross) keeps the refill from being issued while the old
    // contents are still live, which would cost a register copy, and so a
    // wait for the refill, at the loop latch.
#pragma unroll
    for (int sg = 0; sg < SEGS; ++sg)
#pragma unroll
      for (int e = 0; e < E; ++e) asm volatile("" : "+v"(v[sg][e])::"memory");
    load(grp + PD * G, d);  // past the end: an empty range, no traffic
    finish(w);
    if (FAST) {
      // Phase A per segment, its rows written for the transpose (the LDS
      // traffic of one segment overlaps the arithmetic of the next); the
      // previous group's stores once the transpose's barrier is passed;
      // phase B per segment, written back in layout A for the next slot.
#pragma unroll
      for (int sg = 0; sg < SEGS; ++sg) {
        phase_a(v[sg]);
        if (S::TWO) put_a(abuf + sg * SEGW2, v[sg]);
        if (SEGS > 1) __builtin_amdgcn_sched_barrier(0);
      }
      if (S::TWO) {
        sync2();
        flush(w);
#pragma unroll
        for (int sg = 0; sg < SEGS; ++sg) get_b(abuf + sg * SEGW2, v[sg]);
        if (S::LOCAL2) wave_lds_sync();
#pragma unroll
        for (int sg = 0; sg < SEGS; ++sg) {
          phase_b(v[sg]);
          put_b(bbuf + sg * SEGW2, v[sg]);
          if (SEGS > 1) __builtin_amdgcn_sched_barrier(0);
        }
        sync2();
      } else {
        flush(w);
#pragma unroll
        for (int sg = 0; sg < SEGS; ++sg)
#pragma unroll
          for (int e = 0; e < E; ++e) fin[sg][e] = v[sg][e];
      }
      held_grp = grp;
      return;
    }
    // Phase k: [sync for transpose k] -> read every segment -> per segment:
    // rotate, then write it for transpose k+1.  Segment by segment (kept in
    // that order by scheduling barriers), the LDS traffic of one segment
    // overlaps the arithmetic of the next.  The read after the last
    // transpose is the next slot's.
    int gidx = 0;  // workgroup transposes so far in this row (compile-time after unrolling)
#pragma unroll
    for (int k = 0; k <= NPH; ++k) {
      const bool local_in = k > 0 && S::local_transpose(k);
      float* const buf_in = local_in ? lbuf : ((gidx & 1) ? gbuf1 : gbuf0);
      if (k > 0) {
        if (local_in) wave_lds_sync();
        else __syncthreads();
        if (k == NPH) break;
        const int b = phase_base(k, L, LOGE);
#pragma unroll
        for (int sg = 0; sg < SEGS; ++sg)
          lds_get1<LOGE, SEGW>(buf_in + sg * SEGW, v[sg], t, b, S::id_transpose(k));
        if (local_in) wave_lds_sync();
        else ++gidx;
      }
      if (k == 1) flush(w);  // the previous group's outputs, now complete
      const int b = phase_base(k, L, LOGE);
      const int s_end = ((k + 1) * LOGE < L) ? (k + 1) * LOGE : L;
      const bool local_out = S::local_transpose(k + 1);
      float* const buf_out = local_out ? lbuf : ((gidx & 1) ? gbuf1 : gbuf0);
#pragma unroll
      for (int sg = 0; sg < SEGS; ++sg) {
#pragma unroll
        for (int s = k * LOGE; s < s_end; ++s) {
          const int q = s - b;
#pragma unroll
          for (int j = 0; j < E / 2; ++j) {
            const int lo = pair_lo(j, q), hi = lo | (1 << q);
            if (s < L - 1) rotate<FAST>(v[sg][lo], v[sg][hi], C.c0[s][j], C.c1[s][j]);
            else last2x2(v[sg][lo], v[sg][hi], C.last[j]);
          }
        }
        lds_put1<LOGE, SEGW>(buf_out + sg * SEGW, v[sg], t, b, S::id_transpose(k + 1));
        if (SEGS > 1) __builtin_amdgcn_sched_barrier(0);
      }
    }
    held_grp = grp;
  };

  // Row groups g = blockIdx.x + i * gridDim.x, in passes of PD groups so
  // that prefetch slot d = i mod PD is a compile-time register index.
  // The prologue issues the same memory operations, in the same order, as a
  // pass of the main loop (its stores fall in empty ranges and are dropped).
  // The compiler's wait counts at the loop head merge the prologue with the
  // latch; with matching sequences, slot d waits for its own load alone.
  float zero[SEGS][E];
#pragma unroll
  for (int sg = 0; sg < SEGS; ++sg)
#pragma unroll
    for (int e = 0; e < E; ++e) zero[sg][e] = 0.f;
#pragma unroll
  for (int d = 0; d < PD; ++d) {
    if (!PRE) load(blockIdx.x + d * G, d);
    asm volatile("" ::: "memory");
    flush(zero);
    asm volatile("" ::: "memory");
  }
  // Main loop: full passes only, so its body has no branch around memory
  // operations (a conditional slot would make the compiler wait for the
  // most recent load at every slot).
  int64_t g0 = blockIdx.x;
  constexpr int D0 = CHECK ? 1 % PD : 0;  // prefetch slot of the loop's first group
  bool usable = true;
  if (CHECK) {
    // The grid never exceeds the number of groups: every block has this one.
    slot(g0, 0);
    g0 += G;
    bool nan_seen = false;
#pragma unroll
    for (int s = 0; s < L - 1; ++s)
#pragma unroll
      for (int j = 0; j < E / 2; ++j)  // bit test: the build assumes no NaN arithmetic
        nan_seen |= (__float_as_uint(C.c0[s][j]) & 0x7fffffffu) > 0x7f800000u;
    // One word per wave, one barrier.
    constexpr int NW = (S::NT + 63) / 64;
    __shared__ int nan_wave[NW];
    const int any = __builtin_amdgcn_ballot_w64(nan_seen) != 0;
    if ((threadIdx.x & 63) == 0) nan_wave[threadIdx.x >> 6] = any;
    __syncthreads();
    int seen = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) seen |= nan_wave[w];
    usable = __builtin_amdgcn_readfirstlane(seen) == 0;
    // An unusable form leaves the first group's results unstored: the
    // epilogue below then writes an empty range, so nothing reaches memory
    // before the fallback loop re-reads that group's input (which an
    // in-place call shares with the output).
    if (!usable) held_grp = -1;
  }
  const int64_t nrun = usable ? ngrp : 0;
  for (; g0 + (PD - 1) * G < nrun; g0 += PD * G) {
#pragma unroll
    for (int d = 0; d < PD; ++d) slot(g0 + d * G, (D0 + d) % PD);
  }
  // Tail: the block's last, partial pass.
#pragma unroll
  for (int d = 0; d < PD - 1; ++d)
    if (g0 + d * G < nrun) slot(g0 + d * G, (D0 + d) % PD);
  // Epilogue: the last group's outputs.
  float w[SEGS][E];
  read_final(w);
  finish(w);
  flush(w);
  return usable;
}

// One kernel per (input type, output kind, quantizer format): the host picks
// the variant, so each kernel holds just the two row loops below and the
// register allocator sees one loop nest at a time.
template <int LOGNB, int M, int RPT, bool XBF16, int YK, int QM, int XS = 1>
__global__ void __launch_bounds__((FwdShape<LOGNB, M, RPT>::NT))
fwd_kernel(FwdParams P) {
  using S = FwdShape<LOGNB, M, RPT>;
  constexpr int LOGE = S::LOGE, E = S::E, T = S::T, NB = S::NB, L = S::L;
  if constexpr (XS != 1) {
    // Halves of rows XS times longer (fp32 out): blockIdx.y picks the half,
    // its columns and its table (the half tables lie one after the other).
    const int h = blockIdx.y;
    P.x = static_cast<const char*>(P.x) + (size_t)h * NB * (XBF16 ? 2 : 4);
    P.y = static_cast<float*>(P.y) + (size_t)h * NB;
    P.tab = table_at(reinterpret_cast<const char*>(P.tab.cs) + (size_t)h * table_bytes(LOGNB), LOGNB);
  }
  extern __shared__ float4 lds_raw[];
  float* const lds = reinterpret_cast<float*>(lds_raw);
  const int tid = threadIdx.x;
  const int team = tid / T;
  const int t = tid - team * T;

  // Coefficients of every pair this thread rotates, resident for all rows,
  // in the scaled form unless the table marks it unusable (a NaN anywhere:
  // the workgroup covers every pair, so all workgroups decide alike).
  Coeffs<S> C;
  auto load_coeffs = [&](const float2* st, const float4* lst) {
#pragma unroll
    for (int s = 0; s < L; ++s) {
      const int b = phase_base(s / LOGE, L, LOGE);
#pragma unroll
      for (int j = 0; j < E / 2; ++j) {
        const int rank = pair_rank(lay<LOGE>(t, pair_lo(j, s - b), b), s);
        if (s < L - 1) {
          const float2 c = st[s * (NB / 2) + rank];
          C.c0[s][j] = c.x;
          C.c1[s][j] = c.y;
        } else {
          C.last[j] = lst[rank];
        }
      }
    }
  };
  // The scaled form's table is in thread order: 16-byte loads, each wave's
  // one contiguous run, issued in stage order.
  auto load_fast = [&](const float4* tab) {
    const auto rt = buffer_range(tab, (size_t)2 * (L + 1) * T * sizeof(float4));
#pragma unroll
    for (int s = 0; s < L - 1; ++s)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const uint4 q = buf_ld16s(rt, (uint32_t)(t * 16), (uint32_t)((2 * s + h) * T * 16));
        __builtin_amdgcn_sched_barrier(0);  // issue in stage order: phases wait for their own
        C.c0[s][2 * h] = __uint_as_float(q.x);
        C.c1[s][2 * h] = __uint_as_float(q.y);
        C.c0[s][2 * h + 1] = __uint_as_float(q.z);
        C.c1[s][2 * h + 1] = __uint_as_float(q.w);
      }
#pragma unroll
    for (int j = 0; j < E / 2; ++j) {
      const uint4 q = buf_ld16s(rt, (uint32_t)(t * 16), (uint32_t)((2 * (L - 1) + j) * T * 16));
      C.last[j] = make_float4(__uint_as_float(q.x), __uint_as_float(q.y), __uint_as_float(q.z),
                              __uint_as_float(q.w));
    }
  };
  static_assert(E == 8, "the thread-ordered table holds four pairs per stage and thread");
  // The first row groups' input is requested before anything else, so its
  // latency overlaps the coefficient loads and the form check.
  InRegs<S, XBF16> in;
#pragma unroll
  for (int d = 0; d < S::PD; ++d)
    load_group<S, XBF16, XS>(P, P.rows, (int64_t)blockIdx.x + (int64_t)d * gridDim.x, in, d, team,
                         fwd_elem_a(t, 0, S::PL));  // the scaled form's layout A
  load_fast(P.tab.fgt);
  __builtin_amdgcn_sched_barrier(0);
  // A 1 x 1 Kronecker factor scales the last stage's coefficients (a scalar
  // read once; no branch in the row loop).
  const float mix1 = (M == 1 && P.mix != nullptr)
                         ? __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(P.mix[0])))
                         : 1.0f;
  auto scale_last = [&]() {
    if (M == 1) {
#pragma unroll
      for (int j = 0; j < E / 2; ++j) {
        C.last[j].x *= mix1;
        C.last[j].y *= mix1;
        C.last[j].z *= mix1;
        C.last[j].w *= mix1;
      }
    }
  };
  scale_last();
  // The two forms run as consecutive loops, not as two arms of a branch:
  // the register allocator then never holds both coefficient sets at once.
  const bool usable = row_loop<S, XBF16, YK, QM, true, true, true, XS>(P, P.rows, lds, team, t, C, in);
  if (!usable) {
    // Three-shear form, with the general quantizer for every format.
    load_coeffs(P.tab.lift, P.tab.last);
    scale_last();
    row_loop<S, XBF16, YK, (QM == Q_NONE ? Q_NONE : Q_ANY), false, false, false, XS>(P, P.rows, lds, team, t,
                                                                                    C, in);
  }
}

// Host-side launch: pick the variant, size the persistent grid (cached per
// variant on first use).
template <int LOGNB, int M, int RPT, bool XBF16, int YK, int QM, int XS = 1>
hipError_t launch_fwd_variant(const FwdParams& p, hipStream_t stream) {
  using S = FwdShape<LOGNB, M, RPT>;
  auto kern = fwd_kernel<LOGNB, M, RPT, XBF16, YK, QM, XS>;
  int blocks_per_cu = 0, num_cu = 0;
  const hipError_t e =
      kernel_setup(reinterpret_cast<const void*>(kern), S::NT, S::LDS_BYTES, &blocks_per_cu, &num_cu);
  if (e != hipSuccess) return e;
  const int64_t ngrp = (p.rows + S::ROWS_PER_PASS - 1) / S::ROWS_PER_PASS;
  // XS halves run side by side (grid y): together they fill the device once
  const int64_t cap = ((int64_t)blocks_per_cu * num_cu + XS - 1) / XS;
  const int grid = (int)(ngrp < cap ? ngrp : cap);
  const dim3 g3((unsigned)grid, (unsigned)XS);
  const LaunchEvents ev = take_forward_events();
  if (ev.start != nullptr || ev.stop != nullptr)  // timestamps of this dispatch itself
    hipExtLaunchKernelGGL(kern, g3, dim3(S::NT), S::LDS_BYTES, stream, ev.start, ev.stop, 0u, p);
  else
    hipLaunchKernelGGL(kern, g3, dim3(S::NT), S::LDS_BYTES, stream, p);
  return hipGetLastError();
}

template <int LOGNB, int M, int RPT, bool XBF16>
hipError_t launch_fwd_inst(const FwdParams& p, hipStream_t stream) {
  using S = FwdShape<LOGNB, M, RPT>;
  const bool quant = p.codes != nullptr;
  // The fixed formats need a group of 128 to span whole 16-lane rows.
  const bool g128 = quant && p.group == 128 && S::T >= 16;
  const bool s4 = g128 && p.bits == 4 && p.asym == 0;
  const bool a2 = g128 && p.bits == 2 && p.asym != 0;
  if (p.y_kind == Y_BF16) {
    if (!quant) return launch_fwd_variant<LOGNB, M, RPT, XBF16, Y_BF16, Q_NONE>(p, stream);
    if (s4) return launch_fwd_variant<LOGNB, M, RPT, XBF16, Y_BF16, Q_S4G128>(p, stream);
    if (a2) return launch_fwd_variant<LOGNB, M, RPT, XBF16, Y_BF16, Q_A2G128>(p, stream);
    return launch_fwd_variant<LOGNB, M, RPT, XBF16, Y_BF16, Q_ANY>(p, stream);
  }
  if (p.y_kind == Y_NONE) {
    if (s4) return launch_fwd_variant<LOGNB, M, RPT, XBF16, Y_NONE, Q_S4G128>(p, stream);
    if (a2) return launch_fwd_variant<LOGNB, M, RPT, XBF16, Y_NONE, Q_A2G128>(p, stream);
    return launch_fwd_variant<LOGNB, M, RPT, XBF16, Y_NONE, Q_ANY>(p, stream);
  }
  if (!quant) return launch_fwd_variant<LOGNB, M, RPT, XBF16, Y_F32, Q_NONE>(p, stream);
  return launch_fwd_variant<LOGNB, M, RPT, XBF16, Y_F32, Q_ANY>(p, stream);
}

}  // namespace bfly
