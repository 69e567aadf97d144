// Backward of the butterfly for learning the angles, fp32, plus the angle
// preparation kernel.
//
// Pass 1, per row (team of T threads, E elements each, the three-shear
// coefficients resident in VGPRs as in the forward):
//   v <- x (load/store layout), forward phases -> v = Q x in the last
//   phase's layout, y stored from there; g <- dL/dY loaded directly in that
//   layout; then the stages in reverse: for each pair (lo, hi) of stage s
//   with stage output v and output gradient g,
//       acc[s][pair] += g_hi v_lo - g_lo v_hi,
//   then v <- B_s^T v (undoing the stage) and g <- B_s^T g.  After stage 0,
//   g = Q^T dL/dY = dL/dX in the load/store layout.  Each thread keeps one
//   fp32 accumulator per pair it owns across all rows of its workgroup and
//   writes them to the workgroup's slot of the partials buffer at the end.
//   Stages 0..L-2 run as three shears on sign-carrying values (the forward
//   table's three-shear form); their inverse, which is also their transpose,
//   is the same three shears with negated coefficients, for v and for g
//   alike, since g carries the same signs as v.  The accumulated term then
//   carries the product of the pair's two signs, which the table records
//   and which multiplies the accumulator when it is written.  The last stage
//   is the 2x2 matrix that maps signed values to true ones; its inverse is
//   its transpose.
// Pass 2: dtheta[k] = sum over slots of partials[slot][k] in fp64, in an
// order fixed by the slot count alone -- the result is bit-identical from
// run to run and independent of the device (the slot count depends only on
// rows and n).
#include "bfly_calib.h"
#include "bfly_common.h"

namespace bfly {

template <int LOGN>
struct BwdShape {
  static constexpr int LOGE = 3;
  static constexpr int E = 1 << LOGE;
  static constexpr int N = 1 << LOGN;
  static constexpr int T = N >> LOGE;
  static constexpr int LOGT = LOGN - LOGE;
  static constexpr int R = (256 / T) > 0 ? (256 / T) : 1;
  static constexpr int NT = T * R;
  static constexpr int L = LOGN;
  static constexpr int NPH = (L + LOGE - 1) / LOGE;
  static constexpr int W = lds_words(N);  // padded LDS words per row
  // Transpose into phase k (k >= 1) from phase k - 1, and back.
  static constexpr bool local_transpose(int k) {
    return wave_local(phase_base(k - 1, L, LOGE), phase_base(k, L, LOGE), LOGT);
  }
  // Buffers per team: v and g for wave-local transposes; v for the forward
  // workgroup transposes; v and g for the reverse workgroup transposes.
  // Within a row the forward and the reverse workgroup transposes use
  // different buffers, so one barrier per transpose orders every reuse.
  static constexpr int global_transposes() {
    int c = 0;
    for (int k = 1; k < NPH; ++k) c += local_transpose(k) ? 0 : 1;
    return c;
  }
  static_assert(global_transposes() <= 1, "one buffer per direction assumes one workgroup transpose");
  static constexpr int NBUF = 5;
  static constexpr size_t LDS_BYTES = (size_t)NBUF * R * W * sizeof(float);
};

// CALIB: dL/dY is not read but formed from the recomputed Y (calib_grad,
// with each group's max |y| loaded like g and the log-bins in LDS), and dX
// is not stored -- the loss of one calibration step.
// KM > 0: the backward of a Kronecker composite (O kron B) with m = KM
// segments; each row of length N is segment a of row r of g, and its dL/dz
// = sum_b O[b][a] g[r][b N + .] is formed from the m segments of g as they
// are loaded (duidaima.com write-up, section "butterfly": the Kronecker
// composite; the mix is the transpose of the forward's).  A group's
// segments are loaded while the group before it finishes (issued right after
// that group's mix) and mixed after this group's forward recompute.
template <int LOGN, bool CALIB, int KM = 0>
__global__ void __launch_bounds__(BwdShape<LOGN>::NT) bwd_kernel(BwdParams P, CalibGradArgs C) {
  using S = BwdShape<LOGN>;
  constexpr int LOGE = S::LOGE, E = S::E, T = S::T, N = S::N, R = S::R, L = S::L;
  constexpr int NPH = S::NPH, W = S::W;
  constexpr int BL = phase_base(NPH - 1, L, LOGE);  // layout of the last phase
  extern __shared__ float4 lds_raw[];
  float* const lds = reinterpret_cast<float*>(lds_raw);

  const int tid = threadIdx.x;
  const int team = tid / T;
  const int t = tid - team * T;
  float* const lbuf_v = lds + (0 * R + team) * W;
  float* const lbuf_g = lds + (1 * R + team) * W;
  float* const fbuf_v = lds + (2 * R + team) * W;
  float* const rbuf_v = lds + (3 * R + team) * W;
  float* const rbuf_g = lds + (4 * R + team) * W;

  float pp[L - 1][E / 2], uu[L - 1][E / 2], acc[L][E / 2];
  float4 lastc[E / 2];
#pragma unroll
  for (int s = 0; s < L; ++s) {
    const int b = phase_base(s / LOGE, L, LOGE);
#pragma unroll
    for (int j = 0; j < E / 2; ++j) {
      const int rank = pair_rank(lay<LOGE>(t, pair_lo(j, s - b), b), s);
      if (s < L - 1) {
        const float2 c = P.tab.lift[s * (N / 2) + rank];
        pp[s][j] = c.x;
        uu[s][j] = c.y;
      } else {
        lastc[j] = P.tab.last[rank];
      }
      acc[s][j] = 0.f;
    }
  }

  // Memory through buffer resources whose range is exactly the row group's
  // valid rows (R rows, one per team; empty past the last row: loads give
  // zeros, which add nothing to the angle gradients, and stores are
  // dropped), so no memory operation is under a branch.  Base and size are
  // uniform (scalar registers) and each thread adds its team's row to its
  // offsets: a resource built per team would not be provably uniform and
  // would cost a waterfall loop around every access.  x and dX move in the
  // load layout (16-byte vectors), g and y in the last phase's layout
  // (4-byte words, 256 contiguous bytes per wave).
  const int64_t rows = P.rows;
  const int64_t ngrp = (rows + R - 1) / R;
  const uint32_t off0 = (uint32_t)(team * N + t * E) * 4;
  const uint32_t offl = (uint32_t)(team * N + lay<LOGE>(t, 0, BL)) * 4;
  auto group_range = [&](const float* base, int64_t grp) {
    return buffer_range32(base + grp * ((int64_t)R * N), (uint32_t)group_rows(rows, grp, R) * (uint32_t)(N * 4));
  };
  uint4 xc[E / 4];
  uint32_t gc[E];
  // CALIB: the group max of each element this thread holds in the last
  // phase's layout (element lay(t, 0, BL) + e 2^BL of its team's row)
  const int lg_group = CALIB ? 31 - __builtin_clz(C.group) : 0;
  const int ngr = CALIB ? N >> lg_group : 0;
  auto load = [&](int64_t grp) {
    const auto rx = group_range(P.x, grp);
#pragma unroll
    for (int c = 0; c < E / 4; ++c) xc[c] = buf_ld16(rx, off0 + 16 * c);
    if (CALIB) {
      const auto ra = buffer_range32(C.amax + grp * ((int64_t)R * ngr),
                                     (uint32_t)group_rows(rows, grp, R) * (uint32_t)(ngr * 4));
      const int el0 = lay<LOGE>(t, 0, BL);
#pragma unroll
      for (int e = 0; e < E; ++e)
        gc[e] = buf_ld4(ra, (uint32_t)(team * ngr + ((el0 + (e << BL)) >> lg_group)) * 4);
    } else if (KM == 0) {
      const auto rg = group_range(P.g, grp);
#pragma unroll
      for (int e = 0; e < E; ++e) gc[e] = buf_ld4(rg, offl + ((uint32_t)e << BL) * 4);
    }
  };
  // KM > 0: the m = KM segments of g for this team's segment row (row
  // r = sr / m, segment a = sr % m) and the column a of O, through a
  // resource over the rows the group's teams touch (from r0 = its first
  // segment row's row); segment rows past the end read as zeros.  A group's
  // segments are requested once the previous group's are mixed.
  uint32_t gm[KM > 0 ? KM : 1][E], om[KM > 0 ? KM : 1];
  // The group's first segment row is row r0, segment a0 (uniform), tracked
  // from group to group by adding the stride's quotient and remainder: one
  // 64-bit division before the loop instead of several per group.
  constexpr int km = KM > 0 ? KM : 1;
  const int64_t stride_sr = (int64_t)gridDim.x * R;
  const int64_t q_stride = stride_sr / km;
  const int r_stride = (int)(stride_sr - q_stride * km);
  int64_t r0 = ((int64_t)blockIdx.x * R) / km;
  int a0 = (int)((int64_t)blockIdx.x * R - r0 * km);
  auto load_gm = [&]() {
    if constexpr (KM > 0) {
      constexpr int m = km;
      const int64_t avail = rows / m - r0;  // whole rows from r0 on
      const uint32_t nr = (uint32_t)(avail <= 0 ? 0 : (avail < R + 1 ? avail : R + 1));
      const auto rg = buffer_range32(P.g + r0 * ((int64_t)m * N), nr * (uint32_t)(m * N * 4));
      const auto ro = buffer_range32(P.mix, (uint32_t)(m * m * 4));
      const uint32_t at = (uint32_t)(a0 + team);  // < m + R
      const int rrel = (int)(at / (uint32_t)m), a = (int)(at - (uint32_t)rrel * (uint32_t)m);
      const uint32_t el = (uint32_t)lay<LOGE>(t, 0, BL);
      const uint32_t base = ((uint32_t)(rrel * m * N) + el) * 4u;
#pragma unroll
      for (int b = 0; b < KM; ++b) {
        om[b] = buf_ld4(ro, (uint32_t)(b * m + a) * 4u);  // O[b][a]
#pragma unroll
        for (int e = 0; e < E; ++e)
          gm[b][e] = buf_ld4(rg, base + (((uint32_t)(b * N) + ((uint32_t)e << BL)) * 4u));
      }
    }
  };
  __shared__ float lbs[CALIB ? CALIB_MAX_BINS : 1];
  if (CALIB) {
    if (tid < C.bins) lbs[tid] = C.lb[tid];
    __syncthreads();
  }
  const float qmax = CALIB ? (float)((1 << (C.bits - 1)) - 1) : 0.f;
  const float inv_qmax = CALIB ? 1.f / qmax : 0.f;

  load(blockIdx.x);
  load_gm();  // KM > 0: the first group's g segments
  for (int64_t grp = blockIdx.x; grp < ngrp; grp += gridDim.x) {
    float v[E], g[E];
#pragma unroll
    for (int c = 0; c < E / 4; ++c) {
      v[4 * c] = __uint_as_float(xc[c].x);
      v[4 * c + 1] = __uint_as_float(xc[c].y);
      v[4 * c + 2] = __uint_as_float(xc[c].z);
      v[4 * c + 3] = __uint_as_float(xc[c].w);
    }
#pragma unroll
    for (int e = 0; e < E; ++e) g[e] = KM > 0 ? 0.f : __uint_as_float(gc[e]);
    // the registers are free once copied: pin the copies so the refill is
    // issued after them and reuses the registers
#pragma unroll
    for (int e = 0; e < E; ++e) asm volatile("" : "+v"(v[e]), "+v"(g[e])::"memory");
    load(grp + gridDim.x);

    // forward: v = Q x, ending in the last phase's layout
#pragma unroll
    for (int k = 0; k < NPH; ++k) {
      const int b = phase_base(k, L, LOGE);
      if (k > 0) {
        const int bp = phase_base(k - 1, L, LOGE);
        if (S::local_transpose(k)) {
          lds_put1<LOGE, W>(lbuf_v, v, t, bp);
          wave_lds_sync();
          lds_get1<LOGE, W>(lbuf_v, v, t, b);
          wave_lds_sync();
        } else {
          const bool id = same_lane_bits(bp, b);
          lds_put1<LOGE, W>(fbuf_v, v, t, bp, id);
          __syncthreads();
          lds_get1<LOGE, W>(fbuf_v, v, t, b, id);
        }
      }
      const int s_end = ((k + 1) * LOGE < L) ? (k + 1) * LOGE : L;
#pragma unroll
      for (int s = k * LOGE; s < s_end; ++s) {
        const int q = s - b;
#pragma unroll
        for (int j = 0; j < E / 2; ++j) {
          const int lo = pair_lo(j, q), hi = lo | (1 << q);
          if (s < L - 1) shear3(v[lo], v[hi], pp[s][j], uu[s][j]);
          else last2x2(v[lo], v[hi], lastc[j]);
        }
      }
    }
    if (P.y != nullptr) {
      const auto ry = group_range(P.y, grp);
#pragma unroll
      for (int e = 0; e < E; ++e) buf_st4(ry, offl + ((uint32_t)e << BL) * 4, __float_as_uint(v[e]));
    }
    if (CALIB) {  // g held the group maxima: dL/dy from y (= v) and them
#pragma unroll
      for (int e = 0; e < E; ++e)
        g[e] = calib_grad(v[e], g[e], qmax, inv_qmax, C.bins, lbs, C.two_n, C.kl_scale);
    }
    if constexpr (KM > 0) {
      // dL/dz of segment a: the sum over b from 0, in the order of the
      // mixing kernel (the same fp32 value as its (O^T kron I) g pass)
#pragma unroll
      for (int b = 0; b < KM; ++b)
#pragma unroll
        for (int e = 0; e < E; ++e) g[e] = fmaf(__uint_as_float(om[b]), __uint_as_float(gm[b][e]), g[e]);
      // then the next group's segments into the same registers: they have
      // this group's reverse sweep and the next forward to arrive
      a0 += r_stride;
      r0 += q_stride;
      if (a0 >= km) {
        a0 -= km;
        ++r0;
      }
      load_gm();
    }

    // reverse sweep: for each stage from the last, accumulate the angle
    // gradient, then undo the stage on v and apply its transpose to g
#pragma unroll
    for (int k = NPH - 1; k >= 0; --k) {
      const int b = phase_base(k, L, LOGE);
      const int s_end = ((k + 1) * LOGE < L) ? (k + 1) * LOGE : L;
#pragma unroll
      for (int s = s_end - 1; s >= k * LOGE; --s) {
        const int q = s - b;
#pragma unroll
        for (int j = 0; j < E / 2; ++j) {
          const int lo = pair_lo(j, q), hi = lo | (1 << q);
          acc[s][j] = fmaf(g[hi], v[lo], acc[s][j]);
          acc[s][j] = fmaf(-g[lo], v[hi], acc[s][j]);
          if (s < L - 1) {
            shear3(v[lo], v[hi], -pp[s][j], -uu[s][j]);
            shear3(g[lo], g[hi], -pp[s][j], -uu[s][j]);
          } else {
            const float4 m = lastc[j];  // transpose of the last stage's matrix
            const float4 mt = make_float4(m.x, m.z, m.y, m.w);
            last2x2(v[lo], v[hi], mt);
            last2x2(g[lo], g[hi], mt);
          }
        }
      }
      if (k > 0) {
        const int bp = phase_base(k - 1, L, LOGE);
        if (S::local_transpose(k)) {
          lds_put1<LOGE, W>(lbuf_v, v, t, b);
          lds_put1<LOGE, W>(lbuf_g, g, t, b);
          wave_lds_sync();
          lds_get1<LOGE, W>(lbuf_v, v, t, bp);
          lds_get1<LOGE, W>(lbuf_g, g, t, bp);
          wave_lds_sync();
        } else {
          const bool id = same_lane_bits(b, bp);
          lds_put1<LOGE, W>(rbuf_v, v, t, b, id);
          lds_put1<LOGE, W>(rbuf_g, g, t, b, id);
          __syncthreads();
          lds_get1<LOGE, W>(rbuf_v, v, t, bp, id);
          lds_get1<LOGE, W>(rbuf_g, g, t, bp, id);
        }
      }
    }
    if (!CALIB) {
      const auto rd = group_range(P.dx, grp);
#pragma unroll
      for (int c = 0; c < E / 4; ++c)
        buf_st16(rd, off0 + 16 * c,
                 make_uint4(__float_as_uint(g[4 * c]), __float_as_uint(g[4 * c + 1]),
                            __float_as_uint(g[4 * c + 2]), __float_as_uint(g[4 * c + 3])));
    }
  }

  float* part = P.partials + ((int64_t)blockIdx.x * R + team) * (L * (N / 2));
#pragma unroll
  for (int s = 0; s < L; ++s) {
    const int b = phase_base(s / LOGE, L, LOGE);
#pragma unroll
    for (int j = 0; j < E / 2; ++j) {
      const int k = s * (N / 2) + pair_rank(lay<LOGE>(t, pair_lo(j, s - b), b), s);
      part[k] = s < L - 1 ? P.tab.eps[k] * acc[s][j] : acc[s][j];
    }
  }
}

// Pass 2.  A block covers 32 consecutive angles with 8 lanes each: lane q
// sums slots q, q + 8, q + 16, ... in that order (fp64), then lane 0 adds
// the eight sums in order q = 0 .. 7.  The order depends only on the slot
// count, so the result is bit-identical from run to run.  Each lane keeps
// four loads in flight: with one at a time the pass was latency-bound
// (1024 slots of 5120 angles, 21 MB: 39.5 us, now 14.4 us; 256 slots of
// 24576 angles: 15 us, now 7.5 us).  32 lanes per angle was no faster.
constexpr int RED_PARTS = 8, RED_COLS = 32;

__global__ void __launch_bounds__(RED_PARTS * RED_COLS)
reduce_partials_kernel(const float* __restrict__ partials, float* __restrict__ dtheta, int nslots,
                       int count) {
  __shared__ double part[RED_PARTS][RED_COLS];
  const int c = threadIdx.x % RED_COLS, q = threadIdx.x / RED_COLS;
  const int k = blockIdx.x * RED_COLS + c;
  double sum = 0.0;
  if (k < count) {
    const float* const col = partials + k;
    int sl = q;
    for (; sl + 3 * RED_PARTS < nslots; sl += 4 * RED_PARTS) {
      const float a0 = col[(int64_t)sl * count];
      const float a1 = col[(int64_t)(sl + RED_PARTS) * count];
      const float a2 = col[(int64_t)(sl + 2 * RED_PARTS) * count];
      const float a3 = col[(int64_t)(sl + 3 * RED_PARTS) * count];
      sum += (double)a0;
      sum += (double)a1;
      sum += (double)a2;
      sum += (double)a3;
    }
    for (; sl < nslots; sl += RED_PARTS) sum += (double)col[(int64_t)sl * count];
  }
  part[q][c] = sum;
  __syncthreads();
  if (q == 0 && k < count) {
    double tot = part[0][c];
#pragma unroll
    for (int r = 1; r < RED_PARTS; ++r) tot += part[r][c];
    dtheta[k] = (float)tot;
  }
}

// sin and cos, in fp64, of an fp32 angle.  Cody and Waite's additive
// reduction: k = nearest integer to a * 2/pi, r = a - k * pi/2 with pi/2 split
// as P1 + P2 + P3, where P1 has 30 significant bits, so that k * P1 is exact
// and (a fp32 argument having at most 24) a - k * P1 is exact too for
// |k| < 2^20; then the Taylor series of sin and cos on |r| <= pi/4, whose
// first omitted terms are below 1e-19.  Angles of magnitude 1e6 and beyond
// (or not finite) take the library routine.
__device__ __forceinline__ void sincos_of_float(float a, double& sn, double& cn) {
  const double x = (double)a;
  if (!(fabs(x) < 1.0e6)) {
    sincos(x, &sn, &cn);
    return;
  }
  const double P1 = 1.5707963276654482;       // 0x1.921fb548p+0
  const double P2 = -8.705515695504166e-10;
  const double P3 = 1.6446256936324258e-26;
  const double k = rint(x * 0.6366197723675814);  // 2 / pi
  const double r = ((x - k * P1) - k * P2) - k * P3;
  const double r2 = r * r;
  // Horner in r^2 with the coefficients (-1)^m / (2m+1)! and (-1)^m / (2m)!
  double ps = 2.8114572543455206e-15;                     // 1/17!
  ps = fma(ps, r2, -7.647163731819816e-13);               // 1/15!
  ps = fma(ps, r2, 1.6059043836821613e-10);               // 1/13!
  ps = fma(ps, r2, -2.505210838544172e-08);               // 1/11!
  ps = fma(ps, r2, 2.7557319223985893e-06);               // 1/9!
  ps = fma(ps, r2, -0.0001984126984126984);               // 1/7!
  ps = fma(ps, r2, 0.008333333333333333);                 // 1/5!
  ps = fma(ps, r2, -0.16666666666666666);                 // 1/3!
  const double sr = fma(ps * r2, r, r);
  double pc = -1.5619206968586225e-16;                    // 1/18!
  pc = fma(pc, r2, 4.779477332387385e-14);                // 1/16!
  pc = fma(pc, r2, -1.1470745597729725e-11);              // 1/14!
  pc = fma(pc, r2, 2.08767569878681e-09);                 // 1/12!
  pc = fma(pc, r2, -2.755731922398589e-07);               // 1/10!
  pc = fma(pc, r2, 2.48015873015873e-05);                 // 1/8!
  pc = fma(pc, r2, -0.001388888888888889);                // 1/6!
  pc = fma(pc, r2, 0.041666666666666664);                 // 1/4!
  pc = fma(pc, r2, -0.5);                                 // 1/2!
  const double cr = fma(pc, r2, 1.0);
  // a = r + k pi/2: rotate (cos r, sin r) by k quarter turns
  const int q = (int)k & 3;
  sn = (q == 0) ? sr : (q == 1) ? cr : (q == 2) ? -sr : -cr;
  cn = (q == 0) ? cr : (q == 1) ? -sr : (q == 2) ? -cr : sr;
}

// One thread per (stage s, pair p).  Besides (cos t, sin t) it writes the
// coefficients of both forward forms of its pair.  Everything an element
// carries into stage s is a function of the angles of its pairs at the
// stages s' < s: the sign (three-shear form) is the parity of those angles
// exceeding pi/2 in magnitude (each such stage negates both of its
// elements), the scale (scaled form) is the product of their cosines.  So
// every entry is computed independently from the angles.
//
// Four consecutive lanes share one (s, p): lane q takes the earlier stages
// s2 = q, q + 4, q + 8, and the partial histories are combined across the
// four lanes (measured against 2, 8 and 16 lanes: 4 is fastest).  Then the
// pair's table entries are split over its lanes, one quotient and one store
// each, all lanes at once.
constexpr int PREP_LANES = 4;

// HAD: the Hadamard special case -- every angle pi/4 (cos = sin = 1/sqrt 2
// exactly, in fp64) and the +-1 diagonal D = diag((-1)^popcount(i)) on the
// input side, which every element's history starts with: sign parity (three-
// shear form) and scale d_i (scaled form).  The forward calls then compute
// H_n x, H_n the orthonormal Sylvester-ordered Walsh-Hadamard matrix
// (Q(pi/4) D = H_n).  theta is not read.
//
// tstride: floats from one stage's angles to the next (n/2 for a table of
// its own; the halves of a longer butterfly read strided slices of its
// angles).  par0: the sign every element's history starts with (HAD only;
// the upper half of a longer Hadamard starts negated).  gid: the lane's
// index among the table's PREP_LANES * L * n/2 lanes.
template <bool HAD>
__device__ __forceinline__ void prepare_entry(const float* __restrict__ theta,
                                              char* __restrict__ table, int logn, int tstride,
                                              int par0, int64_t gid) {
  const int half = 1 << (logn - 1);
  const int q = (int)(gid % PREP_LANES);
  const int64_t k = gid / PREP_LANES;
  // a pair's lanes leave together (the reductions below need all of them)
  if (k >= (int64_t)logn * half) return;
  const int s = (int)(k / half), p = (int)(k % half);
  const int i = ((p >> s) << (s + 1)) | (p & ((1 << s) - 1));  // lower element of the pair
  const int j = i | (1 << s);
  const double halfpi = 1.5707963267948966;
  const double r2 = 0.70710678118654752;  // cos and sin of pi/4
  const int64_t ka = (int64_t)s * tstride + p;  // this pair's angle
  const double t = HAD ? 0.78539816339744831 : (double)theta[ka];
  double sn, cn;
  if (HAD) sn = cn = r2;
  else sincos_of_float(theta[ka], sn, cn);
  const Table tab = table_at(table, logn);
  float2* cs = const_cast<float2*>(tab.cs);
  float* fgt = reinterpret_cast<float*>(const_cast<float4*>(tab.fgt));
  float2* lift = const_cast<float2*>(tab.lift);
  float4* last = const_cast<float4*>(tab.last);
  // Both elements' histories through stages s2 < s: the sign parity (three-
  // shear form) and the product of cosines (scaled form), this lane's share
  // first.  The angle loads are unconditional (a stage not before s reads
  // the pair's own angle, unused), so all of them are in flight together.
  constexpr int SMAX = 12;  // stages of the largest butterfly
  constexpr int PER = (SMAX + PREP_LANES - 1) / PREP_LANES;
  float ti[PER], tj[PER];
#pragma unroll
  for (int m = 0; m < PER; ++m) {
    const int s2 = q + PREP_LANES * m;
    ti[m] = HAD ? 0.f : theta[s2 < s ? (int64_t)s2 * tstride + pair_rank(i, s2) : ka];
    tj[m] = HAD ? 0.f : theta[s2 < s ? (int64_t)s2 * tstride + pair_rank(j, s2) : ka];
  }
  // the input side's diagonal (identity unless HAD), taken by one lane
  int par_i = (HAD && q == 0) ? ((__builtin_popcount(i) + par0) & 1) : 0;
  int par_j = (HAD && q == 0) ? ((__builtin_popcount(j) + par0) & 1) : 0;
  double sig_i = par_i ? -1.0 : 1.0, sig_j = par_j ? -1.0 : 1.0;
#pragma unroll
  for (int m = 0; m < PER; ++m) {
    if (HAD && q + PREP_LANES * m < s) {
      sig_i *= r2;
      sig_j *= r2;
    } else if (q + PREP_LANES * m < s) {
      // the same predicate (in fp64) as the flip decision below
      par_i ^= fabs((double)ti[m]) > halfpi;
      par_j ^= fabs((double)tj[m]) > halfpi;
      double si2, ci2, sj2, cj2;
      sincos_of_float(ti[m], si2, ci2);
      sincos_of_float(tj[m], sj2, cj2);
      sig_i *= ci2;
      sig_j *= cj2;
    }
  }
  // combine the lanes (products and parities are order independent up to
  // rounding; every lane ends with the same values, taken in the same order)
#pragma unroll
  for (int d = 1; d < PREP_LANES; d <<= 1) {
    const double oi = __shfl_xor(sig_i, d, PREP_LANES);
    const double oj = __shfl_xor(sig_j, d, PREP_LANES);
    sig_i = (q & d) ? oi * sig_i : sig_i * oi;
    sig_j = (q & d) ? oj * sig_j : sig_j * oj;
    par_i ^= __shfl_xor(par_i, d, PREP_LANES);
    par_j ^= __shfl_xor(par_j, d, PREP_LANES);
  }
  // Every lane holds the pair's histories now.  Lane q writes: 0 the
  // (cos, sin); 1 the three-shear entries (or the signed last stage); 2 and
  // 3 the scaled form at the lower and the upper element.  Each lane's one
  // quotient is taken by all lanes together.
  const bool flip = fabs(t) > halfpi;
  // phi = t or t -+ pi (|phi| <= pi/2): sin and cos of phi are +-sin t and
  // +-cos t, and tan(phi/2) = sin(phi) / (1 + cos(phi)), whose denominator
  // lies in [1, 2] -- one sin and cos serve every coefficient.
  const double sp = flip ? -sn : sn, cp = flip ? -cn : cn;
  const double eps = (par_i ^ par_j) ? -1.0 : 1.0;
  // scaled form: usable while every stored value stays within 2^64 of its
  // true value (|sigma| >= 2^-64 after this stage); beta = -tan t sig_j /
  // sig_i and gamma = tan t sig_i / sig_j, each as one quotient
  const double lim = 5.421010862427522e-20;  // 2^-64
  const bool ok = fabs(cn * sig_i) >= lim && fabs(cn * sig_j) >= lim;
  const double num = q == 1 ? sp : (q == 2 ? -sn * sig_j : (q == 3 ? sn * sig_i : 1.0));
  const double den = q == 1 ? 1.0 + cp : (q == 2 ? cn * sig_i : (q == 3 ? cn * sig_j : 1.0));
  const double quo = num / den;
  const float nan = __uint_as_float(0x7fc00000u);  // a quiet NaN, as bits
  if (q == 0) {
    cs[k] = make_float2((float)cn, (float)sn);
  } else if (s < logn - 1) {
    if (q == 1) {
      lift[k] = make_float2((float)(-eps * quo), (float)(eps * sp));
      const_cast<float*>(tab.eps)[k] = (float)eps;
    } else {
      fgt[fwd_coef_index(s, q == 2 ? i : j, logn)] = ok ? (float)quo : nan;
    }
  } else {
    const double si = par_i ? -1.0 : 1.0, sj = par_j ? -1.0 : 1.0;
    const float ki = (float)(cn * sig_i), kij = (float)(-sn * sig_j);
    const float kji = (float)(sn * sig_i), kj = (float)(cn * sig_j);
    if (q == 1) {
      last[p] = make_float4((float)(cn * si), (float)(-sn * sj), (float)(sn * si), (float)(cn * sj));
    } else if (fwd_plan(logn).SA < logn) {  // a register pair: its 2x2 matrix
      if (q == 2) *reinterpret_cast<float4*>(fgt + fwd_last_index(i, logn)) = make_float4(ki, kij, kji, kj);
    } else {  // lane-mapped: each element's (own, partner) weights
      if (q == 2) *reinterpret_cast<float2*>(fgt + fwd_last_index(i, logn)) = make_float2(ki, kij);
      else *reinterpret_cast<float2*>(fgt + fwd_last_index(j, logn)) = make_float2(kj, kji);
    }
  }
}

template <bool HAD>
__global__ void prepare_kernel(const float* __restrict__ theta, char* __restrict__ table, int logn) {
  prepare_entry<HAD>(theta, table, logn, 1 << (logn - 1), 0,
                     (int64_t)blockIdx.x * blockDim.x + threadIdx.x);
}

// (cos, sin) of one angle in fp64, rounded to fp32 (theta nullptr: pi/4).
__device__ __forceinline__ void last_stage_entry(const float* __restrict__ theta,
                                                 float2* __restrict__ cs, int i) {
  double sn = 0.70710678118654752, cn = 0.70710678118654752;  // pi/4 without angles
  if (theta != nullptr) sincos_of_float(theta[i], sn, cn);
  cs[i] = make_float2((float)cn, (float)sn);
}

// The whole table of n = 8192 in one launch: the lanes of the two half
// tables (length 4096, stage stride 4096 in theta, the upper half from
// column 2048; for H_8192 the upper half's diagonal starts with one more
// sign), then one lane per angle of stage 12.
template <bool HAD>
__global__ void prepare8k_kernel(const float* __restrict__ theta, char* __restrict__ table) {
  constexpr int64_t lanes = (int64_t)12 * 2048 * PREP_LANES;  // one half table
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid < 2 * lanes) {
    const int h = gid >= lanes ? 1 : 0;  // whole PREP_LANES groups per half
    prepare_entry<HAD>(HAD ? nullptr : theta + h * 2048, table + h * table_bytes(12), 12, 4096,
                       HAD ? h : 0, gid - h * lanes);
  } else if (gid < 2 * lanes + 4096) {
    last_stage_entry(HAD ? nullptr : theta + 12 * 4096,
                     reinterpret_cast<float2*>(table + 2 * table_bytes(12)), (int)(gid - 2 * lanes));
  }
}

hipError_t launch_prepare_8192(const float* theta, void* table, bool hadamard, hipStream_t s) {
  const int threads = 64;
  const int64_t count = (int64_t)2 * 12 * 2048 * PREP_LANES + 4096;
  const unsigned blocks = (unsigned)((count + threads - 1) / threads);
  if (hadamard)
    hipLaunchKernelGGL(prepare8k_kernel<true>, dim3(blocks), dim3(threads), 0, s, nullptr,
                       static_cast<char*>(table));
  else
    hipLaunchKernelGGL(prepare8k_kernel<false>, dim3(blocks), dim3(threads), 0, s, theta,
                       static_cast<char*>(table));
  return hipGetLastError();
}

hipError_t launch_prepare(const float* theta, void* table, int logn, hipStream_t s, bool hadamard) {
  const int threads = 64;  // small blocks spread the angles over every CU
  const int64_t count = ((int64_t)logn << (logn - 1)) * PREP_LANES;
  const int64_t blocks = (count + threads - 1) / threads;
  if (hadamard)
    hipLaunchKernelGGL(prepare_kernel<true>, dim3((unsigned)blocks), dim3(threads), 0, s, theta,
                       static_cast<char*>(table), logn);
  else
    hipLaunchKernelGGL(prepare_kernel<false>, dim3((unsigned)blocks), dim3(threads), 0, s, theta,
                       static_cast<char*>(table), logn);
  return hipGetLastError();
}

int backward_blocks(int64_t rows, int logn) {
  const int T = (1 << logn) >> 3;
  const int R = (256 / T) > 0 ? (256 / T) : 1;
  const int64_t ngrp = (rows + R - 1) / R;
  // one workgroup per CU at n = 4096 (512 threads), two of 256 threads
  // below; a constant of the shape, never of the device
  const int64_t cap = T >= 512 ? 256 : 512;
  return (int)(ngrp < cap ? (ngrp > 0 ? ngrp : 1) : cap);
}

template <int LOGN, bool CALIB = false, int KM = 0>
static hipError_t launch_bwd_inst(const BwdParams& p, float* dtheta, hipStream_t s,
                                  const CalibGradArgs& c = CalibGradArgs{}) {
  using S = BwdShape<LOGN>;
  const hipError_t lds_ok =
      kernel_setup(reinterpret_cast<const void*>(bwd_kernel<LOGN, CALIB, KM>), S::NT, S::LDS_BYTES,
                   nullptr, nullptr);
  if (lds_ok != hipSuccess) return lds_ok;
  if (p.nblk > 0) {
    hipLaunchKernelGGL((bwd_kernel<LOGN, CALIB, KM>), dim3(p.nblk), dim3(S::NT), S::LDS_BYTES, s, p, c);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int count = S::L * (S::N / 2);
  const int nslots = p.nblk * S::R;
  hipLaunchKernelGGL(reduce_partials_kernel, dim3((count + RED_COLS - 1) / RED_COLS),
                     dim3(RED_PARTS * RED_COLS), 0, s, p.partials, dtheta, nslots, count);
  return hipGetLastError();
}

hipError_t launch_backward_calib(const BwdParams& p, const CalibGradArgs& c, float* dtheta,
                                 hipStream_t s) {
  switch (p.logn) {
    case 6: return launch_bwd_inst<6, true>(p, dtheta, s, c);
    case 7: return launch_bwd_inst<7, true>(p, dtheta, s, c);
    case 8: return launch_bwd_inst<8, true>(p, dtheta, s, c);
    case 9: return launch_bwd_inst<9, true>(p, dtheta, s, c);
    case 10: return launch_bwd_inst<10, true>(p, dtheta, s, c);
    case 11: return launch_bwd_inst<11, true>(p, dtheta, s, c);
    case 12: return launch_bwd_inst<12, true>(p, dtheta, s, c);
    default: return hipErrorInvalidValue;
  }
}

template <int KM>
static hipError_t launch_bwd_kron_m(const BwdParams& p, float* dtheta, hipStream_t s) {
  switch (p.logn) {  // segment lengths of the Kronecker composites: 256 .. 4096
    case 8: return launch_bwd_inst<8, false, KM>(p, dtheta, s);
    case 9: return launch_bwd_inst<9, false, KM>(p, dtheta, s);
    case 10: return launch_bwd_inst<10, false, KM>(p, dtheta, s);
    case 11: return launch_bwd_inst<11, false, KM>(p, dtheta, s);
    case 12: return launch_bwd_inst<12, false, KM>(p, dtheta, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_backward_kron(const BwdParams& p, float* dtheta, hipStream_t s) {
  if (p.mix == nullptr) return hipErrorInvalidValue;
  static_assert(kKronBwdFusedM == 5, "one kernel per segment count 2 .. 5");
  switch (p.m) {  // the segment count is a compile-time constant of each kernel
    case 2: return launch_bwd_kron_m<2>(p, dtheta, s);
    case 3: return launch_bwd_kron_m<3>(p, dtheta, s);
    case 4: return launch_bwd_kron_m<4>(p, dtheta, s);
    case 5: return launch_bwd_kron_m<5>(p, dtheta, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_backward(const BwdParams& p, float* dtheta, hipStream_t s) {
  switch (p.logn) {
    case 6: return launch_bwd_inst<6>(p, dtheta, s);
    case 7: return launch_bwd_inst<7>(p, dtheta, s);
    case 8: return launch_bwd_inst<8>(p, dtheta, s);
    case 9: return launch_bwd_inst<9>(p, dtheta, s);
    case 10: return launch_bwd_inst<10>(p, dtheta, s);
    case 11: return launch_bwd_inst<11>(p, dtheta, s);
    case 12: return launch_bwd_inst<12>(p, dtheta, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace bfly
