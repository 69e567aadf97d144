// Forward butterfly (plain and Kronecker composite) fused with per-group
// round-to-nearest quantization.  Included by the instantiation units.
//
// Per row of n = M * NB elements (M = 1: plain butterfly of length NB):
//   load (bf16 or fp32, 16-byte vectors) -> L = log2 NB Givens stages on each
//   of the M segments -> [M > 1: mix the segments with the M x M factor,
//   column by column] -> store y (bf16 / fp32 / none) -> group max/min ->
//   fp16 scale (and zero) -> codes, packed, stored.
//
// The (cos, sin) of every pair a thread rotates stay in its VGPRs for all
// the rows it processes (L * E/2 pairs per thread), so after the prologue
// the only HBM traffic is the rows themselves.  Stages whose pair bit is in
// the thread's register bits need no data movement; between register
// phases the row is transposed through LDS (double-buffered, one barrier per
// transpose).  The grid is persistent: each workgroup walks row groups with
// stride gridDim.x and prefetches the next group's input while computing.
#pragma once

#include "bfly_common.h"

namespace bfly {

template <int LOGNB, int M>
struct FwdShape {
  static constexpr int LOGE = 3;
  static constexpr int NB = 1 << LOGNB;
  static constexpr int E = 1 << LOGE;
  static constexpr int T = NB >> LOGE;             // threads per row
  static constexpr int N = M * NB;                 // row length
  static constexpr int R_THREADS = (256 / T) > 0 ? (256 / T) : 1;
  static constexpr int SEGW = lds_words(NB);     // padded LDS words per segment
  static constexpr int R_LDS = (8192 / N) > 0 ? (8192 / N) : 1;
  static constexpr int R = R_THREADS < R_LDS ? R_THREADS : R_LDS;  // rows per pass
  static constexpr int NT = T * R;                 // threads per workgroup
  static constexpr int L = LOGNB;
  static constexpr int NPH = (L + LOGE - 1) / LOGE;  // register phases
  static constexpr size_t LDS_BYTES = 2ull * R * M * SEGW * sizeof(float);
};

__device__ __forceinline__ void givens(float& a, float& b, float c, float s) {
  const float na = fmaf(c, a, -(s * b));
  const float nb = fmaf(s, a, c * b);
  a = na;
  b = nb;
}

// Write registers in layout b to an LDS row buffer.
template <int LOGE, int M, int SEGW>
__device__ __forceinline__ void lds_put(float* buf, const float (&v)[M][1 << LOGE], int t, int b) {
  constexpr int E = 1 << LOGE;
  if (b == 0) {
#pragma unroll
    for (int a = 0; a < M; ++a)
#pragma unroll
      for (int c = 0; c < E / 4; ++c)
        *reinterpret_cast<float4*>(buf + a * SEGW + lds_addr(t * E + 4 * c)) =
            make_float4(v[a][4 * c], v[a][4 * c + 1], v[a][4 * c + 2], v[a][4 * c + 3]);
  } else {
#pragma unroll
    for (int a = 0; a < M; ++a)
#pragma unroll
      for (int e = 0; e < E; ++e) buf[a * SEGW + lds_addr(lay<LOGE>(t, e, b))] = v[a][e];
  }
}

template <int LOGE, int M, int SEGW>
__device__ __forceinline__ void lds_get(const float* buf, float (&v)[M][1 << LOGE], int t, int b) {
  constexpr int E = 1 << LOGE;
  if (b == 0) {
#pragma unroll
    for (int a = 0; a < M; ++a)
#pragma unroll
      for (int c = 0; c < E / 4; ++c) {
        const float4 q = *reinterpret_cast<const float4*>(buf + a * SEGW + lds_addr(t * E + 4 * c));
        v[a][4 * c] = q.x;
        v[a][4 * c + 1] = q.y;
        v[a][4 * c + 2] = q.z;
        v[a][4 * c + 3] = q.w;
      }
  } else {
#pragma unroll
    for (int a = 0; a < M; ++a)
#pragma unroll
      for (int e = 0; e < E; ++e) v[a][e] = buf[a * SEGW + lds_addr(lay<LOGE>(t, e, b))];
  }
}

// Quantize the E consecutive values of one thread (part of a group spread
// over group/E consecutive lanes) and store codes, scale and zero point.
// Every lane of the wave executes the reductions; only `store` lanes write.
template <int E>
__device__ __forceinline__ void quantize_store(const float (&v)[E], const FwdParams& P,
                                               int64_t row, int64_t n, int col, bool store) {
  const int gt = P.group / E;  // lanes per group (power of two, <= 64)
  const bool asym = P.asym != 0;
  const int bits = P.bits;
  float lo, hi;
  if (asym) {
    lo = v[0];
    hi = v[0];
#pragma unroll
    for (int e = 1; e < E; ++e) {
      lo = fminf(lo, v[e]);
      hi = fmaxf(hi, v[e]);
    }
    for (int msk = 1; msk < gt; msk <<= 1) {
      lo = fminf(lo, __shfl_xor(lo, msk));
      hi = fmaxf(hi, __shfl_xor(hi, msk));
    }
  } else {
    hi = fabsf(v[0]);
#pragma unroll
    for (int e = 1; e < E; ++e) hi = fmaxf(hi, fabsf(v[e]));
    for (int msk = 1; msk < gt; msk <<= 1) hi = fmaxf(hi, __shfl_xor(hi, msk));
    lo = 0.f;
  }
  const float top = asym ? (float)((1 << bits) - 1) : (float)((1 << (bits - 1)) - 1);
  float s_pre = asym ? (hi - lo) / top : hi / top;
  s_pre = fminf(s_pre, 65504.f);
  const _Float16 s16 = (_Float16)s_pre;
  const float sc = (float)s16;
  // codes: q = rne(clamp(y, qlo*sc, qhi*sc) * (1/sc)) (+ zero).  qlo*sc and
  // qhi*sc are exact in fp32, and clamping y first is the same as clamping
  // q afterwards.  fma(y, r, 1.5*2^23) rounds the exact product y*r once,
  // to an integer, ties to even; its low mantissa bits are q.
  float r = 0.f, clo = 0.f, chi = 0.f, z = 0.f;
  if (sc != 0.f) {
    r = 1.0f / sc;
    if (asym) {
      z = fminf(fmaxf(rintf(-lo / sc), 0.f), top);
      clo = -z * sc;
      chi = (top - z) * sc;
    } else {
      clo = -top * sc;
      chi = top * sc;
    }
  }
  const uint32_t zi = (uint32_t)z;
  const uint32_t mask = (1u << bits) - 1u;
  uint64_t packed = 0;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const float yc = fminf(fmaxf(v[e], clo), chi);
    const float f = fmaf(yc, r, 12582912.0f);
    const uint32_t q = (__float_as_uint(f) - 0x4B400000u + zi) & mask;
    packed |= (uint64_t)q << (bits * e);
  }
  if (store) {
    const int64_t rowbytes = n * bits / 8;
    uint8_t* cp = P.codes + row * rowbytes + (int64_t)col * bits / 8;
    const int nbytes = E * bits / 8;  // 2, 4 or 8
    if (nbytes == 8) *reinterpret_cast<uint2*>(cp) = make_uint2((uint32_t)packed, (uint32_t)(packed >> 32));
    else if (nbytes == 4) *reinterpret_cast<uint32_t*>(cp) = (uint32_t)packed;
    else *reinterpret_cast<uint16_t*>(cp) = (uint16_t)packed;
    if (((col / E) & (gt - 1)) == 0) {
      const int64_t gi = row * (n / P.group) + col / P.group;
      P.scales[gi] = __builtin_bit_cast(uint16_t, s16);
      if (asym) P.zeros[gi] = __builtin_bit_cast(uint16_t, (_Float16)z);
    }
  }
}

template <int LOGNB, int M, bool XBF16>
__global__ void __launch_bounds__((FwdShape<LOGNB, M>::NT))
fwd_kernel(FwdParams P) {
  using S = FwdShape<LOGNB, M>;
  constexpr int LOGE = S::LOGE, E = S::E, T = S::T, NB = S::NB, N = S::N, R = S::R;
  constexpr int SEGW = S::SEGW;
  constexpr int L = S::L, NPH = S::NPH;
  constexpr int RAW = XBF16 ? E / 8 : E / 4;  // 16-byte vectors per segment
  extern __shared__ float4 lds_raw[];
  float* lds = reinterpret_cast<float*>(lds_raw);

  const int tid = threadIdx.x;
  const int team = tid / T;
  const int t = tid - team * T;

  // (cos, sin) of every pair this thread rotates, resident for all rows.
  float cc[L][E / 2], ss[L][E / 2];
#pragma unroll
  for (int s = 0; s < L; ++s) {
    const int b = phase_base(s / LOGE, L, LOGE);
#pragma unroll
    for (int j = 0; j < E / 2; ++j) {
      const int ilo = lay<LOGE>(t, pair_lo(j, s - b), b);
      const float2 c = P.cs[s * (NB / 2) + pair_rank(ilo, s)];
      cc[s][j] = c.x;
      ss[s][j] = c.y;
    }
  }

  const int64_t rows = P.rows;
  const int64_t ngrp = (rows + R - 1) / R;
  const char* xb = reinterpret_cast<const char*>(P.x);
  constexpr int ESZ = XBF16 ? 2 : 4;

  // Input registers of the current row group; refilled with the next
  // group's row as soon as they have been unpacked (zeros past the end).
  uint4 cur[M][RAW];
  auto load = [&](int64_t grp, uint4 (&dst)[M][RAW]) {
    const int64_t row = grp * R + team;
    const bool ok = row < rows;
#pragma unroll
    for (int a = 0; a < M; ++a) {
      const uint4* src = reinterpret_cast<const uint4*>(
          xb + (((ok ? row : 0) * N + a * NB + (int64_t)t * E) * ESZ));
#pragma unroll
      for (int c = 0; c < RAW; ++c) dst[a][c] = ok ? src[c] : make_uint4(0u, 0u, 0u, 0u);
    }
  };

  int64_t grp = blockIdx.x;
  if (grp < ngrp) load(grp, cur);
  int bufsel = 0;
  for (; grp < ngrp; grp += gridDim.x) {
    const int64_t gnext = grp + gridDim.x;
    const int64_t row = grp * R + team;
    const bool valid = row < rows;

    float v[M][E];
#pragma unroll
    for (int a = 0; a < M; ++a) {
      if (XBF16) {
#pragma unroll
        for (int c = 0; c < RAW; ++c) {
          const uint32_t w[4] = {cur[a][c].x, cur[a][c].y, cur[a][c].z, cur[a][c].w};
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            v[a][8 * c + 2 * k] = bf16_lo(w[k]);
            v[a][8 * c + 2 * k + 1] = bf16_hi(w[k]);
          }
        }
      } else {
#pragma unroll
        for (int c = 0; c < RAW; ++c) {
          v[a][4 * c] = __uint_as_float(cur[a][c].x);
          v[a][4 * c + 1] = __uint_as_float(cur[a][c].y);
          v[a][4 * c + 2] = __uint_as_float(cur[a][c].z);
          v[a][4 * c + 3] = __uint_as_float(cur[a][c].w);
        }
      }
    }

    if (gnext < ngrp) load(gnext, cur);

#pragma unroll
    for (int k = 0; k < NPH; ++k) {
      const int b = phase_base(k, L, LOGE);
      if (k > 0) {
        float* buf = lds + (size_t)(bufsel * R + team) * (M * SEGW);
        lds_put<LOGE, M, SEGW>(buf, v, t, phase_base(k - 1, L, LOGE));
        __syncthreads();
        lds_get<LOGE, M, SEGW>(buf, v, t, b);
        bufsel ^= 1;
      }
      const int s_end = ((k + 1) * LOGE < L) ? (k + 1) * LOGE : L;
#pragma unroll
      for (int s = k * LOGE; s < s_end; ++s) {
        const int q = s - b;
#pragma unroll
        for (int j = 0; j < E / 2; ++j) {
          const int lo = pair_lo(j, q), hi = lo | (1 << q);
#pragma unroll
          for (int a = 0; a < M; ++a) givens(v[a][lo], v[a][hi], cc[s][j], ss[s][j]);
        }
      }
    }
    {  // back to the load/store layout
      float* buf = lds + (size_t)(bufsel * R + team) * (M * SEGW);
      lds_put<LOGE, M, SEGW>(buf, v, t, phase_base(NPH - 1, L, LOGE));
      __syncthreads();
      lds_get<LOGE, M, SEGW>(buf, v, t, 0);
      bufsel ^= 1;
    }

    if (M > 1 || P.mix != nullptr) {  // Kronecker mix across segments, column by column
#pragma unroll
      for (int e = 0; e < E; ++e) {
        float w[M];
#pragma unroll
        for (int a = 0; a < M; ++a) {
          float acc = P.mix[a * M] * v[0][e];
#pragma unroll
          for (int a2 = 1; a2 < M; ++a2) acc = fmaf(P.mix[a * M + a2], v[a2][e], acc);
          w[a] = acc;
        }
#pragma unroll
        for (int a = 0; a < M; ++a) v[a][e] = w[a];
      }
    }

    if (valid && P.y_kind != Y_NONE) {
#pragma unroll
      for (int a = 0; a < M; ++a) {
        const int64_t off = row * N + a * NB + (int64_t)t * E;
        if (P.y_kind == Y_BF16) {
          uint4* dst = reinterpret_cast<uint4*>(reinterpret_cast<uint16_t*>(P.y) + off);
#pragma unroll
          for (int c = 0; c < E / 8; ++c)
            dst[c] = make_uint4(pack_bf16(v[a][8 * c], v[a][8 * c + 1]),
                                pack_bf16(v[a][8 * c + 2], v[a][8 * c + 3]),
                                pack_bf16(v[a][8 * c + 4], v[a][8 * c + 5]),
                                pack_bf16(v[a][8 * c + 6], v[a][8 * c + 7]));
        } else {
          float4* dst = reinterpret_cast<float4*>(reinterpret_cast<float*>(P.y) + off);
#pragma unroll
          for (int c = 0; c < E / 4; ++c)
            dst[c] = make_float4(v[a][4 * c], v[a][4 * c + 1], v[a][4 * c + 2], v[a][4 * c + 3]);
        }
      }
    }
    if (P.codes != nullptr) {
#pragma unroll
      for (int a = 0; a < M; ++a) quantize_store<E>(v[a], P, row, N, a * NB + t * E, valid);
    }
  }
}

// Host-side launch of one instantiation.
template <int LOGNB, int M, bool XBF16>
hipError_t launch_fwd_inst(const FwdParams& p, hipStream_t stream) {
  using S = FwdShape<LOGNB, M>;
  auto kern = fwd_kernel<LOGNB, M, XBF16>;
  static int blocks_per_cu = -1;
  static int num_cu = 0;
  if (blocks_per_cu < 0) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    e = allow_lds(reinterpret_cast<const void*>(kern), S::LDS_BYTES);
    if (e != hipSuccess) return e;
    e = hipDeviceGetAttribute(&num_cu, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    int bpc = 0;
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&bpc, kern, S::NT, S::LDS_BYTES);
    if (e != hipSuccess) return e;
    blocks_per_cu = bpc > 0 ? bpc : 1;
  }
  const int64_t ngrp = (p.rows + S::R - 1) / S::R;
  const int64_t cap = (int64_t)blocks_per_cu * num_cu;
  const int grid = (int)(ngrp < cap ? ngrp : cap);
  hipLaunchKernelGGL(kern, dim3(grid), dim3(S::NT), S::LDS_BYTES, stream, p);
  return hipGetLastError();
}

}  // namespace bfly
