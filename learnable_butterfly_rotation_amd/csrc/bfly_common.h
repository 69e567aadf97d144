// Device helpers shared by the forward and backward kernels: the register /
// LDS layouts of a row, the LDS swizzle, bf16 packing.
#pragma once

#include "bfly_internal.h"

namespace bfly {

// A row of NB = 2^LOGNB elements is owned by a team of T = NB / E threads,
// each holding E = 2^LOGE elements in registers.  In "phase" k the register
// index e of thread t carries the E index bits starting at bit b_k:
//     i = (t mod 2^b) | (e << b) | ((t >> b) << (b + LOGE)),
// so the Givens stages whose pair bit lies in [b, b + LOGE) are done entirely
// in registers.  Phase k performs stages [k LOGE, min((k+1) LOGE, L)) with
// b_k = min(k LOGE, L - LOGE); between phases the row goes through LDS.
// Layout b = 0 (E consecutive elements per thread) is the load/store layout.
template <int LOGE>
__device__ __forceinline__ int lay(int t, int e, int b) {
  return (t & ((1 << b) - 1)) | (e << b) | ((t >> b) << (b + LOGE));
}

__host__ __device__ constexpr int phase_base(int k, int L, int LOGE) {
  return (k * LOGE < L - LOGE) ? k * LOGE : L - LOGE;
}

// LDS word address of row element i: 4 pad words after every 32 and 16
// more after every 256.  The padding is linear in the index bits, so in
// every layout the address of register e is (thread part) + (constant for
// e) and needs one base register plus immediate offsets.  Every transpose
// access is conflict-free: layout b = 0 is accessed as aligned 16-byte
// vectors (8 lanes cover 32 distinct banks), every other layout as 4-byte
// words whose 32 consecutive lanes land in 32 distinct banks.
__host__ __device__ constexpr int lds_addr(int i) { return i + 4 * (i >> 5) + 16 * (i >> 8); }

// Words of LDS one padded segment of nb elements occupies.
__host__ __device__ constexpr int lds_words(int nb) { return nb + 4 * (nb >> 5) + 16 * (nb >> 8); }

// bf16 <-> fp32.  Widening is exact; narrowing rounds to nearest even.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
// Two values in one v_cvt_pk_bf16_f32 (round to nearest even).
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  const f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// Rank of the pair (i, i + 2^s) among the stage-s pairs ordered by i.
__device__ __forceinline__ int pair_rank(int i, int s) {
  return ((i >> (s + 1)) << s) | (i & ((1 << s) - 1));
}

// Register index of the lower element of pair j (0 <= j < E/2) when the
// pair bit is local bit q: insert a zero at bit q of j.
__device__ __forceinline__ int pair_lo(int j, int q) {
  return ((j >> q) << (q + 1)) | (j & ((1 << q) - 1));
}

// Buffer resources: a raw buffer over [base, base + bytes).  Accesses outside
// the range read zeros and drop writes in hardware, so row tails, row groups
// past the end and masked lanes need no branches around memory operations.
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
constexpr uint32_t kOutOfRange = 0xFFFFFFF0u;  // an offset beyond any range below

__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_range(const void* base, int64_t bytes) {
  const uint32_t n = bytes <= 0 ? 0u : (bytes >= (int64_t)kOutOfRange ? kOutOfRange : (uint32_t)bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)n, 0x00020000);
}
// The same for a size known to fit 32 bits.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_range32(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
// Rows of row group grp (groups of cap rows) that lie below rows; 0 for a
// negative group.  Written as 32-bit tests on the halves of the 64-bit
// values, which keeps uniform arguments on the scalar unit (it has no
// signed 64-bit compare).
__device__ __forceinline__ int group_rows(int64_t rows, int64_t grp, int cap) {
  const int64_t r = rows - grp * cap;
  const int r_hi = (int)(r >> 32), g_hi = (int)(grp >> 32);
  const uint32_t r_lo = (uint32_t)r;
  return (g_hi < 0 || r_hi < 0) ? 0 : (r_hi > 0 || r_lo >= (uint32_t)cap) ? cap : (int)r_lo;
}
// Cache policy of a buffer access: kNonTemporal sets the nt bit (streaming:
// the line is not kept for reuse), for data the kernel touches once.
constexpr int kCached = 0, kNonTemporal = 2;
template <int POLICY = kCached>
__device__ __forceinline__ uint4 buf_ld16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, POLICY);
  return make_uint4(v.x, v.y, v.z, v.w);
}
// With a uniform part in the instruction's scalar offset (no address VALU,
// no extra VGPR).  The hardware range check does not cover the scalar part:
// only for offsets known to lie inside the range.
__device__ __forceinline__ uint4 buf_ld16s(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, 0);
  return make_uint4(v.x, v.y, v.z, v.w);
}
template <int POLICY = kCached>
__device__ __forceinline__ void buf_st16(__amdgpu_buffer_rsrc_t r, uint32_t off, uint4 v) {
  const u32x4_t w = {v.x, v.y, v.z, v.w};
  __builtin_amdgcn_raw_buffer_store_b128(w, r, (int)off, 0, POLICY);
}
__device__ __forceinline__ uint32_t buf_ld4(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0);
}
template <int POLICY = kCached>
__device__ __forceinline__ void buf_st4(__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t v) {
  __builtin_amdgcn_raw_buffer_store_b32(v, r, (int)off, 0, POLICY);
}
template <int POLICY = kCached>
__device__ __forceinline__ void buf_st2(__amdgpu_buffer_rsrc_t r, uint32_t off, uint16_t v) {
  __builtin_amdgcn_raw_buffer_store_b16(v, r, (int)off, 0, POLICY);
}

// Allow a kernel more than the default 64 KiB of dynamic LDS (gfx950 has
// 160 KiB per CU); fails if the device cannot provide `bytes`.
inline hipError_t allow_lds(const void* kernel, size_t bytes) {
  if (bytes <= 65536) return hipSuccess;
  int dev = 0, maxb = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  e = hipDeviceGetAttribute(&maxb, hipDeviceAttributeMaxSharedMemoryPerBlock, dev);
  if (e != hipSuccess) return e;
  if ((size_t)maxb < bytes) return hipErrorInvalidConfiguration;
  return hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
}

// Whether the transpose from register layout b0 to b1 keeps every element
// inside its wavefront.  Thread bit j carries index bit j (j < b) or j + LOGE
// (j >= b); when each wave-index bit (thread bits 6 .. logt-1) carries the
// same index bit in both layouts, no data crosses a wave and a wave-level
// ordering suffices instead of a workgroup barrier.
__host__ __device__ constexpr bool wave_local(int b0, int b1, int logt) {
  for (int j = 6; j < logt; ++j)
    if ((j < b0) != (j < b1)) return false;
  return true;
}

__host__ __device__ constexpr int ilog2c(int v) { return v <= 1 ? 0 : 1 + ilog2c(v / 2); }

// Write / read registers in layout b to / from an LDS row buffer.  lds_addr
// is additive over disjoint index bits, so the address of register e is the
// thread's base for the layout plus a compile-time offset for e.
//
// Other addressings (`mode`), each additive over index bits as well:
//   LDS_ID    word = index, for transposes in which every lane keeps the same
//             low 6 index bits on both sides: each access of one register
//             covers 64 consecutive words (no bank conflicts), and registers
//             lie multiples of 64 words apart, so the compiler pairs them
//             into ds_read2st64 / ds_write2st64, twice the words per
//             instruction;
//   LDS_P512  4 pad words after every 32 within each block of 512, blocks
//             576 words apart, for the transpose from registers 512 elements
//             apart (n = 4096) back to 8 consecutive elements: the strided
//             side pairs into ds_write2st64 (576 = 9 * 64), the 16-byte side
//             stays conflict-free (8 lanes of a 16-byte access land on
//             distinct banks).
enum LdsMode : int { LDS_PAD = 0, LDS_ID = 1, LDS_P512 = 2 };
__host__ __device__ constexpr int lds_index(int i, int mode) {
  return mode == LDS_ID     ? i
         : mode == LDS_P512 ? (i >> 9) * 576 + (i & 511) + 4 * ((i >> 5) & 15)
                            : lds_addr(i);
}

template <int LOGE, int NSEG, int SEGW>
__device__ __forceinline__ void lds_put(float* buf, const float (&v)[NSEG][1 << LOGE], int t, int b,
                                        int id = LDS_PAD) {
  constexpr int E = 1 << LOGE;
  float* const base = buf + lds_index(lay<LOGE>(t, 0, b), id);
  if (b == 0) {
#pragma unroll
    for (int a = 0; a < NSEG; ++a)
#pragma unroll
      for (int c = 0; c < E / 4; ++c)
        *reinterpret_cast<float4*>(base + a * SEGW + lds_index(4 * c, id)) =
            make_float4(v[a][4 * c], v[a][4 * c + 1], v[a][4 * c + 2], v[a][4 * c + 3]);
  } else {
#pragma unroll
    for (int a = 0; a < NSEG; ++a)
#pragma unroll
      for (int e = 0; e < E; ++e) base[a * SEGW + lds_index(e << b, id)] = v[a][e];
  }
}

template <int LOGE, int NSEG, int SEGW>
__device__ __forceinline__ void lds_get(const float* buf, float (&v)[NSEG][1 << LOGE], int t, int b,
                                        int id = LDS_PAD) {
  constexpr int E = 1 << LOGE;
  const float* const base = buf + lds_index(lay<LOGE>(t, 0, b), id);
  if (b == 0) {
#pragma unroll
    for (int a = 0; a < NSEG; ++a)
#pragma unroll
      for (int c = 0; c < E / 4; ++c) {
        const float4 q = *reinterpret_cast<const float4*>(base + a * SEGW + lds_index(4 * c, id));
        v[a][4 * c] = q.x;
        v[a][4 * c + 1] = q.y;
        v[a][4 * c + 2] = q.z;
        v[a][4 * c + 3] = q.w;
      }
  } else {
#pragma unroll
    for (int a = 0; a < NSEG; ++a)
#pragma unroll
      for (int e = 0; e < E; ++e) v[a][e] = base[a * SEGW + lds_index(e << b, id)];
  }
}

template <int LOGE, int SEGW>
__device__ __forceinline__ void lds_put1(float* buf, const float (&v)[1 << LOGE], int t, int b,
                                         int id = LDS_PAD) {
  lds_put<LOGE, 1, SEGW>(buf, reinterpret_cast<const float (&)[1][1 << LOGE]>(v), t, b, id);
}
template <int LOGE, int SEGW>
__device__ __forceinline__ void lds_get1(const float* buf, float (&v)[1 << LOGE], int t, int b,
                                         int id = LDS_PAD) {
  lds_get<LOGE, 1, SEGW>(buf, reinterpret_cast<float (&)[1][1 << LOGE]>(v), t, b, id);
}

// Whether every lane keeps the same low 6 index bits in layouts b0 and b1
// (thread bit j < 6 carries index bit j when j < b, else j + LOGE).
__host__ __device__ constexpr bool same_lane_bits(int b0, int b1) {
  for (int j = 0; j < 6; ++j)
    if ((j < b0) != (j < b1)) return false;
  return true;
}

// Orders this wave's LDS writes before its later LDS reads.  The LDS
// executes one wave's instructions in issue order, so a read issued after a
// write sees it without waiting for the write to complete; only the
// compiler must be kept from moving the accesses across each other.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_wave_barrier();
  asm volatile("" ::: "memory");
}

// Givens rotation of (a, b) by phi, |phi| <= pi/2, as three shears:
// p = -tan(phi/2), u = sin(phi).  Three in-place FMAs, no temporaries.
__device__ __forceinline__ void shear3(float& a, float& b, float p, float u) {
  a = fmaf(p, b, a);
  b = fmaf(u, a, b);
  a = fmaf(p, b, a);
}

// The last stage: (a, b) <- (k.x a + k.y b, k.z a + k.w b).
__device__ __forceinline__ void last2x2(float& a, float& b, float4 k) {
  const float na = fmaf(k.x, a, k.y * b);
  const float nb = fmaf(k.z, a, k.w * b);
  a = na;
  b = nb;
}

}  // namespace bfly
