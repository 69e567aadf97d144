// Internal interface between the C-ABI layer (bfly_api.cpp) and the HIP
// kernels.  Not installed; callers use include/bfly.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace bfly {

// Output selector for the rotated rows.
enum YKind : int { Y_NONE = -1, Y_F32 = 0, Y_BF16 = 1 };

// The prepared coefficient table of a butterfly of length n = 2^L, in one
// device allocation (half = n/2 pairs per stage):
//   cs    float2 [L][half]    (cos t, sin t) of every angle (backward)
//   fgt   float4 [2(L+1)][n/8] the scaled form, in forward-thread order:
//                             row q of thread t holds what the forward
//                             kernel's thread t loads q-th, so that every
//                             load of a wave is one contiguous 1 KiB run:
//                             8 floats per stage s < L-1, 16 for the last
//                             one with the scales folded in (fwd_coef_index
//                             and fwd_last_index give the places).
//   lift  float2 [L-1][half]  (p, u): stages 0..L-2 as three shears
//   last  float4 [half]       the last stage with the tracked signs folded in
//
// Scaled form (the "fast Givens" rotation): every element carries a scale
// sigma (1 on input) and the kernel stores w = x / sigma.  A rotation by t of
// the pair (i, j) becomes two fused multiply-adds on the stored values,
//   w_i <- w_i + beta w_j,  w_j <- w_j + gamma w_i  (both from the old values)
// with beta = -tan t * sigma_j / sigma_i, gamma = tan t * sigma_i / sigma_j,
// after which both scales are multiplied by cos t.  The last stage maps the
// stored values to the true outputs with the 2x2 matrix
// (c sigma_i, -s sigma_j, s sigma_i, c sigma_j).  Scales are tracked in fp64
// when the table is prepared.  Stored magnitudes grow like 1 / |sigma| (for
// angles drawn uniformly, 1/|sigma| reaches ~2^31 at n = 4096); a pair
// whose scales would fall below 2^-64 has beta set to NaN, and a forward
// launch that sees any NaN uses the three-shear form instead.
//
// Three-shear form: x += p y; y += u x; x += p y is the Givens rotation by
// an angle phi with |phi| <= pi/2 (p = -tan(phi/2), u = sin phi).  A
// rotation by t with |t| > pi/2 equals minus the rotation by t -+ pi; the
// minus is not applied but tracked as a sign on both elements, and a
// rotation of sign-carrying elements is again a rotation (by +-t).  The last
// stage maps the sign-carrying values straight to the true outputs.
//   eps   float [L-1][half]   the product of the signs the pair's two
//                             elements carry in the three-shear form (the
//                             backward's angle gradients are accumulated on
//                             signed values and multiplied by it at the end)
struct Table {
  const float2* cs;
  const float4* fgt;
  const float2* lift;
  const float4* last;
  const float* eps;
};

__host__ __device__ constexpr size_t table_bytes(int logn) {
  const size_t half = (size_t)1 << (logn - 1);
  return half * 8 * (size_t)(3 * logn + 2) + half * 4 * (size_t)(logn - 1);
}

__host__ __device__ inline Table table_at(const void* base, int logn) {
  const size_t half = (size_t)1 << (logn - 1);
  const char* b = static_cast<const char*>(base);
  Table t;
  t.cs = reinterpret_cast<const float2*>(b);
  t.fgt = reinterpret_cast<const float4*>(b + half * 8 * logn);
  t.lift = reinterpret_cast<const float2*>(b + half * 8 * (2 * logn + 1));
  t.last = reinterpret_cast<const float4*>(b + half * 8 * (3 * logn));
  t.eps = reinterpret_cast<const float*>(b + half * 8 * (3 * logn + 2));
  return t;
}

// Forward layouts of the scaled form.  A row goes to a team of T = n/8
// threads holding 8 elements each, in at most two phases.  A phase rotates
// element bits that are either register bits (the thread's 8 elements) or
// lane bits that one DPP lane swap reaches: within 16-lane rows, xor masks
// 1 and 2 (quad permutes), 7 (half-row mirror) and 15 (row mirror).  The
// lane-mapped element bits c_0.. sit on lane bits 0..3 through the linear
// map lane = XOR of mask_j over the c_j set (dpp_mix), so a stage on c_j
// pairs lane l with l ^ mask_j, and c_0..c_{k-1} range over lanes 0..2^k-1.
//   phase A: stages 0..SA-1; register bits 0..2, lane-mapped bits 3..SA-1,
//            thread bits above DL on element bits SA..
//   phase B: stages SA..L-1; register bits L-3..L-1, lane-mapped bits
//            SA..L-4, the other thread bits on element bits 0..SA-1
// with DL = min(4, L-3) lane-mapped bits at most and SA = min(L, 3 + DL).
// Rows of up to 128 elements need one phase; the others, two transposes.
__host__ __device__ constexpr int dpp_mix(int c) {
  return ((c & 1) ? 1 : 0) ^ ((c & 2) ? 2 : 0) ^ ((c & 4) ? 7 : 0) ^ ((c & 8) ? 15 : 0);
}
__host__ __device__ constexpr int dpp_unmix(int l) {
  const int l0 = l & 1, l1 = (l >> 1) & 1, l2 = (l >> 2) & 1, l3 = (l >> 3) & 1;
  return (l0 ^ l2) | ((l1 ^ l2) << 1) | ((l2 ^ l3) << 2) | (l3 << 3);
}
struct FwdPlan {
  int L, DL, SA, DB;
};
__host__ __device__ constexpr FwdPlan fwd_plan(int L) {
  const int DL = L - 3 < 4 ? L - 3 : 4;
  const int SA = L < 3 + DL ? L : 3 + DL;
  const int DB = L - 3 - SA > 0 ? L - 3 - SA : 0;
  return FwdPlan{L, DL, SA, DB};
}
__host__ __device__ constexpr int fwd_elem_a(int t, int e, FwdPlan p) {
  return e | (dpp_unmix(t & ((1 << p.DL) - 1)) << 3) | ((t >> p.DL) << (3 + p.DL));
}
__host__ __device__ constexpr int fwd_elem_b(int t, int e, FwdPlan p) {
  return (e << (p.L - 3)) | (dpp_unmix(t & ((1 << p.DB) - 1)) << p.SA) | (t >> p.DB);
}
// Inverses: the thread and register of element i.
__host__ __device__ inline void fwd_place_a(int i, FwdPlan p, int& t, int& e) {
  e = i & 7;
  t = dpp_mix((i >> 3) & ((1 << p.DL) - 1)) | ((i >> (3 + p.DL)) << p.DL);
}
__host__ __device__ inline void fwd_place_b(int i, FwdPlan p, int& t, int& e) {
  e = i >> (p.L - 3);
  const int r = i & ((1 << (p.L - 3)) - 1);
  t = dpp_mix((r >> p.SA) & ((1 << p.DB) - 1)) | ((r & ((1 << p.SA) - 1)) << p.DB);
}
// Float index in fgt of the coefficient stage s < L-1 applies at element i
// (beta at its pair's lower element, gamma at the upper one).  Each stage
// fills 8 floats of every thread, rows 2s and 2s+1: on register bit q, pair
// slot j (the register pair (j with a zero inserted at bit q, and | 2^q))
// holds (beta, gamma) at floats 2j, 2j+1; on a lane-mapped bit, float e is
// register e's own coefficient.
__host__ __device__ inline int64_t fwd_coef_index(int s, int i, int L) {
  const FwdPlan p = fwd_plan(L);
  const bool in_a = s < p.SA;
  int t, e;
  if (in_a) fwd_place_a(i, p, t, e);
  else fwd_place_b(i, p, t, e);
  const bool reg = in_a ? s < 3 : s >= L - 3;
  int comp = e;
  if (reg) {
    const int q = in_a ? s : s - (L - 3);
    const int j = ((e >> (q + 1)) << q) | (e & ((1 << q) - 1));
    comp = 2 * j + ((e >> q) & 1);
  }
  const int64_t T = (int64_t)1 << (L - 3);
  return ((2 * s + (comp >> 2)) * T + t) * 4 + (comp & 3);
}
// The last stage, 16 floats per thread in rows 2(L-1)..2(L-1)+3.  In phase
// B (register bit 2): pair slot j's 2x2 matrix (k.x, k.y, k.z, k.w) as
// row 2(L-1)+j; returns the index of its first float, i the lower element.
// In phase A (one-phase rows, a lane-mapped bit): element e's (a, b) of
// y_e = a w_e + b w_partner at floats 2e, 2e+1; returns the index of a.
__host__ __device__ inline int64_t fwd_last_index(int i, int L) {
  const FwdPlan p = fwd_plan(L);
  const int64_t T = (int64_t)1 << (L - 3);
  int t, e;
  if (p.SA < L) {
    fwd_place_b(i, p, t, e);
    return ((2 * (L - 1) + (e & 3)) * T + t) * 4;
  }
  fwd_place_a(i, p, t, e);
  return ((2 * (L - 1) + (e >> 1)) * T + t) * 4 + 2 * (e & 1);
}

// Everything one forward launch needs.  tab is the prepared table of the
// butterfly of length nb; mix is the m x m Kronecker factor (nullptr for a
// plain butterfly).
struct FwdParams {
  const void* x;
  void* y;
  uint8_t* codes;     // nullptr: no quantization
  uint16_t* scales;
  uint16_t* zeros;    // asymmetric mode only
  Table tab;
  const float* mix;
  int64_t rows;
  int32_t m;          // segments per row (1 = plain butterfly)
  int32_t lognb;      // log2 of the butterfly length
  int32_t x_bf16;     // 1: bf16 input, 0: fp32 input
  int32_t y_kind;     // YKind
  int32_t bits;       // 2 or 4 (ignored without codes)
  int32_t group;      // elements per quantization group
  int32_t asym;       // 1: asymmetric min-max, 0: symmetric absmax
};

struct BwdParams {
  const float* x;
  const float* g;
  float* y;           // optional
  float* dx;
  float* partials;    // [nblk][log2 n][n/2]
  Table tab;
  int64_t rows;
  int32_t logn;
  int32_t nblk;       // number of partial slots = grid size
  // Kronecker composites (launch_backward_kron): g is [rows / m][m n] and
  // the kernel forms each segment's dL/dz = (O^T kron I) g as it loads it;
  // mix = O, [m][m] row-major (the caller's).  m = 0 otherwise.
  const float* mix;
  int32_t m;
};

// Kernel-launch helpers; each returns the hipError_t of the launch.
// hadamard: the table of H_n = Q(pi/4) D (theta unused); see prepare_kernel.
hipError_t launch_prepare(const float* theta, void* table, int logn, hipStream_t s,
                          bool hadamard = false);
hipError_t launch_forward(const FwdParams& p, hipStream_t s);

// The butterfly of length 8192 (two passes, bfly_fwd8k.hip).  Its table:
// the two half tables (n = 4096 layout), then (cos, sin) of stage 12's
// 4096 angles, table8k_bytes() in all.
struct Fwd8kParams {
  const void* x;      // [rows][8192], bf16 (x_bf16) or fp32
  int32_t x_bf16;
  void* y;            // [rows][8192] of y_kind, or nullptr
  int32_t y_kind;     // YKind
  uint8_t* codes;     // nullptr: no quantization
  uint16_t* scales;
  uint16_t* zeros;
  int32_t bits, group, asym;
  int64_t rows;
  const void* table;  // table8k_bytes()
  float* v;           // [rows][8192] fp32 scratch between the passes
};
size_t table8k_bytes();
// The table of n = 8192 from theta (or of H_8192), in one launch.
hipError_t launch_prepare_8192(const float* theta, void* table, bool hadamard, hipStream_t s);
hipError_t launch_forward_8192(const Fwd8kParams& p, hipStream_t s);

// The wide Kronecker composite in one pass (bfly_kron_fused.hip): segments
// of 256, bf16 rows, m in [2, 64].
struct KronFusedParams {
  const void* x;       // [rows][m * 256] bf16
  void* y;             // [rows][m * 256] bf16 (y_bf16) or fp32, or nullptr
  int32_t y_bf16;
  uint8_t* codes;      // nullptr: no quantization
  uint16_t* scales;
  uint16_t* zeros;
  int32_t bits, group, asym;
  const float* mix;    // [m][m] fp32
  const float2* cs;    // the table's (cos, sin) of B's 8 x 128 pairs
  const float* fgt;    // the table's scaled form (forward layout)
  int64_t rows;
  int32_t m;
};
bool kron_fused_supported(int m, int nb, bool xbf16);
hipError_t launch_kron_fused(const KronFusedParams& p, hipStream_t s);

// Events attached to the next forward-kernel dispatch (kernel-only timing):
// returns the pair armed by bfly_time_next_forward and disarms it (both null
// when nothing is armed).
struct LaunchEvents {
  hipEvent_t start = nullptr, stop = nullptr;
};
LaunchEvents take_forward_events();
void arm_forward_events(hipEvent_t start, hipEvent_t stop);
hipError_t launch_backward(const BwdParams& p, float* dtheta, hipStream_t s);
// The backward of (O kron B) over rows / m rows of m segments (p.rows counts
// segments), the O^T mix folded into the gradient loads: m <= kKronBwdFusedM,
// g not aliased by dx.
constexpr int kKronBwdFusedM = 5;
hipError_t launch_backward_kron(const BwdParams& p, float* dtheta, hipStream_t s);

// Whether a forward instantiation exists for (lognb, m); validation uses it.
bool forward_supported(int lognb, int m);

// Launch facts of one kernel on the current device: its dynamic-LDS limit
// raised to lds_bytes (when above the 64 KiB default), how many of its
// workgroups of `threads` threads one CU holds at once (per_cu >= 1) and the
// device's CU count.  Worked out once per (kernel, device) under a lock and
// cached; thread-safe.  Either output pointer may be NULL.
hipError_t kernel_setup(const void* kernel, int threads, size_t lds_bytes, int* per_cu,
                        int* num_cu);

// Grid size of the backward: a function of (rows, logn) only, so that the
// angle-gradient summation order never depends on the device.
int backward_blocks(int64_t rows, int logn);

}  // namespace bfly
