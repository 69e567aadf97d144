// One calibration step whose reconstruction term is the layer's output
// (duidaima.com write-up of ButterflyQuant, section "training and results":
// the quantized model's output should match the original one; the
// ButterflyQuant abstract: computational invariance W x = (W Q^T)(Q x) and
// 2-bit weights).  With Xr = Q X, Wr = W Q^T and What the group quantizer's
// value of Wr:
//   L_rec = ||Xr What^T - X W^T||^2 / (rows * out),
// the quantizer's rounding passed straight through (E = What - Wr held
// constant).  Because Q is orthogonal, Xr What^T - X W^T = Xr E^T exactly,
// and the two chain-rule branches (through Xr and through Wr) collapse into
// one: dL/dXr = 2 (Xr E^T) E / (rows * out), so the angle gradient is the
// butterfly backward of X alone.  The two products are dense contractions
// and run on the matrix cores in fp32 (v_mfma_f32_32x32x2_f32); the rest are
// the library's butterfly, quantizer and histogram kernels.
#include "bfly_calib.h"
#include "bfly_calib_w.h"
#include "bfly_common.h"

namespace bfly {
namespace {

typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int GM = 128, GN = 128, GK = 16;  // workgroup tile and k chunk
constexpr int GTHREADS = 256;               // 2 x 2 waves of 64 x 64
constexpr int APAD = GK + 1;                // LDS row of a k-contiguous tile (odd: no bank conflicts)

// C[M][N] = alpha * sum_k A[m][k] B(k, n) in fp32 on the matrix cores.
//   A: row-major [M][K];  BT: B given as Bt[N][K] row-major, else B[K][N].
//   K % 16 == 0.  Rows of A (and of Bt) past the end read zeros through the
//   buffer ranges; columns of B[K][N] past N read the next row's values,
//   which only reach outputs that are not stored.
// ss (optional): per workgroup, the sum of squares of its stored outputs, in
// a fixed order (lane pairs by xor shuffles, then the four waves in order).
template <bool BT>
__global__ __launch_bounds__(GTHREADS) void gemm_f32_kernel(const float* __restrict__ A,
                                                            const float* __restrict__ B,
                                                            float* __restrict__ C, int64_t M,
                                                            int32_t N, int32_t K, float alpha,
                                                            float* __restrict__ ss) {
  __shared__ __align__(16) float as[2][GM * APAD];
  __shared__ __align__(16) float bs[2][BT ? GN * APAD : GK * GN];
  __shared__ float wsum[GTHREADS / 64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int ntn = (N + GN - 1) / GN;
  const int64_t tm = blockIdx.x / ntn;
  const int tn = (int)(blockIdx.x - tm * ntn);
  const int64_t m0 = tm * GM;
  const int n0 = tn * GN;
  const int64_t mrows = M - m0 < GM ? M - m0 : GM;
  const auto ra = buffer_range32(A + m0 * K, (uint32_t)mrows * (uint32_t)K * 4u);
  const int nrows = N - n0 < GN ? N - n0 : GN;
  const auto rb = BT ? buffer_range32(B + (int64_t)n0 * K, (uint32_t)nrows * (uint32_t)K * 4u)
                     : buffer_range32(B + n0, (uint32_t)((int64_t)K * N - n0) * 4u);
  // this thread's part of a chunk: 8 consecutive floats
  const int ar = tid >> 1, ak = (tid & 1) * 8;           // A and Bt: row, k offset
  const int bk = tid >> 4, bn = (tid & 15) * 8;          // B[K][N]: k row, n offset
  uint4 la[2], lb[2];
  auto gload = [&](int k0) {
#pragma unroll
    for (int h = 0; h < 2; ++h) la[h] = buf_ld16(ra, (uint32_t)(ar * K + k0 + ak + 4 * h) * 4u);
#pragma unroll
    for (int h = 0; h < 2; ++h)
      lb[h] = BT ? buf_ld16(rb, (uint32_t)(ar * K + k0 + ak + 4 * h) * 4u)
                 : buf_ld16(rb, (uint32_t)((k0 + bk) * N + bn + 4 * h) * 4u);
  };
  auto lstore = [&](int buf) {
    const uint32_t va[8] = {la[0].x, la[0].y, la[0].z, la[0].w, la[1].x, la[1].y, la[1].z, la[1].w};
#pragma unroll
    for (int i = 0; i < 8; ++i) as[buf][ar * APAD + ak + i] = __uint_as_float(va[i]);
    if (BT) {
      const uint32_t vb[8] = {lb[0].x, lb[0].y, lb[0].z, lb[0].w, lb[1].x, lb[1].y, lb[1].z, lb[1].w};
#pragma unroll
      for (int i = 0; i < 8; ++i) bs[buf][ar * APAD + ak + i] = __uint_as_float(vb[i]);
    } else {
#pragma unroll
      for (int h = 0; h < 2; ++h)
        *reinterpret_cast<uint4*>(&bs[buf][bk * GN + bn + 4 * h]) = lb[h];
    }
  };
  f32x16_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const int nk = K / GK;
  gload(0);
  lstore(0);
  __syncthreads();
  for (int kc = 0; kc < nk; ++kc) {
    const int cb = kc & 1;
    if (kc + 1 < nk) gload((kc + 1) * GK);  // the next chunk is in flight during this one
#pragma unroll
    for (int ks = 0; ks < GK / 2; ++ks) {
      const int k = 2 * ks + (lane >> 5);
      float a[2], b[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) a[i] = as[cb][(wm * 64 + i * 32 + (lane & 31)) * APAD + k];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int col = wn * 64 + j * 32 + (lane & 31);
        b[j] = BT ? bs[cb][col * APAD + k] : bs[cb][k * GN + col];
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[i], b[j], acc[i][j], 0, 0, 0);
    }
    if (kc + 1 < nk) lstore(cb ^ 1);
    __syncthreads();
  }

  // outputs: lane holds column (lane & 31) of each 32 x 32 tile, rows
  // 8 (r / 4) + 4 (lane / 32) + r % 4
  const auto rc = buffer_range32(C + m0 * N, (uint32_t)mrows * (uint32_t)N * 4u);
  float sq = 0.f;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int col = wn * 64 + j * 32 + (lane & 31);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = wm * 64 + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        const float v = alpha * acc[i][j][r];
        const bool ok = n0 + col < N && row < mrows;
        sq = ok ? fmaf(v, v, sq) : sq;
        buf_st4(rc, ok ? (uint32_t)(row * N + n0 + col) * 4u : kOutOfRange, __float_as_uint(v));
      }
    }
  if (ss != nullptr) {
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) sq += __shfl_xor(sq, o, 64);
    if (lane == 0) wsum[wave] = sq;
    __syncthreads();
    if (tid == 0) ss[blockIdx.x] = ((wsum[0] + wsum[1]) + wsum[2]) + wsum[3];
  }
}

__device__ __forceinline__ float half_bits_to_float(uint16_t h) {
  return (float)__builtin_bit_cast(_Float16, h);
}

// E[o][k] = What[o][k] - Wr[o][k] in place: the group quantizer's value
// (scale * q, or scale * (q - zero)) minus the rotated weight.  Each thread
// takes 8 consecutive elements of one row.
__global__ __launch_bounds__(256) void quant_residual_kernel(float* __restrict__ wr,
                                                             const uint8_t* __restrict__ codes,
                                                             const uint16_t* __restrict__ scales,
                                                             const uint16_t* __restrict__ zeros,
                                                             int64_t out, int32_t n, int32_t bits,
                                                             int32_t group, int32_t asym) {
  const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;  // chunk of 8
  const int64_t chunks = out * (int64_t)(n / 8);
  if (c >= chunks) return;
  const int64_t o = c / (n / 8);
  const int k0 = (int)(c - o * (n / 8)) * 8;
  const int ng = n / group;
  const int64_t gi = o * ng + k0 / group;
  const float s = half_bits_to_float(scales[gi]);
  const float z = asym ? half_bits_to_float(zeros[gi]) : 0.f;
  // 8 codes: one 32-bit word (INT4) or 16 bits (INT2), element e in bits [bits e, bits (e+1))
  uint32_t word;
  if (bits == 4) word = *reinterpret_cast<const uint32_t*>(codes + o * (n / 2) + k0 / 2);
  else word = *reinterpret_cast<const uint16_t*>(codes + o * (n / 4) + k0 / 4);
  float4* p = reinterpret_cast<float4*>(wr + o * n + k0);
  float4 v0 = p[0], v1 = p[1];
  float w8[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
  const uint32_t mask = (1u << bits) - 1u;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    int q = (int)((word >> (bits * e)) & mask);
    if (!asym && q >= (1 << (bits - 1))) q -= 1 << bits;  // two's complement field
    w8[e] = s * ((float)q - z) - w8[e];                   // the product is exact in fp32
  }
  p[0] = make_float4(w8[0], w8[1], w8[2], w8[3]);
  p[1] = make_float4(w8[4], w8[5], w8[6], w8[7]);
}

// G += lambda's share of dL/dXr: the uniformity term of the rotated
// activations (the same soft histogram as the activation-side step, from
// the group maxima and log-bins of the histogram pass).  Four elements per
// thread through 16-byte accesses (count is a multiple of 4, a group at
// least 8 elements, Xr and G 16-byte aligned in the workspace); each element
// takes the same operations as one at a time did (one element per thread
// ran at 2.5 TB/s).
__global__ __launch_bounds__(256) void kl_grad_add_kernel(const float* __restrict__ xr,
                                                          const float* __restrict__ amax,
                                                          const float* __restrict__ lb_in,
                                                          float* __restrict__ g, int64_t count,
                                                          int32_t group, int32_t bins,
                                                          float kl_scale) {
  __shared__ float lb[CALIB_MAX_BINS];
  if (threadIdx.x < bins) lb[threadIdx.x] = lb_in[threadIdx.x];
  __syncthreads();
  const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i >= count) return;
  const float a = amax[i / group];
  if (!(a > 0.f)) return;
  const float h_inv = 0.5f * (float)bins;
  const float4 x4 = *reinterpret_cast<const float4*>(xr + i);
  float4 g4 = *reinterpret_cast<const float4*>(g + i);
  const float xs[4] = {x4.x, x4.y, x4.z, x4.w};
  float gs[4] = {g4.x, g4.y, g4.z, g4.w};
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const float t = fmaf(xs[k] / a, h_inv, h_inv - 0.5f);  // (u + 1) / h - 1/2
    if (t >= 0.f && t <= (float)(bins - 1)) {
      const int j = min((int)t, bins - 2);
      gs[k] = fmaf(kl_scale / a, lb[j + 1] - lb[j], gs[k]);
    }
  }
  *reinterpret_cast<float4*>(g + i) = make_float4(gs[0], gs[1], gs[2], gs[3]);
}

// loss[1] = sum of the partial sums of squares / n_rec (fixed order, fp64),
// loss[0] = loss[1] + lambda * loss[2] (the uniformity term, already there).
__global__ __launch_bounds__(256) void weight_loss_kernel(const float* __restrict__ ss, int64_t nparts,
                                                          double n_rec, float lambda_kl,
                                                          float* __restrict__ loss) {
  __shared__ double part[256];
  const int t = threadIdx.x;
  double acc = 0.0;
  int64_t k = t;
  for (; k + 3 * 256 < nparts; k += 4 * 256) {  // in order, four loads in flight
    const float a0 = ss[k], a1 = ss[k + 256], a2 = ss[k + 512], a3 = ss[k + 768];
    acc += (double)a0;
    acc += (double)a1;
    acc += (double)a2;
    acc += (double)a3;
  }
  for (; k < nparts; k += 256) acc += (double)ss[k];
  part[t] = acc;
  __syncthreads();
  if (t == 0) {
    double s = 0.0;
    for (int k = 0; k < 256; ++k) s += part[k];
    const double rec = s / n_rec;
    loss[1] = (float)rec;
    loss[0] = (float)(rec + (double)lambda_kl * (double)loss[2]);
  }
}

}  // namespace

int64_t gemm_f32_tiles(int64_t M, int32_t N) { return ((M + GM - 1) / GM) * ((N + GN - 1) / GN); }

hipError_t launch_gemm_f32(const float* A, const float* B, bool b_transposed, float* C, int64_t M,
                           int32_t N, int32_t K, float alpha, float* ss, hipStream_t s) {
  const int64_t tiles = gemm_f32_tiles(M, N);
  if (b_transposed)
    hipLaunchKernelGGL(gemm_f32_kernel<true>, dim3((unsigned)tiles), dim3(GTHREADS), 0, s, A, B, C,
                       M, N, K, alpha, ss);
  else
    hipLaunchKernelGGL(gemm_f32_kernel<false>, dim3((unsigned)tiles), dim3(GTHREADS), 0, s, A, B,
                       C, M, N, K, alpha, ss);
  return hipGetLastError();
}

hipError_t launch_quant_residual(float* wr, const uint8_t* codes, const uint16_t* scales,
                                 const uint16_t* zeros, int64_t out, int32_t n, int32_t bits,
                                 int32_t group, bool asym, hipStream_t s) {
  const int64_t chunks = out * (int64_t)(n / 8);
  hipLaunchKernelGGL(quant_residual_kernel, dim3((unsigned)((chunks + 255) / 256)), dim3(256), 0, s,
                     wr, codes, scales, zeros, out, n, bits, group, asym ? 1 : 0);
  return hipGetLastError();
}

hipError_t launch_kl_grad_add(const float* xr, const float* amax, const float* lb, float* g,
                              int64_t count, int32_t group, int32_t bins, float kl_scale,
                              hipStream_t s) {
  hipLaunchKernelGGL(kl_grad_add_kernel, dim3((unsigned)((count / 4 + 255) / 256)), dim3(256), 0, s,
                     xr, amax, lb, g, count, group, bins, kl_scale);
  return hipGetLastError();
}

hipError_t launch_weight_loss(const float* ss, int64_t nparts, double n_rec, float lambda_kl,
                              float* loss, hipStream_t s) {
  hipLaunchKernelGGL(weight_loss_kernel, dim3(1), dim3(256), 0, s, ss, nparts, n_rec, lambda_kl,
                     loss);
  return hipGetLastError();
}

}  // namespace bfly
