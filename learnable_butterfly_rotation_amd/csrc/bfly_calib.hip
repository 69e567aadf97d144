// One calibration step for the angles (ButterflyQuant write-up, section
// "training and results": a reconstruction loss plus a uniformity
// regulariser, the KL divergence between the rotated activations'
// distribution and the uniform one; ButterflyQuant abstract: the angles are
// learned by gradient descent on a few calibration samples).
//
// Loss on Y = Q X (N elements, groups of `group` consecutive elements of a
// row, a = the group's max |y|, s = fp16(a / qmax), y^ = s clamp(rne(y / s))):
//   L_rec = sum (y - y^)^2 / N, with y^ held constant;
//   u = y / a (a held constant); on `bins` bins of width h = 2 / bins over
//   [-1, 1] (centres c_b) each u adds linear-interpolation weights to its
//   two nearest centres (u clamped to [c_0, c_{bins-1}]): p_b = weights / N;
//   smoothed p'_b = (p_b + 1e-6) / (1 + bins 1e-6);
//   KL = sum p'_b log(bins p'_b);   L = L_rec + lambda KL.
// Gradient: dL/dy = 2 (y - y^) / N
//   + lambda (lb[j+1] - lb[j]) / (h N (1 + bins 1e-6) a)  (u inside, a > 0),
// lb[b] = log(bins p'_b), j the lower centre of u.
//
// Passes: histogram (per-lane LDS bins, fixed-order block sums; it also
// stores each group's max |y|), a one-block fixed-order reduction (fp64) to
// lb and the loss; the gradient is then formed inside the butterfly
// backward from the Y it recomputes (calib_grad), so dL/dY never goes
// through memory.  All reductions run in a fixed order: results repeat bit
// for bit.
#include "bfly_calib.h"
#include "bfly_common.h"

namespace bfly {
namespace {


// Per-group quantities of the thread's 8 elements: gt = group / 8 lanes
// share a group (gt a power of two <= 64).
struct Elt {
  float y[CALIB_EPT];
  float a;   // group max |y|
  float s;   // fp16 scale (as float)
};

__device__ __forceinline__ float group_absmax(float v, int gt) {
  for (int o = 1; o < gt; o <<= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}





__global__ __launch_bounds__(CALIB_THREADS) void calib_hist_kernel(const CalibLossParams P) {
  // lane-private bins, bin-major ([bins][256]), sized to `bins` so that more
  // workgroups fit on a CU; then the lanes' squared errors
  extern __shared__ float lh[];
  float* red = lh + P.bins * CALIB_THREADS;
  const int t = threadIdx.x, bins = P.bins;
  for (int b = 0; b < bins; ++b) lh[b * CALIB_THREADS + t] = 0.f;
  const int gt = P.group / CALIB_EPT;
  const float qmax = (float)((1 << (P.bits - 1)) - 1);
  const int64_t nchunks = P.rows * P.n / CALIB_EPT;
  const int64_t stride = (int64_t)gridDim.x * CALIB_THREADS;
  float sse = 0.f;
  int64_t c = (int64_t)blockIdx.x * CALIB_THREADS + t;
  // the next chunk's values are loaded before this one's bins are updated
  float4 n0 = make_float4(0.f, 0.f, 0.f, 0.f), n1 = n0;
  if (c < nchunks) {
    n0 = *reinterpret_cast<const float4*>(P.y + c * CALIB_EPT);
    n1 = *reinterpret_cast<const float4*>(P.y + c * CALIB_EPT + 4);
  }
  for (; c < nchunks; c += stride) {
    Elt e;
    e.y[0] = n0.x; e.y[1] = n0.y; e.y[2] = n0.z; e.y[3] = n0.w;
    e.y[4] = n1.x; e.y[5] = n1.y; e.y[6] = n1.z; e.y[7] = n1.w;
    if (c + stride < nchunks) {
      n0 = *reinterpret_cast<const float4*>(P.y + (c + stride) * CALIB_EPT);
      n1 = *reinterpret_cast<const float4*>(P.y + (c + stride) * CALIB_EPT + 4);
    }
    float m = 0.f;
#pragma unroll
    for (int k = 0; k < CALIB_EPT; ++k) m = fmaxf(m, fabsf(e.y[k]));
    e.a = group_absmax(m, gt);
    e.s = calib_fp16_rne(e.a / qmax);
    if ((t & (gt - 1)) == 0) P.amax[c * CALIB_EPT / P.group] = e.a;  // one lane per group
    // reciprocals instead of divisions: the pass is bound by its vector work
    const float inv_a = e.a > 0.f ? __builtin_amdgcn_rcpf(e.a) : 0.f;
    const float inv_s = e.s > 0.f ? __builtin_amdgcn_rcpf(e.s) : 0.f;
#pragma unroll
    for (int k = 0; k < CALIB_EPT; ++k) {
      const float yq = fminf(fmaxf(rintf(e.y[k] * inv_s), -qmax), qmax) * e.s;
      const float d = e.y[k] - yq;
      sse = fmaf(d, d, sse);
      int j;
      float f;
      bool inside;
      calib_bin(e.y[k] * inv_a, bins, j, f, inside);
      // this lane's own bins, in program order (plain read-modify-write:
      // LDS float atomics measured 7x slower here)
      lh[j * CALIB_THREADS + t] += 1.f - f;
      lh[(j + 1) * CALIB_THREADS + t] += f;
    }
  }
  red[t] = sse;
  __syncthreads();
  // fixed-order block sums: thread b < bins sums bin b over the 256 lanes
  float* out = P.partials + (int64_t)blockIdx.x * (bins + 1);
  if (t < bins) {
    float acc = 0.f;
    for (int l = 0; l < CALIB_THREADS; ++l) acc += lh[t * CALIB_THREADS + l];
    out[t] = acc;
  } else if (t == bins) {
    float acc = 0.f;
    for (int l = 0; l < CALIB_THREADS; ++l) acc += red[l];
    out[bins] = acc;
  }
}

// Fixed-order sums of the block partials: thread (q, b) adds slice q of
// the blocks for column b, then thread b adds the slices in order.
constexpr int CALIB_SLICES = 16;

__global__ __launch_bounds__(CALIB_SLICES*(CALIB_MAX_BINS + 1)) void calib_reduce_kernel(
    const CalibLossParams P, int nblk) {
  __shared__ double part[CALIB_SLICES][CALIB_MAX_BINS + 1];
  __shared__ double p[CALIB_MAX_BINS + 1];
  __shared__ double klt[CALIB_MAX_BINS];  // each bin's KL term, added in bin order below
  const int t = threadIdx.x, bins = P.bins;
  const double N = (double)P.rows * (double)P.n;
  {
    const int q = t / (CALIB_MAX_BINS + 1), b = t - q * (CALIB_MAX_BINS + 1);
    if (b <= bins) {
      const int per = (nblk + CALIB_SLICES - 1) / CALIB_SLICES;
      const int k1 = min(nblk, (q + 1) * per);
      // in order, four loads in flight (one at a time left the pass latency-bound)
      const float* const col = P.partials + b;
      const int64_t stride = bins + 1;
      double acc = 0.0;
      int k = q * per;
      for (; k + 3 < k1; k += 4) {
        const float a0 = col[k * stride], a1 = col[(k + 1) * stride];
        const float a2 = col[(k + 2) * stride], a3 = col[(k + 3) * stride];
        acc += (double)a0;
        acc += (double)a1;
        acc += (double)a2;
        acc += (double)a3;
      }
      for (; k < k1; ++k) acc += (double)col[k * stride];
      part[q][b] = acc;
    }
  }
  __syncthreads();
  if (t <= bins) {
    double acc = 0.0;
    for (int q = 0; q < CALIB_SLICES; ++q) acc += part[q][t];
    p[t] = acc / N;
  }
  __syncthreads();
  if (t < bins) {
    const double ps = (p[t] + (double)kCalibSmooth) / (1.0 + bins * (double)kCalibSmooth);
    const double lg = log(bins * ps);
    P.lb[t] = (float)lg;
    klt[t] = ps * lg;
  }
  __syncthreads();
  if (t == 0) {
    double kl = 0.0;
    for (int b = 0; b < bins; ++b) kl += klt[b];
    const double rec = p[bins];  // squared error / N
    P.loss[0] = (float)(rec + P.lambda_kl * kl);
    P.loss[1] = (float)rec;
    P.loss[2] = (float)kl;
  }
}

__global__ void adam_kernel(float* theta, float* m, float* v, const float* g, int count, float lr,
                            float beta1, float beta2, float eps, float bc1, float bc2) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= count) return;
  const float gi = g[i];
  const float mi = fmaf(beta1, m[i], (1.f - beta1) * gi);
  const float vi = fmaf(beta2, v[i], (1.f - beta2) * gi * gi);
  m[i] = mi;
  v[i] = vi;
  theta[i] -= lr * (mi / bc1) / (sqrtf(vi / bc2) + eps);
}

}  // namespace

int calib_blocks(int64_t rows, int n) {
  const int64_t chunks = rows * n / CALIB_EPT;
  const int64_t b = (chunks + CALIB_THREADS - 1) / CALIB_THREADS;
  return (int)(b < CALIB_MAX_BLOCKS ? (b < 1 ? 1 : b) : CALIB_MAX_BLOCKS);
}

hipError_t launch_calib_hist(const CalibLossParams& p, hipStream_t s) {
  const size_t lds = sizeof(float) * (size_t)(p.bins + 1) * CALIB_THREADS;
  hipLaunchKernelGGL(calib_hist_kernel, dim3(calib_blocks(p.rows, p.n)), dim3(CALIB_THREADS), lds,
                     s, p);
  return hipGetLastError();
}

hipError_t launch_calib_reduce(const CalibLossParams& p, hipStream_t s) {
  hipLaunchKernelGGL(calib_reduce_kernel, dim3(1), dim3(CALIB_SLICES * (CALIB_MAX_BINS + 1)), 0, s,
                     p, calib_blocks(p.rows, p.n));
  return hipGetLastError();
}

hipError_t launch_adam(float* theta, float* m, float* v, const float* g, int count, int step,
                       float lr, float beta1, float beta2, float eps, hipStream_t s) {
  const float bc1 = 1.f - powf(beta1, (float)step), bc2 = 1.f - powf(beta2, (float)step);
  hipLaunchKernelGGL(adam_kernel, dim3((count + 255) / 256), dim3(256), 0, s, theta, m, v, g, count,
                     lr, beta1, beta2, eps, bc1, bc2);
  return hipGetLastError();
}

}  // namespace bfly
