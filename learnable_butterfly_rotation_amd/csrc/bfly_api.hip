// C ABI of libbfly (include/bfly.h): argument validation, workspace
// accounting and dispatch to the kernel instantiations.  Every argument is
// checked before the first HIP call, so all error paths can be exercised on
// a machine without a GPU.
#include <stdint.h>
#include <string.h>

#include <mutex>

#include "../../include/bfly.h"
#include "bfly_internal.h"
#include "bfly_calib.h"
#include "bfly_qgemm.h"

namespace bfly {
hipError_t launch_forward_plain(const FwdParams& p, hipStream_t s);
hipError_t launch_forward_kron_m2(const FwdParams& p, hipStream_t s);
hipError_t launch_forward_kron_m3(const FwdParams& p, hipStream_t s);
hipError_t launch_forward_kron_m4(const FwdParams& p, hipStream_t s);
hipError_t launch_forward_kron_m5(const FwdParams& p, hipStream_t s);
hipError_t launch_forward_kron_m6(const FwdParams& p, hipStream_t s);
hipError_t launch_forward_kron_m7(const FwdParams& p, hipStream_t s);
hipError_t launch_forward_kron_m8(const FwdParams& p, hipStream_t s);
hipError_t launch_kron_mix(const void* x, bool xbf16, float* v, const float* mix, int64_t rows,
                           int m, int nb, hipStream_t s);
hipError_t launch_kron_bwd_setup(const float* mix, int m, float* mix_t, float* theta0, int n_theta,
                                 hipStream_t s);

bool forward_supported(int lognb, int m) {
  if (m == 1) return lognb >= 6 && lognb <= 12;
  if (m < 2 || m > 8) return false;
  return lognb >= 8 && lognb <= 12 && ((int64_t)m << lognb) <= 8192;
}

hipError_t launch_forward(const FwdParams& p, hipStream_t s) {
  switch (p.m) {
    case 1: return launch_forward_plain(p, s);
    case 2: return launch_forward_kron_m2(p, s);
    case 3: return launch_forward_kron_m3(p, s);
    case 4: return launch_forward_kron_m4(p, s);
    case 5: return launch_forward_kron_m5(p, s);
    case 6: return launch_forward_kron_m6(p, s);
    case 7: return launch_forward_kron_m7(p, s);
    case 8: return launch_forward_kron_m8(p, s);
    default: return hipErrorInvalidValue;
  }
}

namespace {
std::mutex g_events_mu;
LaunchEvents g_events;  // armed by bfly_time_next_forward, taken by the next forward launch
}  // namespace

LaunchEvents take_forward_events() {
  std::lock_guard<std::mutex> lock(g_events_mu);
  const LaunchEvents ev = g_events;
  g_events = LaunchEvents{};
  return ev;
}

void arm_forward_events(hipEvent_t start, hipEvent_t stop) {
  std::lock_guard<std::mutex> lock(g_events_mu);
  g_events.start = start;
  g_events.stop = stop;
}
}  // namespace bfly

namespace {

thread_local int32_t g_last_hip_error = 0;

bfly_status hip_fail(hipError_t e) {
  g_last_hip_error = (int32_t)e;
  return BFLY_ERR_HIP;
}

int log2_pow2(int64_t n) {
  if (n < 1 || (n & (n - 1)) != 0) return -1;
  int l = 0;
  while ((int64_t(1) << l) < n) ++l;
  return l;
}

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

// Butterfly length: power of two in [64, 8192] (smaller powers of two are
// valid sizes the library does not handle).
bfly_status check_n(int64_t n, int max_log, int* logn) {
  const int l = log2_pow2(n);
  if (l < 1) return BFLY_ERR_SIZE;
  if (l < 6 || l > max_log) return BFLY_ERR_UNSUPPORTED;
  *logn = l;
  return BFLY_OK;
}

bool dtype_ok(int d) { return d == BFLY_F32 || d == BFLY_BF16; }

size_t coeff_bytes_l(int logn) { return bfly::table_bytes(logn); }

size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// Rows handled together by one backward workgroup (threads per row = n / 8).
int bwd_rows_per_block(int logn) {
  const int t = (1 << logn) >> 3;
  return (256 / t) > 0 ? 256 / t : 1;
}

// Data pointers may be NULL when there are no rows (empty tensors).
bfly_status check_quant(const uint8_t* codes, const uint16_t* scales, const uint16_t* zeros,
                        int64_t rows, int64_t n, int64_t seg, int logseg, int32_t bits,
                        int32_t group, bfly_qmode mode) {
  if (rows > 0 && (!codes || !scales)) return BFLY_ERR_NULL;
  if (bits != 2 && bits != 4) return BFLY_ERR_QUANT;
  if (mode != BFLY_SYM_ABSMAX && mode != BFLY_ASYM_MINMAX) return BFLY_ERR_QUANT;
  if (rows > 0 && (mode == BFLY_ASYM_MINMAX) != (zeros != nullptr)) return BFLY_ERR_QUANT;
  if (rows == 0 && mode == BFLY_SYM_ABSMAX && zeros != nullptr) return BFLY_ERR_QUANT;
  const int lg = log2_pow2(group);
  if (lg < 3 || lg > 9 || group > seg || seg % group != 0 || n % group != 0) return BFLY_ERR_QUANT;
  if ((group * bits) % 8 != 0) return BFLY_ERR_QUANT;
  // a thread holds 16 elements at length 8192 (8 elsewhere): groups of 8 would split it
  if (logseg >= 13 && group < 16) return BFLY_ERR_UNSUPPORTED;
  if (!aligned(codes, 16)) return BFLY_ERR_ALIGN;
  if (!aligned(scales, 2) || (zeros && !aligned(zeros, 2))) return BFLY_ERR_ALIGN;
  return BFLY_OK;
}

// Runs `launch` with the coefficient table `coeffs`, or -- when coeffs is
// NULL -- prepares the table from theta into stream-ordered scratch first.
template <class F>
bfly_status with_table(const float* theta, const void* coeffs, int logn, hipStream_t s, F launch) {
  if (coeffs) {
    const hipError_t e = launch(coeffs);
    return e == hipSuccess ? BFLY_OK : hip_fail(e);
  }
  void* tab = nullptr;
  hipError_t e = hipMallocAsync(&tab, coeff_bytes_l(logn), s);
  if (e != hipSuccess) return hip_fail(e);
  e = bfly::launch_prepare(theta, tab, logn, s);
  if (e == hipSuccess) e = launch(tab);
  const hipError_t ef = hipFreeAsync(tab, s);
  if (e != hipSuccess) return hip_fail(e);
  if (ef != hipSuccess) return hip_fail(ef);
  return BFLY_OK;
}

}  // namespace

extern "C" {

size_t bfly_coeff_bytes(int32_t n) {
  int l = 0;
  if (check_n(n, 13, &l) != BFLY_OK) return 0;
  return coeff_bytes_l(l);
}

bfly_status bfly_prepare(const float* theta, int32_t n, void* coeffs, size_t coeff_bytes,
                         void* hip_stream) {
  if (!theta || !coeffs) return BFLY_ERR_NULL;
  int l = 0;
  const bfly_status st = check_n(n, 13, &l);
  if (st != BFLY_OK) return st;
  if (coeff_bytes < coeff_bytes_l(l)) return BFLY_ERR_WORKSPACE;
  if (!aligned(coeffs, 16) || !aligned(theta, 4)) return BFLY_ERR_ALIGN;
  const hipError_t e = bfly::launch_prepare(theta, coeffs, l, (hipStream_t)hip_stream);
  return e == hipSuccess ? BFLY_OK : hip_fail(e);
}

bfly_status bfly_time_next_forward(void* start_event, void* stop_event) {
  if (!start_event != !stop_event) return BFLY_ERR_NULL;  // both NULL: disarm
  bfly::arm_forward_events((hipEvent_t)start_event, (hipEvent_t)stop_event);
  return BFLY_OK;
}

bfly_status bfly_prepare_hadamard(int32_t n, void* coeffs, size_t coeff_bytes, void* hip_stream) {
  if (!coeffs) return BFLY_ERR_NULL;
  int l = 0;
  const bfly_status st = check_n(n, 13, &l);
  if (st != BFLY_OK) return st;
  if (coeff_bytes < coeff_bytes_l(l)) return BFLY_ERR_WORKSPACE;
  if (!aligned(coeffs, 16)) return BFLY_ERR_ALIGN;
  const hipError_t e = bfly::launch_prepare(nullptr, coeffs, l, (hipStream_t)hip_stream, true);
  return e == hipSuccess ? BFLY_OK : hip_fail(e);
}

static bfly_status forward_common(const void* x, bfly_dtype x_dt, void* y, bfly_dtype y_dt,
                                  uint8_t* codes, uint16_t* scales, uint16_t* zeros, int64_t rows,
                                  int32_t m, int32_t nb, const float* theta, const void* coeffs,
                                  const float* mix, int32_t bits, int32_t group, bfly_qmode mode,
                                  bool quant, void* hip_stream) {
  if (rows > 0 && !x) return BFLY_ERR_NULL;
  if (!theta && !coeffs) return BFLY_ERR_NULL;
  if (rows > 0 && !y && !quant) return BFLY_ERR_NULL;
  if (!dtype_ok(x_dt) || (y && !dtype_ok(y_dt))) return BFLY_ERR_DTYPE;
  if (rows < 0) return BFLY_ERR_SIZE;
  int lognb = 0;
  bfly_status st = check_n(nb, 13, &lognb);
  if (st != BFLY_OK) return st;
  const int64_t n = (int64_t)m * nb;
  if (n > 8192) return BFLY_ERR_UNSUPPORTED;
  if (quant) {
    st = check_quant(codes, scales, zeros, rows, n, nb, lognb, bits, group, mode);
    if (st != BFLY_OK) return st;
  }
  if (!bfly::forward_supported(lognb, m)) return BFLY_ERR_UNSUPPORTED;
  if (!aligned(x, 16) || (y && !aligned(y, 16))) return BFLY_ERR_ALIGN;
  if ((coeffs && !aligned(coeffs, 16)) || (theta && !aligned(theta, 4)) ||
      (mix && !aligned(mix, 4)))
    return BFLY_ERR_ALIGN;
  if (rows == 0) return BFLY_OK;

  bfly::FwdParams p;
  memset(&p, 0, sizeof(p));
  p.x = x;
  p.y = y;
  p.codes = quant ? codes : nullptr;
  p.scales = quant ? scales : nullptr;
  p.zeros = quant ? zeros : nullptr;
  p.mix = mix;
  p.rows = rows;
  p.m = m;
  p.lognb = lognb;
  p.x_bf16 = x_dt == BFLY_BF16;
  p.y_kind = !y ? bfly::Y_NONE : (y_dt == BFLY_BF16 ? bfly::Y_BF16 : bfly::Y_F32);
  p.bits = quant ? bits : 0;
  p.group = quant ? group : 0;
  p.asym = quant && mode == BFLY_ASYM_MINMAX;
  const hipStream_t s = (hipStream_t)hip_stream;
  return with_table(theta, coeffs, lognb, s, [&](const void* tab) {
    p.tab = bfly::table_at(tab, lognb);
    return bfly::launch_forward(p, s);
  });
}

bfly_status bfly_forward(const void* x, bfly_dtype x_dt, void* y, bfly_dtype y_dt, int64_t rows,
                         int32_t n, const float* theta, const void* coeffs, void* hip_stream) {
  if (rows > 0 && !y) return BFLY_ERR_NULL;
  return forward_common(x, x_dt, y, y_dt, nullptr, nullptr, nullptr, rows, 1, n, theta, coeffs,
                        nullptr, 0, 0, BFLY_SYM_ABSMAX, false, hip_stream);
}

bfly_status bfly_forward_quant(const void* x, bfly_dtype x_dt, void* y, bfly_dtype y_dt,
                               uint8_t* codes, uint16_t* scales, uint16_t* zeros, int64_t rows,
                               int32_t n, const float* theta, const void* coeffs, int32_t bits,
                               int32_t group, bfly_qmode mode, void* hip_stream) {
  return forward_common(x, x_dt, y, y_dt, codes, scales, zeros, rows, 1, n, theta, coeffs,
                        nullptr, bits, group, mode, true, hip_stream);
}

bfly_status bfly_kron_forward(const void* x, bfly_dtype x_dt, void* y, bfly_dtype y_dt,
                              uint8_t* codes, uint16_t* scales, uint16_t* zeros, int64_t rows,
                              int32_t m, int32_t nb, const float* theta_b, const void* coeffs_b,
                              const float* mix, int32_t bits, int32_t group, bfly_qmode mode,
                              void* hip_stream) {
  if (!mix) return BFLY_ERR_NULL;
  if (m < 1 || m > 8) return BFLY_ERR_SIZE;
  if (!codes && (scales || zeros)) return BFLY_ERR_QUANT;
  if (log2_pow2(nb) >= 13) return BFLY_ERR_UNSUPPORTED;
  return forward_common(x, x_dt, y, y_dt, codes, scales, zeros, rows, m, nb, theta_b, coeffs_b,
                        mix, bits, group, mode, codes != nullptr, hip_stream);
}

size_t bfly_backward_workspace_bytes(int64_t rows, int32_t n) {
  int l = 0;
  if (rows < 0 || check_n(n, 12, &l) != BFLY_OK) return 0;
  const size_t slots = (size_t)bfly::backward_blocks(rows, l) * bwd_rows_per_block(l);
  return align_up(coeff_bytes_l(l), 256) + slots * ((size_t)l << (l - 1)) * sizeof(float);
}

bfly_status bfly_backward(const float* x, const float* g, float* y, float* dx, float* dtheta,
                          int64_t rows, int32_t n, const float* theta, const void* coeffs,
                          void* workspace, size_t workspace_bytes, void* hip_stream) {
  if ((rows > 0 && (!x || !g || !dx)) || !dtheta || !workspace) return BFLY_ERR_NULL;
  if (!theta && !coeffs) return BFLY_ERR_NULL;
  if (rows < 0) return BFLY_ERR_SIZE;
  int l = 0;
  const bfly_status st = check_n(n, 12, &l);
  if (st != BFLY_OK) return st;
  if (workspace_bytes < bfly_backward_workspace_bytes(rows, n)) return BFLY_ERR_WORKSPACE;
  if (!aligned(x, 16) || !aligned(g, 16) || !aligned(dx, 16) || !aligned(y, 16) ||
      !aligned(workspace, 16) || !aligned(dtheta, 4) || (coeffs && !aligned(coeffs, 16)) ||
      (theta && !aligned(theta, 4)))
    return BFLY_ERR_ALIGN;
  const hipStream_t s = (hipStream_t)hip_stream;
  char* ws = static_cast<char*>(workspace);
  const void* tab = coeffs;
  if (!tab) {
    const hipError_t e = bfly::launch_prepare(theta, ws, l, s);
    if (e != hipSuccess) return hip_fail(e);
    tab = ws;
  }
  bfly::BwdParams p;
  memset(&p, 0, sizeof(p));
  p.x = x;
  p.g = g;
  p.y = y;
  p.dx = dx;
  p.partials = reinterpret_cast<float*>(ws + align_up(coeff_bytes_l(l), 256));
  p.tab = bfly::table_at(tab, l);
  p.rows = rows;
  p.logn = l;
  p.nblk = rows == 0 ? 0 : bfly::backward_blocks(rows, l);
  const hipError_t e = bfly::launch_backward(p, dtheta, s);
  return e == hipSuccess ? BFLY_OK : hip_fail(e);
}

// Wide Kronecker composites: m in [2, 64], nb in [256, 4096], m * nb <= 65536.
static bool kron_wide_sizes(int32_t m, int32_t nb, int* lognb) {
  if (m < 2 || m > 64) return false;
  if (check_n(nb, 12, lognb) != BFLY_OK || *lognb < 8) return false;
  return (int64_t)m * nb <= 65536;
}

size_t bfly_kron_forward_wide_workspace_bytes(int64_t rows, int32_t m, int32_t nb) {
  int l = 0;
  if (rows < 0 || !kron_wide_sizes(m, nb, &l)) return 0;
  return (size_t)rows * (size_t)m * (size_t)nb * sizeof(float);
}

bfly_status bfly_kron_forward_wide(const void* x, bfly_dtype x_dt, void* y, bfly_dtype y_dt,
                                   uint8_t* codes, uint16_t* scales, uint16_t* zeros,
                                   int64_t rows, int32_t m, int32_t nb, const float* theta_b,
                                   const void* coeffs_b, const float* mix, int32_t bits,
                                   int32_t group, bfly_qmode mode, void* workspace,
                                   size_t workspace_bytes, void* hip_stream) {
  const bool quant = codes != nullptr;
  if (!mix || !workspace) return BFLY_ERR_NULL;
  if (rows > 0 && (!x || (!y && !quant))) return BFLY_ERR_NULL;
  if (!theta_b && !coeffs_b) return BFLY_ERR_NULL;
  if (!quant && (scales || zeros)) return BFLY_ERR_QUANT;
  if (!dtype_ok(x_dt) || (y && !dtype_ok(y_dt))) return BFLY_ERR_DTYPE;
  if (rows < 0 || m < 2 || m > 64) return BFLY_ERR_SIZE;
  int l = 0;
  const bfly_status sn = check_n(nb, 13, &l);
  if (sn != BFLY_OK) return sn;
  if (!kron_wide_sizes(m, nb, &l)) return BFLY_ERR_UNSUPPORTED;
  if (quant) {
    const bfly_status sq = check_quant(codes, scales, zeros, rows, (int64_t)m * nb, nb, l, bits,
                                       group, mode);
    if (sq != BFLY_OK) return sq;
  }
  if (workspace_bytes < bfly_kron_forward_wide_workspace_bytes(rows, m, nb))
    return BFLY_ERR_WORKSPACE;
  if (!aligned(x, 16) || (y && !aligned(y, 16)) || !aligned(workspace, 16) || !aligned(mix, 4) ||
      (coeffs_b && !aligned(coeffs_b, 16)) || (theta_b && !aligned(theta_b, 4)))
    return BFLY_ERR_ALIGN;
  if (rows == 0) return BFLY_OK;
  // v = (O kron I) x into the workspace, then the butterfly (and the
  // quantizer) on its rows * m segments: (O kron B) = (I kron B)(O kron I)
  float* v = static_cast<float*>(workspace);
  const hipError_t e = bfly::launch_kron_mix(x, x_dt == BFLY_BF16, v, mix, rows, m, nb,
                                             (hipStream_t)hip_stream);
  if (e != hipSuccess) return hip_fail(e);
  return forward_common(v, BFLY_F32, y, y_dt, codes, scales, zeros, rows * m, 1, nb, theta_b,
                        coeffs_b, nullptr, bits, group, mode, quant, hip_stream);
}

// Workspace of the Kronecker backward: O^T, a zero angle set and its
// (identity) table, then the butterfly backward's own workspace for the
// rows * m segments.
static size_t kron_bwd_parts(int64_t rows, int32_t m, int lognb, size_t* off_theta0,
                             size_t* off_table, size_t* off_bwd) {
  const int nb = 1 << lognb;
  const size_t t0 = 256;
  const size_t tab = align_up(t0 + sizeof(float) * (size_t)lognb * (nb / 2), 256);
  const size_t bwd = align_up(tab + coeff_bytes_l(lognb), 256);
  const size_t total = bwd + bfly_backward_workspace_bytes(rows * m, nb);
  if (off_theta0) *off_theta0 = t0;
  if (off_table) *off_table = tab;
  if (off_bwd) *off_bwd = bwd;
  return total;
}

size_t bfly_kron_backward_workspace_bytes(int64_t rows, int32_t m, int32_t nb) {
  int l = 0;
  if (rows < 0 || m < 2 || m > 8 || check_n(nb, 12, &l) != BFLY_OK) return 0;
  if (!bfly::forward_supported(l, m)) return 0;
  return kron_bwd_parts(rows, m, l, nullptr, nullptr, nullptr);
}

bfly_status bfly_kron_backward(const float* x, const float* g, float* dx, float* dtheta_b,
                               int64_t rows, int32_t m, int32_t nb, const float* theta_b,
                               const void* coeffs_b, const float* mix, void* workspace,
                               size_t workspace_bytes, void* hip_stream) {
  if ((rows > 0 && (!x || !g || !dx)) || !dtheta_b || !mix || !workspace) return BFLY_ERR_NULL;
  if (!theta_b && !coeffs_b) return BFLY_ERR_NULL;
  if (rows < 0) return BFLY_ERR_SIZE;
  if (m < 1 || m > 8) return BFLY_ERR_SIZE;
  int l = 0;
  const bfly_status st = check_n(nb, 12, &l);
  if (st != BFLY_OK) return st;
  if (m == 1 || !bfly::forward_supported(l, m)) return BFLY_ERR_UNSUPPORTED;
  size_t o_th0 = 0, o_tab = 0, o_bwd = 0;
  if (workspace_bytes < kron_bwd_parts(rows, m, l, &o_th0, &o_tab, &o_bwd))
    return BFLY_ERR_WORKSPACE;
  if (!aligned(x, 16) || !aligned(g, 16) || !aligned(dx, 16) || !aligned(workspace, 16) ||
      !aligned(dtheta_b, 4) || !aligned(mix, 4) || (coeffs_b && !aligned(coeffs_b, 16)) ||
      (theta_b && !aligned(theta_b, 4)))
    return BFLY_ERR_ALIGN;
  const hipStream_t s = (hipStream_t)hip_stream;
  char* ws = static_cast<char*>(workspace);
  float* mix_t = reinterpret_cast<float*>(ws);
  float* theta0 = reinterpret_cast<float*>(ws + o_th0);
  // O^T into the workspace (the zero-angle and table regions that follow it
  // are no longer used; the layout keeps the size the query reports)
  hipError_t e = bfly::launch_kron_bwd_setup(mix, m, mix_t, theta0, 0, s);
  if (e != hipSuccess) return hip_fail(e);
  if (rows > 0) {
    // dL/dz = (O^T kron I) G: the mixing step with O^T (each thread reads all
    // m segments of its columns before writing them, so dx == g is safe)
    e = bfly::launch_kron_mix(g, false, dx, mix_t, rows, m, nb, s);
    if (e != hipSuccess) return hip_fail(e);
  }
  // then the butterfly backward on the rows * m segments, in place on dx
  const size_t bwd_bytes = workspace_bytes - o_bwd;
  return bfly_backward(x, dx, nullptr, dx, dtheta_b, rows * m, nb, theta_b, coeffs_b, ws + o_bwd,
                       bwd_bytes, hip_stream);
}

// Workspace of a calibration step: Y, the groups' max |y| (sized for the
// smallest group, 8), dtheta, the histogram partials and log-bins, then the
// backward's workspace (its table first).
static size_t calib_parts(int64_t rows, int logn, size_t* o_amax, size_t* o_dth, size_t* o_part,
                          size_t* o_lb, size_t* o_bwd) {
  const int64_t n = int64_t(1) << logn;
  const size_t amax = align_up((size_t)rows * (size_t)n * sizeof(float), 256);
  const size_t dth = align_up(amax + (size_t)rows * (size_t)(n / 8) * sizeof(float), 256);
  const size_t part = align_up(dth + sizeof(float) * (size_t)logn * (size_t)(n / 2), 256);
  const size_t lb = align_up(part + sizeof(float) * (size_t)bfly::CALIB_MAX_BLOCKS *
                                        (bfly::CALIB_MAX_BINS + 1), 256);
  const size_t bwd = align_up(lb + sizeof(float) * bfly::CALIB_MAX_BINS, 256);
  if (o_amax) *o_amax = amax;
  if (o_dth) *o_dth = dth;
  if (o_part) *o_part = part;
  if (o_lb) *o_lb = lb;
  if (o_bwd) *o_bwd = bwd;
  return bwd + bfly_backward_workspace_bytes(rows, (int32_t)n);
}

size_t bfly_calib_workspace_bytes(int64_t rows, int32_t n) {
  int l = 0;
  if (rows < 1 || check_n(n, 12, &l) != BFLY_OK) return 0;
  return calib_parts(rows, l, nullptr, nullptr, nullptr, nullptr, nullptr);
}

bfly_status bfly_calib_step(const float* x, int64_t rows, int32_t n, float* theta, float* adam_m,
                            float* adam_v, int32_t step, const bfly_calib_config* cfg,
                            float* loss, void* workspace, size_t workspace_bytes,
                            void* hip_stream) {
  if (!x || !theta || !adam_m || !adam_v || !cfg || !loss || !workspace) return BFLY_ERR_NULL;
  if (rows < 1 || step < 1) return BFLY_ERR_SIZE;
  int l = 0;
  const bfly_status sn = check_n(n, 12, &l);
  if (sn != BFLY_OK) return sn;
  const int lg = log2_pow2(cfg->group);
  if ((cfg->bits != 2 && cfg->bits != 4) || lg < 3 || lg > 9 || cfg->group > n ||
      cfg->bins < 2 || cfg->bins > bfly::CALIB_MAX_BINS)
    return BFLY_ERR_QUANT;
  size_t o_amax = 0, o_dth = 0, o_part = 0, o_lb = 0, o_bwd = 0;
  if (workspace_bytes < calib_parts(rows, l, &o_amax, &o_dth, &o_part, &o_lb, &o_bwd))
    return BFLY_ERR_WORKSPACE;
  if (!aligned(x, 16) || !aligned(workspace, 16) || !aligned(theta, 4) || !aligned(adam_m, 4) ||
      !aligned(adam_v, 4) || !aligned(loss, 4))
    return BFLY_ERR_ALIGN;
  const hipStream_t s = (hipStream_t)hip_stream;
  char* ws = static_cast<char*>(workspace);
  float* y = reinterpret_cast<float*>(ws);
  float* amax = reinterpret_cast<float*>(ws + o_amax);
  float* dth = reinterpret_cast<float*>(ws + o_dth);
  float* lb = reinterpret_cast<float*>(ws + o_lb);
  char* wsb = ws + o_bwd;  // the backward's workspace; its table area holds the table
  hipError_t e = bfly::launch_prepare(theta, wsb, l, s);
  if (e != hipSuccess) return hip_fail(e);
  // Y = Q X for the loss statistics
  const bfly_status st = bfly_forward(x, BFLY_F32, y, BFLY_F32, rows, n, nullptr, wsb, hip_stream);
  if (st != BFLY_OK) return st;
  bfly::CalibLossParams p;
  p.y = y;
  p.amax = amax;
  p.rows = rows;
  p.n = n;
  p.group = cfg->group;
  p.bits = cfg->bits;
  p.bins = cfg->bins;
  p.lambda_kl = cfg->lambda_kl;
  p.partials = reinterpret_cast<float*>(ws + o_part);
  p.lb = lb;
  p.loss = loss;
  if ((e = bfly::launch_calib_hist(p, s)) != hipSuccess) return hip_fail(e);
  if ((e = bfly::launch_calib_reduce(p, s)) != hipSuccess) return hip_fail(e);
  // dtheta: the backward forms dL/dY itself from the Y it recomputes
  const double N = (double)rows * (double)n;
  bfly::CalibGradArgs c;
  c.amax = amax;
  c.lb = lb;
  c.group = cfg->group;
  c.bits = cfg->bits;
  c.bins = cfg->bins;
  c.two_n = (float)(2.0 / N);
  c.kl_scale = (float)(cfg->lambda_kl / (N * (1.0 + cfg->bins * (double)bfly::kCalibSmooth))) /
               (2.f / cfg->bins);
  bfly::BwdParams bp;
  memset(&bp, 0, sizeof(bp));
  bp.x = x;
  bp.partials = reinterpret_cast<float*>(wsb + align_up(coeff_bytes_l(l), 256));
  bp.tab = bfly::table_at(wsb, l);
  bp.rows = rows;
  bp.logn = l;
  bp.nblk = bfly::backward_blocks(rows, l);
  if ((e = bfly::launch_backward_calib(bp, c, dth, s)) != hipSuccess) return hip_fail(e);
  e = bfly::launch_adam(theta, adam_m, adam_v, dth, l * (n / 2), step, cfg->lr, cfg->beta1,
                        cfg->beta2, cfg->eps, s);
  return e == hipSuccess ? BFLY_OK : hip_fail(e);
}

bfly_status bfly_quant_matmul(const void* a, bfly_dtype a_dt, const uint8_t* codes,
                              const uint16_t* scales, const uint16_t* zeros, void* y,
                              bfly_dtype y_dt, int64_t rows, int32_t n_out, int32_t k,
                              int32_t bits, int32_t group, bfly_qmode mode, void* hip_stream) {
  if (rows < 0 || n_out <= 0 || k <= 0) return BFLY_ERR_SIZE;
  if (rows > 0 && (!a || !y)) return BFLY_ERR_NULL;
  if (!codes || !scales) return BFLY_ERR_NULL;
  if (a_dt != BFLY_BF16 || !dtype_ok(y_dt)) return BFLY_ERR_DTYPE;
  if ((bits != 2 && bits != 4) || (mode != BFLY_SYM_ABSMAX && mode != BFLY_ASYM_MINMAX) ||
      (mode == BFLY_ASYM_MINMAX) != (zeros != nullptr))
    return BFLY_ERR_QUANT;
  if (group != 64 && group != 128 && group != 256 && group != 512) return BFLY_ERR_QUANT;
  if (k % group != 0) return BFLY_ERR_QUANT;
  if (n_out % bfly::QG_BN != 0 || n_out > (1 << 20) || k % bfly::QG_BK != 0 || k > 65536)
    return BFLY_ERR_UNSUPPORTED;
  const int64_t tiles = (rows + bfly::QG_BM - 1) / bfly::QG_BM * (n_out / bfly::QG_BN);
  if (tiles >= (int64_t(1) << 31)) return BFLY_ERR_UNSUPPORTED;
  if ((a && !aligned(a, 16)) || !aligned(codes, 16) || !aligned(scales, 2) ||
      (zeros && !aligned(zeros, 2)) || (y && !aligned(y, 16)))
    return BFLY_ERR_ALIGN;
  if (rows == 0) return BFLY_OK;
  bfly::QgemmParams p;
  p.a = static_cast<const uint16_t*>(a);
  p.codes = codes;
  p.scales = scales;
  p.zeros = zeros;
  p.y = y;
  p.rows = rows;
  p.n_out = n_out;
  p.k = k;
  p.group = group;
  p.bits = bits;
  p.asym = mode == BFLY_ASYM_MINMAX;
  p.y_bf16 = y_dt == BFLY_BF16;
  const hipError_t e = bfly::launch_qgemm(p, (hipStream_t)hip_stream);
  return e == hipSuccess ? BFLY_OK : hip_fail(e);
}

const char* bfly_status_string(bfly_status s) {
  switch (s) {
    case BFLY_OK: return "ok";
    case BFLY_ERR_NULL: return "a required pointer is NULL";
    case BFLY_ERR_SIZE: return "invalid size (rows, n, m or nb)";
    case BFLY_ERR_DTYPE: return "invalid dtype";
    case BFLY_ERR_ALIGN: return "misaligned pointer";
    case BFLY_ERR_QUANT: return "invalid quantization arguments";
    case BFLY_ERR_WORKSPACE: return "workspace or coefficient buffer too small";
    case BFLY_ERR_UNSUPPORTED: return "size not supported by the library";
    case BFLY_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

int32_t bfly_last_hip_error(void) { return g_last_hip_error; }

}  // extern "C"
