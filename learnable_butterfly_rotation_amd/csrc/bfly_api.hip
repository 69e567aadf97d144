// C ABI of libbfly (include/bfly.h): argument validation, workspace
// accounting and dispatch to the kernel instantiations.  Every argument is
// checked before the first HIP call, so all error paths can be exercised on
// a machine without a GPU.
#include <stdint.h>
#include <string.h>

#include <mutex>

#include "../../include/bfly.h"
#include "bfly_internal.h"
#include "bfly_common.h"
#include "bfly_calib.h"
#include "bfly_calib_w.h"
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
hipError_t launch_kron_bwd_setup(const float* mix, int m, float* mix_t, hipStream_t s);

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

namespace {
// Fixed-size open-addressing cache of kernel_setup's results (no heap
// allocation): one entry per (kernel, device) that has been launched.
struct SetupEntry {
  const void* kernel;
  int device, per_cu, num_cu;
};
constexpr int kSetupSlots = 4096;  // well above the library's kernel count
std::mutex g_setup_mu;
SetupEntry g_setup[kSetupSlots];
}  // namespace

hipError_t kernel_setup(const void* kernel, int threads, size_t lds_bytes, int* per_cu,
                        int* num_cu) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lock(g_setup_mu);
  size_t h = (reinterpret_cast<uintptr_t>(kernel) >> 4) * 0x9E3779B97F4A7C15ull + (size_t)dev;
  SetupEntry* slot = nullptr;
  for (int probe = 0; probe < kSetupSlots; ++probe) {
    SetupEntry& c = g_setup[(h + probe) % kSetupSlots];
    if (c.kernel == kernel && c.device == dev) {
      slot = &c;
      break;
    }
    if (c.kernel == nullptr) {  // not cached yet: work it out into this slot
      e = allow_lds(kernel, lds_bytes);
      if (e != hipSuccess) return e;
      int cus = 0, bpc = 0;
      e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
      if (e != hipSuccess) return e;
      e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&bpc, kernel, threads, lds_bytes);
      if (e != hipSuccess) return e;
      c.kernel = kernel;
      c.device = dev;
      c.per_cu = bpc > 0 ? bpc : 1;
      c.num_cu = cus;
      slot = &c;
      break;
    }
  }
  if (!slot) return hipErrorOutOfMemory;  // more (kernel, device) pairs than slots
  if (per_cu) *per_cu = slot->per_cu;
  if (num_cu) *num_cu = slot->num_cu;
  return hipSuccess;
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

// Row counts beyond what any device holds are a valid size the library does
// not handle: below 2^46 elements per matrix every byte count and grid size
// in this file stays far from overflow.
constexpr int64_t kMaxElems = int64_t(1) << 46;
bool rows_fit(int64_t rows, int64_t width) { return width > 0 && rows <= kMaxElems / width; }

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

// n = 8192 keeps the two half tables of its two-pass forward (bfly_fwd8k.hip).
size_t coeff_bytes_l(int logn) { return logn == 13 ? bfly::table8k_bytes() : bfly::table_bytes(logn); }

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
  if (!aligned(codes, 16)) return BFLY_ERR_ALIGN;
  if (!aligned(scales, 2) || (zeros && !aligned(zeros, 2))) return BFLY_ERR_ALIGN;
  return BFLY_OK;
}

}  // namespace

// The fixed scratch of bfly_forward_quant_noalloc: room for the coefficient
// table of the longest butterfly the forward handles.  Every device the
// library runs on holds its own copy until the process ends.
constexpr int kScratchMaxLogN = 12;
constexpr size_t kScratchBytes = (bfly::table_bytes(kScratchMaxLogN) + 255) / 256 * 256;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

// scratch's device address, looked up once per device with that device
// current (the host-side name is only a stand-in for it).
constexpr int kMaxDevices = 64;
static std::mutex g_scratch_mu;
static void* g_scratch_ptr[kMaxDevices] = {};

static hipError_t scratch_address(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

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
  const hipError_t e = l == 13 ? bfly::launch_prepare_8192(theta, coeffs, false, (hipStream_t)hip_stream)
                               : bfly::launch_prepare(theta, coeffs, l, (hipStream_t)hip_stream);
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
  const hipError_t e = l == 13 ? bfly::launch_prepare_8192(nullptr, coeffs, true, (hipStream_t)hip_stream)
                               : bfly::launch_prepare(nullptr, coeffs, l, (hipStream_t)hip_stream, true);
  return e == hipSuccess ? BFLY_OK : hip_fail(e);
}

// Validates a forward call and fills its launch parameters (all but the
// table).  With coeffs == NULL the table is prepared from theta into the
// first bfly_coeff_bytes(nb) bytes of `workspace`.
static bfly_status forward_args(const void* x, bfly_dtype x_dt, void* y, bfly_dtype y_dt,
                                uint8_t* codes, uint16_t* scales, uint16_t* zeros, int64_t rows,
                                int32_t m, int32_t nb, const float* theta, const void* coeffs,
                                const float* mix, int32_t bits, int32_t group, bfly_qmode mode,
                                bool quant, const void* workspace, size_t workspace_bytes,
                                bfly::FwdParams* p) {
  if (rows > 0 && !x) return BFLY_ERR_NULL;
  if (!coeffs && (!theta || !workspace)) return BFLY_ERR_NULL;
  if (rows > 0 && !y && !quant) return BFLY_ERR_NULL;
  if (!dtype_ok(x_dt) || (y && !dtype_ok(y_dt))) return BFLY_ERR_DTYPE;
  if (rows < 0) return BFLY_ERR_SIZE;
  int lognb = 0;
  bfly_status st = check_n(nb, 13, &lognb);
  if (st != BFLY_OK) return st;
  const int64_t n = (int64_t)m * nb;
  if (n > 8192 || !rows_fit(rows, n)) return BFLY_ERR_UNSUPPORTED;
  if (quant) {
    st = check_quant(codes, scales, zeros, rows, n, nb, lognb, bits, group, mode);
    if (st != BFLY_OK) return st;
  }
  if (!bfly::forward_supported(lognb, m)) return BFLY_ERR_UNSUPPORTED;
  if (!coeffs && workspace_bytes < coeff_bytes_l(lognb)) return BFLY_ERR_WORKSPACE;
  if (!aligned(x, 16) || (y && !aligned(y, 16))) return BFLY_ERR_ALIGN;
  if ((coeffs && !aligned(coeffs, 16)) || (theta && !aligned(theta, 4)) ||
      (mix && !aligned(mix, 4)) || (!coeffs && !aligned(workspace, 16)))
    return BFLY_ERR_ALIGN;
  memset(p, 0, sizeof(*p));
  p->x = x;
  p->y = y;
  p->codes = quant ? codes : nullptr;
  p->scales = quant ? scales : nullptr;
  p->zeros = quant ? zeros : nullptr;
  p->mix = mix;
  p->rows = rows;
  p->m = m;
  p->lognb = lognb;
  p->x_bf16 = x_dt == BFLY_BF16;
  p->y_kind = !y ? bfly::Y_NONE : (y_dt == BFLY_BF16 ? bfly::Y_BF16 : bfly::Y_F32);
  p->bits = quant ? bits : 0;
  p->group = quant ? group : 0;
  p->asym = quant && mode == BFLY_ASYM_MINMAX;
  return BFLY_OK;
}

// Enqueues a validated forward: the table (prepared into `table_ws` from
// theta when coeffs is NULL), then the fused kernel.  Nothing for rows == 0.
static bfly_status forward_run(bfly::FwdParams& p, const float* theta, const void* coeffs,
                               void* table_ws, hipStream_t s) {
  if (p.rows == 0) return BFLY_OK;
  const void* tab = coeffs;
  if (!tab) {
    const hipError_t e = bfly::launch_prepare(theta, table_ws, p.lognb, s);
    if (e != hipSuccess) return hip_fail(e);
    tab = table_ws;
  }
  p.tab = bfly::table_at(tab, p.lognb);
  const hipError_t e = bfly::launch_forward(p, s);
  return e == hipSuccess ? BFLY_OK : hip_fail(e);
}

static bfly_status forward_common(const void* x, bfly_dtype x_dt, void* y, bfly_dtype y_dt,
                                  uint8_t* codes, uint16_t* scales, uint16_t* zeros, int64_t rows,
                                  int32_t m, int32_t nb, const float* theta, const void* coeffs,
                                  const float* mix, int32_t bits, int32_t group, bfly_qmode mode,
                                  bool quant, void* workspace, size_t workspace_bytes,
                                  void* hip_stream) {
  bfly::FwdParams p;
  const bfly_status st = forward_args(x, x_dt, y, y_dt, codes, scales, zeros, rows, m, nb, theta,
                                      coeffs, mix, bits, group, mode, quant, workspace,
                                      workspace_bytes, &p);
  if (st != BFLY_OK) return st;
  return forward_run(p, theta, coeffs, workspace, (hipStream_t)hip_stream);
}

// n = 8192 (two passes): the workspace always holds the fp32 rows between
// the passes, after the table area (used when the table comes from theta).
static size_t fwd8k_v_offset() { return align_up(coeff_bytes_l(13), 256); }

static bfly_status forward_8192(const void* x, bfly_dtype x_dt, void* y, bfly_dtype y_dt,
                                uint8_t* codes, uint16_t* scales, uint16_t* zeros, int64_t rows,
                                const float* theta, const void* coeffs, int32_t bits,
                                int32_t group, bfly_qmode mode, bool quant, void* workspace,
                                size_t workspace_bytes, void* hip_stream) {
  if (rows > 0 && !x) return BFLY_ERR_NULL;
  if (!coeffs && !theta) return BFLY_ERR_NULL;
  if (rows > 0 && !y && !quant) return BFLY_ERR_NULL;
  if (!workspace) return BFLY_ERR_NULL;
  if (!dtype_ok(x_dt) || (y && !dtype_ok(y_dt))) return BFLY_ERR_DTYPE;
  if (rows < 0) return BFLY_ERR_SIZE;
  if (!rows_fit(rows, 8192)) return BFLY_ERR_UNSUPPORTED;
  if (quant) {
    const bfly_status st = check_quant(codes, scales, zeros, rows, 8192, 8192, 13, bits, group, mode);
    if (st != BFLY_OK) return st;
  }
  if (workspace_bytes < fwd8k_v_offset() + (size_t)rows * 8192 * sizeof(float))
    return BFLY_ERR_WORKSPACE;
  if (!aligned(x, 16) || (y && !aligned(y, 16)) || !aligned(workspace, 16) ||
      (coeffs && !aligned(coeffs, 16)) || (theta && !aligned(theta, 4)))
    return BFLY_ERR_ALIGN;
  if (rows == 0) return BFLY_OK;
  const hipStream_t s = (hipStream_t)hip_stream;
  char* ws = static_cast<char*>(workspace);
  const void* tab = coeffs;
  if (!tab) {
    const hipError_t e = bfly::launch_prepare_8192(theta, ws, false, s);
    if (e != hipSuccess) return hip_fail(e);
    tab = ws;
  }
  bfly::Fwd8kParams p;
  p.x = x;
  p.x_bf16 = x_dt == BFLY_BF16;
  p.y = y;
  p.y_kind = !y ? bfly::Y_NONE : (y_dt == BFLY_BF16 ? bfly::Y_BF16 : bfly::Y_F32);
  p.codes = quant ? codes : nullptr;
  p.scales = quant ? scales : nullptr;
  p.zeros = quant ? zeros : nullptr;
  p.bits = quant ? bits : 0;
  p.group = quant ? group : 0;
  p.asym = quant && mode == BFLY_ASYM_MINMAX;
  p.rows = rows;
  p.table = tab;
  p.v = reinterpret_cast<float*>(ws + fwd8k_v_offset());
  const hipError_t e = bfly::launch_forward_8192(p, s);
  return e == hipSuccess ? BFLY_OK : hip_fail(e);
}

size_t bfly_forward_workspace_bytes(int64_t rows, int32_t n) {
  int l = 0;
  if (rows < 0 || check_n(n, 13, &l) != BFLY_OK || !rows_fit(rows, n)) return 0;
  if (l == 13) return fwd8k_v_offset() + (size_t)rows * 8192 * sizeof(float);
  return coeff_bytes_l(l);
}

bfly_status bfly_forward(const void* x, bfly_dtype x_dt, void* y, bfly_dtype y_dt, int64_t rows,
                         int32_t n, const float* theta, const void* coeffs, void* workspace,
                         size_t workspace_bytes, void* hip_stream) {
  if (rows > 0 && !y) return BFLY_ERR_NULL;
  if (n == 8192)
    return forward_8192(x, x_dt, y, y_dt, nullptr, nullptr, nullptr, rows, theta, coeffs, 0, 0,
                        BFLY_SYM_ABSMAX, false, workspace, workspace_bytes, hip_stream);
  return forward_common(x, x_dt, y, y_dt, nullptr, nullptr, nullptr, rows, 1, n, theta, coeffs,
                        nullptr, 0, 0, BFLY_SYM_ABSMAX, false, workspace, workspace_bytes,
                        hip_stream);
}

bfly_status bfly_forward_quant(const void* x, bfly_dtype x_dt, void* y, bfly_dtype y_dt,
                               uint8_t* codes, uint16_t* scales, uint16_t* zeros, int64_t rows,
                               int32_t n, const float* theta, const void* coeffs, int32_t bits,
                               int32_t group, bfly_qmode mode, void* workspace,
                               size_t workspace_bytes, void* hip_stream) {
  if (n == 8192)
    return forward_8192(x, x_dt, y, y_dt, codes, scales, zeros, rows, theta, coeffs, bits, group,
                        mode, true, workspace, workspace_bytes, hip_stream);
  return forward_common(x, x_dt, y, y_dt, codes, scales, zeros, rows, 1, n, theta, coeffs,
                        nullptr, bits, group, mode, true, workspace, workspace_bytes, hip_stream);
}

bfly_status bfly_kron_forward(const void* x, bfly_dtype x_dt, void* y, bfly_dtype y_dt,
                              uint8_t* codes, uint16_t* scales, uint16_t* zeros, int64_t rows,
                              int32_t m, int32_t nb, const float* theta_b, const void* coeffs_b,
                              const float* mix, int32_t bits, int32_t group, bfly_qmode mode,
                              void* workspace, size_t workspace_bytes, void* hip_stream) {
  if (!mix) return BFLY_ERR_NULL;
  if (m < 1 || m > 8) return BFLY_ERR_SIZE;
  if (!codes && (scales || zeros)) return BFLY_ERR_QUANT;
  if (log2_pow2(nb) >= 13) return BFLY_ERR_UNSUPPORTED;
  return forward_common(x, x_dt, y, y_dt, codes, scales, zeros, rows, m, nb, theta_b, coeffs_b,
                        mix, bits, group, mode, codes != nullptr, workspace, workspace_bytes,
                        hip_stream);
}

size_t bfly_backward_workspace_bytes(int64_t rows, int32_t n) {
  int l = 0;
  if (rows < 0 || check_n(n, 12, &l) != BFLY_OK || !rows_fit(rows, n)) return 0;
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
  if (!rows_fit(rows, n)) return BFLY_ERR_UNSUPPORTED;
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

// Workspace of the wide composite: the coefficient table (when prepared
// from theta_b), then v = (O kron I) x in fp32.
static size_t kron_wide_parts(int64_t rows, int32_t m, int lognb, size_t* o_v) {
  const size_t v = align_up(coeff_bytes_l(lognb), 256);
  if (o_v) *o_v = v;
  return v + (size_t)rows * (size_t)m * ((size_t)1 << lognb) * sizeof(float);
}

size_t bfly_kron_forward_wide_workspace_bytes(int64_t rows, int32_t m, int32_t nb) {
  int l = 0;
  if (rows < 0 || !kron_wide_sizes(m, nb, &l) || !rows_fit(rows, (int64_t)m * nb)) return 0;
  return kron_wide_parts(rows, m, l, nullptr);
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
  if (!kron_wide_sizes(m, nb, &l) || !rows_fit(rows, (int64_t)m * nb)) return BFLY_ERR_UNSUPPORTED;
  size_t o_v = 0;
  if (workspace_bytes < kron_wide_parts(rows, m, l, &o_v)) return BFLY_ERR_WORKSPACE;
  if (!aligned(x, 16) || !aligned(workspace, 16) || !aligned(mix, 4)) return BFLY_ERR_ALIGN;
  // v = (O kron I) x into the workspace, then the butterfly (and the
  // quantizer) on its rows * m segments: (O kron B) = (I kron B)(O kron I).
  // The second pass is validated in full before the first is enqueued.
  char* ws = static_cast<char*>(workspace);
  float* v = reinterpret_cast<float*>(ws + o_v);
  bfly::FwdParams p;
  const bfly_status st = forward_args(v, BFLY_F32, y, y_dt, codes, scales, zeros, rows * m, 1, nb,
                                      theta_b, coeffs_b, nullptr, bits, group, mode, quant, ws,
                                      o_v, &p);
  if (st != BFLY_OK) return st;
  if (rows == 0) return BFLY_OK;
  const hipStream_t s = (hipStream_t)hip_stream;
  if (bfly::kron_fused_supported(m, nb, x_dt == BFLY_BF16)) {
    // one pass: the mix, the butterfly and the quantizer per row (the
    // workspace holds only the table, when it comes from theta_b)
    const void* tab = coeffs_b;
    if (!tab) {
      const hipError_t e = bfly::launch_prepare(theta_b, ws, l, s);
      if (e != hipSuccess) return hip_fail(e);
      tab = ws;
    }
    bfly::KronFusedParams f;
    f.x = x;
    f.y = y;
    f.y_bf16 = y_dt == BFLY_BF16;
    f.codes = quant ? codes : nullptr;
    f.scales = quant ? scales : nullptr;
    f.zeros = quant ? zeros : nullptr;
    f.bits = quant ? bits : 0;
    f.group = quant ? group : 0;
    f.asym = quant && mode == BFLY_ASYM_MINMAX;
    f.mix = mix;
    f.cs = bfly::table_at(tab, l).cs;
    f.fgt = reinterpret_cast<const float*>(bfly::table_at(tab, l).fgt);
    f.rows = rows;
    f.m = m;
    const hipError_t e = bfly::launch_kron_fused(f, s);
    return e == hipSuccess ? BFLY_OK : hip_fail(e);
  }
  const hipError_t e = bfly::launch_kron_mix(x, x_dt == BFLY_BF16, v, mix, rows, m, nb, s);
  if (e != hipSuccess) return hip_fail(e);
  return forward_run(p, theta_b, coeffs_b, ws, s);
}

// Workspace of the Kronecker backward: O^T, then the butterfly backward's
// own workspace for the rows * m segments.
static size_t kron_bwd_parts(int64_t rows, int32_t m, int lognb, size_t* off_bwd) {
  const size_t bwd = align_up(sizeof(float) * (size_t)m * (size_t)m, 256);
  if (off_bwd) *off_bwd = bwd;
  return bwd + bfly_backward_workspace_bytes(rows * m, 1 << lognb);
}

size_t bfly_kron_backward_workspace_bytes(int64_t rows, int32_t m, int32_t nb) {
  int l = 0;
  if (rows < 0 || !kron_wide_sizes(m, nb, &l) || !rows_fit(rows, (int64_t)m * nb)) return 0;
  return kron_bwd_parts(rows, m, l, nullptr);
}

bfly_status bfly_kron_backward(const float* x, const float* g, float* dx, float* dtheta_b,
                               int64_t rows, int32_t m, int32_t nb, const float* theta_b,
                               const void* coeffs_b, const float* mix, void* workspace,
                               size_t workspace_bytes, void* hip_stream) {
  if ((rows > 0 && (!x || !g || !dx)) || !dtheta_b || !mix || !workspace) return BFLY_ERR_NULL;
  if (!theta_b && !coeffs_b) return BFLY_ERR_NULL;
  if (rows < 0) return BFLY_ERR_SIZE;
  if (m < 1 || m > 64) return BFLY_ERR_SIZE;
  int l = 0;
  const bfly_status st = check_n(nb, 12, &l);
  if (st != BFLY_OK) return st;
  // m = 1 is the plain butterfly (bfly_backward)
  if (m == 1 || !kron_wide_sizes(m, nb, &l) || !rows_fit(rows, (int64_t)m * nb))
    return BFLY_ERR_UNSUPPORTED;
  size_t o_bwd = 0;
  if (workspace_bytes < kron_bwd_parts(rows, m, l, &o_bwd)) return BFLY_ERR_WORKSPACE;
  if (!aligned(x, 16) || !aligned(g, 16) || !aligned(dx, 16) || !aligned(workspace, 16) ||
      !aligned(dtheta_b, 4) || !aligned(mix, 4) || (coeffs_b && !aligned(coeffs_b, 16)) ||
      (theta_b && !aligned(theta_b, 4)))
    return BFLY_ERR_ALIGN;
  if (rows > 0 && m <= bfly::kKronBwdFusedM && dx != g) {
    // One pass: the backward kernel forms (O^T kron I) G from G's segments
    // and O's columns as it loads them (the same fp32 values as the mixing
    // pass below).
    char* wsb = static_cast<char*>(workspace) + o_bwd;
    const void* tab = coeffs_b;
    if (!tab) {
      const hipError_t e = bfly::launch_prepare(theta_b, wsb, l, (hipStream_t)hip_stream);
      if (e != hipSuccess) return hip_fail(e);
      tab = wsb;
    }
    bfly::BwdParams p;
    memset(&p, 0, sizeof(p));
    p.x = x;
    p.g = g;
    p.dx = dx;
    p.partials = reinterpret_cast<float*>(wsb + align_up(coeff_bytes_l(l), 256));
    p.tab = bfly::table_at(tab, l);
    p.rows = rows * m;
    p.logn = l;
    p.nblk = bfly::backward_blocks(rows * m, l);
    p.mix = mix;
    p.m = m;
    const hipError_t e = bfly::launch_backward_kron(p, dtheta_b, (hipStream_t)hip_stream);
    return e == hipSuccess ? BFLY_OK : hip_fail(e);
  }
  const hipStream_t s = (hipStream_t)hip_stream;
  char* ws = static_cast<char*>(workspace);
  float* mix_t = reinterpret_cast<float*>(ws);
  hipError_t e = bfly::launch_kron_bwd_setup(mix, m, mix_t, s);  // O^T
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
  if (rows < 1 || check_n(n, 12, &l) != BFLY_OK || !rows_fit(rows, n)) return 0;
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
  if (!rows_fit(rows, n)) return BFLY_ERR_UNSUPPORTED;
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
  const bfly_status st =
      bfly_forward(x, BFLY_F32, y, BFLY_F32, rows, n, nullptr, wsb, nullptr, 0, hip_stream);
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

// Workspace of the layer-output calibration step (every part 256-aligned):
// the backward's own workspace (the coefficient table first), Xr = Q X,
// E (first W Q^T, then the quantizer's error), the weight codes, scales and
// zero points (sized for 4-bit codes and groups of 8), R = Xr E^T, G = dL/dXr,
// the group maxima of Xr, the histogram partials and log-bins, the sums of
// squares of R, dtheta.
struct CalibWParts {
  size_t bwd, xr, e, codes, scales, zeros, r, g, amax, hpart, lb, ss, dth, total;
};
static CalibWParts calib_w_parts(int64_t rows, int64_t out, int logn) {
  const size_t n = (size_t)1 << logn;
  CalibWParts o;
  size_t at = 0;
  auto take = [&](size_t bytes) {
    const size_t here = at;
    at = align_up(at + bytes, 256);
    return here;
  };
  o.bwd = take(bfly_backward_workspace_bytes(rows, (int32_t)n));
  o.xr = take((size_t)rows * n * sizeof(float));
  o.e = take((size_t)out * n * sizeof(float));
  o.codes = take((size_t)out * n / 2);
  o.scales = take((size_t)out * (n / 8) * 2);
  o.zeros = take((size_t)out * (n / 8) * 2);
  o.r = take((size_t)rows * (size_t)out * sizeof(float));
  o.g = take((size_t)rows * n * sizeof(float));
  o.amax = take((size_t)rows * (n / 8) * sizeof(float));
  o.hpart = take(sizeof(float) * (size_t)bfly::CALIB_MAX_BLOCKS * (bfly::CALIB_MAX_BINS + 1));
  o.lb = take(sizeof(float) * bfly::CALIB_MAX_BINS);
  o.ss = take(sizeof(float) * (size_t)bfly::gemm_f32_tiles(rows, (int32_t)out));
  o.dth = take(sizeof(float) * (size_t)logn * (n / 2));
  o.total = at;
  return o;
}

static bool calib_w_sizes(int64_t rows, int32_t out, int32_t n, int* logn) {
  if (rows < 1 || out < 16 || out % 16 != 0 || out > 65536) return false;
  if (check_n(n, 12, logn) != BFLY_OK) return false;
  if (!rows_fit(rows, n) || !rows_fit(rows, out)) return false;
  // every matrix of the products stays below 4 GiB
  if ((int64_t)out * n * 4 >= (int64_t(1) << 32)) return false;
  return true;
}

size_t bfly_calib_step_weight_workspace_bytes(int64_t rows, int32_t out, int32_t n) {
  int l = 0;
  if (!calib_w_sizes(rows, out, n, &l)) return 0;
  return calib_w_parts(rows, out, l).total;
}

bfly_status bfly_calib_step_weight(const float* x, int64_t rows, const void* w, bfly_dtype w_dt,
                                   int32_t out, int32_t n, float* theta, float* adam_m,
                                   float* adam_v, int32_t step,
                                   const bfly_calib_weight_config* cfg, float* loss,
                                   void* workspace, size_t workspace_bytes, void* hip_stream) {
  if (!x || !w || !theta || !adam_m || !adam_v || !cfg || !loss || !workspace) return BFLY_ERR_NULL;
  if (!dtype_ok(w_dt)) return BFLY_ERR_DTYPE;
  if (rows < 1 || step < 1 || out < 1) return BFLY_ERR_SIZE;
  int l = 0;
  const bfly_status sn = check_n(n, 12, &l);
  if (sn != BFLY_OK) return sn;
  if (!calib_w_sizes(rows, out, n, &l)) return BFLY_ERR_UNSUPPORTED;
  const int lg = log2_pow2(cfg->group);
  if ((cfg->bits != 2 && cfg->bits != 4) || lg < 3 || lg > 9 || cfg->group > n ||
      (cfg->mode != BFLY_SYM_ABSMAX && cfg->mode != BFLY_ASYM_MINMAX) || cfg->bins < 2 ||
      cfg->bins > bfly::CALIB_MAX_BINS || (cfg->bins & (cfg->bins - 1)) != 0)
    return BFLY_ERR_QUANT;
  const CalibWParts o = calib_w_parts(rows, out, l);
  if (workspace_bytes < o.total) return BFLY_ERR_WORKSPACE;
  if (!aligned(x, 16) || !aligned(w, 16) || !aligned(workspace, 16) || !aligned(theta, 4) ||
      !aligned(adam_m, 4) || !aligned(adam_v, 4) || !aligned(loss, 4))
    return BFLY_ERR_ALIGN;
  const hipStream_t s = (hipStream_t)hip_stream;
  char* ws = static_cast<char*>(workspace);
  char* wsb = ws + o.bwd;  // the backward's workspace; its table area holds the table
  float* xr = reinterpret_cast<float*>(ws + o.xr);
  float* e = reinterpret_cast<float*>(ws + o.e);
  uint8_t* codes = reinterpret_cast<uint8_t*>(ws + o.codes);
  uint16_t* scales = reinterpret_cast<uint16_t*>(ws + o.scales);
  uint16_t* zeros = cfg->mode == BFLY_ASYM_MINMAX ? reinterpret_cast<uint16_t*>(ws + o.zeros)
                                                  : nullptr;
  float* r = reinterpret_cast<float*>(ws + o.r);
  float* g = reinterpret_cast<float*>(ws + o.g);
  float* dth = reinterpret_cast<float*>(ws + o.dth);
  float* ss = reinterpret_cast<float*>(ws + o.ss);
  hipError_t err = bfly::launch_prepare(theta, wsb, l, s);
  if (err != hipSuccess) return hip_fail(err);
  // Xr = Q X; Wr = W Q^T with its group codes; E = What - Wr in place
  bfly_status st = bfly_forward(x, BFLY_F32, xr, BFLY_F32, rows, n, nullptr, wsb, nullptr, 0,
                                hip_stream);
  if (st != BFLY_OK) return st;
  st = bfly_forward_quant(w, w_dt, e, BFLY_F32, codes, scales, zeros, out, n, nullptr, wsb,
                          cfg->bits, cfg->group, (bfly_qmode)cfg->mode, nullptr, 0, hip_stream);
  if (st != BFLY_OK) return st;
  if ((err = bfly::launch_quant_residual(e, codes, scales, zeros, out, n, cfg->bits, cfg->group,
                                         zeros != nullptr, s)) != hipSuccess)
    return hip_fail(err);
  // the uniformity term on Xr: group maxima, log-bins, KL into loss[2]
  bfly::CalibLossParams p;
  p.y = xr;
  p.amax = reinterpret_cast<float*>(ws + o.amax);
  p.rows = rows;
  p.n = n;
  p.group = cfg->group;
  p.bits = 4;  // the histogram pass's own quantizer error is not used here
  p.bins = cfg->bins;
  p.lambda_kl = cfg->lambda_kl;
  p.partials = reinterpret_cast<float*>(ws + o.hpart);
  p.lb = reinterpret_cast<float*>(ws + o.lb);
  p.loss = loss;
  if ((err = bfly::launch_calib_hist(p, s)) != hipSuccess) return hip_fail(err);
  if ((err = bfly::launch_calib_reduce(p, s)) != hipSuccess) return hip_fail(err);
  // R = Xr E^T (= Yhat - Y), its sum of squares -> loss[0], loss[1]
  const double n_rec = (double)rows * (double)out;
  if ((err = bfly::launch_gemm_f32(xr, e, true, r, rows, out, n, 1.0f, ss, s)) != hipSuccess)
    return hip_fail(err);
  if ((err = bfly::launch_weight_loss(ss, bfly::gemm_f32_tiles(rows, out), n_rec, cfg->lambda_kl,
                                      loss, s)) != hipSuccess)
    return hip_fail(err);
  // G = dL/dXr = 2 R E / N_rec + the uniformity term's share
  if ((err = bfly::launch_gemm_f32(r, e, false, g, rows, n, out, (float)(2.0 / n_rec), nullptr,
                                   s)) != hipSuccess)
    return hip_fail(err);
  const double nx = (double)rows * (double)n;
  const float kl_scale =
      (float)(cfg->lambda_kl / (nx * (1.0 + cfg->bins * (double)bfly::kCalibSmooth))) /
      (2.f / cfg->bins);
  if ((err = bfly::launch_kl_grad_add(xr, p.amax, p.lb, g, rows * (int64_t)n, cfg->group,
                                      cfg->bins, kl_scale, s)) != hipSuccess)
    return hip_fail(err);
  // dtheta: the butterfly backward of X with G (dX written over G)
  st = bfly_backward(x, g, nullptr, g, dth, rows, n, nullptr, wsb,
                     wsb, bfly_backward_workspace_bytes(rows, n), hip_stream);
  if (st != BFLY_OK) return st;
  err = bfly::launch_adam(theta, adam_m, adam_v, dth, l * (n / 2), step, cfg->lr, cfg->beta1,
                          cfg->beta2, cfg->eps, s);
  return err == hipSuccess ? BFLY_OK : hip_fail(err);
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
  if (!rows_fit(rows, k) || !rows_fit(rows, n_out)) return BFLY_ERR_UNSUPPORTED;
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

bfly_status bfly_forward_quant_noalloc(const void* x, bfly_dtype x_dt, void* y, bfly_dtype y_dt,
                                       uint8_t* codes, uint16_t* scales, uint16_t* zeros,
                                       int64_t rows, int32_t n, const float* theta, int32_t bits,
                                       int32_t group, bfly_qmode mode, void* hip_stream) {
  if (!theta) return BFLY_ERR_NULL;
  // Validated as bfly_forward_quant with a workspace of the scratch's size;
  // the placeholder pointer is never dereferenced.
  bfly::FwdParams p;
  const bfly_status st =
      forward_args(x, x_dt, y, y_dt, codes, scales, zeros, rows, 1, n, theta, nullptr, nullptr,
                   bits, group, mode, true, reinterpret_cast<const void*>(uintptr_t(256)),
                   kScratchBytes, &p);
  if (st != BFLY_OK) return st;
  if (rows == 0) return BFLY_OK;
  void* table = nullptr;
  const hipError_t e = scratch_address(&table);
  if (e != hipSuccess) return hip_fail(e);
  return forward_run(p, theta, nullptr, table, (hipStream_t)hip_stream);
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
    default: break;
  }
  return "unknown status";
}

int32_t bfly_last_hip_error(void) { return g_last_hip_error; }

}  // extern "C"
