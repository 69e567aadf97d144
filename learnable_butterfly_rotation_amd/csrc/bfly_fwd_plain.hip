// Instantiations of the forward kernel for plain butterflies, n = 64 .. 4096.
#include "bfly_fwd_kernel.h"

namespace bfly {

// Rows per thread: two rows in flight per thread give each wave independent
// work to overlap with its own LDS and barrier waits.  Measured at n = 4096
// (one row per 8-wave workgroup): 41 vs 45 us for 8192 rows; at n = 128 ...
// 2048 (90 M elements, INT4 g128): 3-10 % faster for fp32 and bf16 input; at
// n = 64 one row per thread is faster (116 vs 120 us fp32, 82 vs 94 us bf16).
template <int LOGNB>
static hipError_t plain(const FwdParams& p, hipStream_t s) {
  constexpr int RPT = LOGNB >= 7 ? 2 : 1;
  return p.x_bf16 ? launch_fwd_inst<LOGNB, 1, RPT, true>(p, s)
                  : launch_fwd_inst<LOGNB, 1, RPT, false>(p, s);
}

hipError_t launch_forward_plain(const FwdParams& p, hipStream_t s) {
  switch (p.lognb) {
    case 6: return plain<6>(p, s);
    case 7: return plain<7>(p, s);
    case 8: return plain<8>(p, s);
    case 9: return plain<9>(p, s);
    case 10: return plain<10>(p, s);
    case 11: return plain<11>(p, s);
    case 12: return plain<12>(p, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace bfly
