// Instantiations of the forward kernel for plain butterflies, n = 64 .. 4096.
#include "bfly_fwd_kernel.h"

namespace bfly {

// One row per thread: measured faster than two in lockstep at n = 4096.
template <int LOGNB>
static hipError_t plain(const FwdParams& p, hipStream_t s) {
  return p.x_bf16 ? launch_fwd_inst<LOGNB, 1, 1, true>(p, s) : launch_fwd_inst<LOGNB, 1, 1, false>(p, s);
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
