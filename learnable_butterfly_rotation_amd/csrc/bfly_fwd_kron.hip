// Instantiations of the forward kernel for Kronecker composites n = m * nb,
// one object per segment count m (compiled with -DKRON_M=m, m = 2 .. 8),
// for nb = 256 .. 4096 with m * nb <= 8192.
#include "bfly_fwd_kernel.h"

#ifndef KRON_M
#error "compile once per segment count with -DKRON_M=<m>"
#endif

namespace bfly {

#define BFLY_CAT2(a, b) a##b
#define BFLY_CAT(a, b) BFLY_CAT2(a, b)

template <int LOGNB>
static hipError_t kron(const FwdParams& p, hipStream_t s) {
  if constexpr ((KRON_M << LOGNB) <= 8192) {
    return p.x_bf16 ? launch_fwd_inst<LOGNB, KRON_M, 1, true>(p, s)
                    : launch_fwd_inst<LOGNB, KRON_M, 1, false>(p, s);
  } else {
    return hipErrorInvalidValue;
  }
}

hipError_t BFLY_CAT(launch_forward_kron_m, KRON_M)(const FwdParams& p, hipStream_t s) {
  switch (p.lognb) {
    case 8: return kron<8>(p, s);
    case 9: return kron<9>(p, s);
    case 10: return kron<10>(p, s);
    case 11: return kron<11>(p, s);
    case 12: return kron<12>(p, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace bfly
