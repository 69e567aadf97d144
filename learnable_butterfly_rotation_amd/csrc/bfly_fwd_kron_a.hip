// Instantiations of the forward kernel for Kronecker composites (m = 2, 3, 4).
#include "bfly_fwd_kernel.h"

namespace bfly {

template <int LOGNB, int M>
static hipError_t kron(const FwdParams& p, hipStream_t s) {
  return p.x_bf16 ? launch_fwd_inst<LOGNB, M, true>(p, s) : launch_fwd_inst<LOGNB, M, false>(p, s);
}

hipError_t launch_forward_kron_a(const FwdParams& p, hipStream_t s) {
  switch (p.m * 16 + p.lognb) {
    case 2 * 16 + 8: return kron<8, 2>(p, s);
    case 2 * 16 + 9: return kron<9, 2>(p, s);
    case 2 * 16 + 10: return kron<10, 2>(p, s);
    case 2 * 16 + 11: return kron<11, 2>(p, s);
    case 2 * 16 + 12: return kron<12, 2>(p, s);
    case 3 * 16 + 8: return kron<8, 3>(p, s);
    case 3 * 16 + 9: return kron<9, 3>(p, s);
    case 3 * 16 + 10: return kron<10, 3>(p, s);
    case 3 * 16 + 11: return kron<11, 3>(p, s);
    case 4 * 16 + 8: return kron<8, 4>(p, s);
    case 4 * 16 + 9: return kron<9, 4>(p, s);
    case 4 * 16 + 10: return kron<10, 4>(p, s);
    case 4 * 16 + 11: return kron<11, 4>(p, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace bfly
