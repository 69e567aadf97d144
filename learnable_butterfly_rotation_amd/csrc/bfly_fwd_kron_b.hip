// Instantiations of the forward kernel for Kronecker composites (m = 5, 6, 7, 8).
#include "bfly_fwd_kernel.h"

namespace bfly {

template <int LOGNB, int M>
static hipError_t kron(const FwdParams& p, hipStream_t s) {
  return p.x_bf16 ? launch_fwd_inst<LOGNB, M, true>(p, s) : launch_fwd_inst<LOGNB, M, false>(p, s);
}

hipError_t launch_forward_kron_b(const FwdParams& p, hipStream_t s) {
  switch (p.m * 16 + p.lognb) {
    case 5 * 16 + 8: return kron<8, 5>(p, s);
    case 5 * 16 + 9: return kron<9, 5>(p, s);
    case 5 * 16 + 10: return kron<10, 5>(p, s);
    case 6 * 16 + 8: return kron<8, 6>(p, s);
    case 6 * 16 + 9: return kron<9, 6>(p, s);
    case 6 * 16 + 10: return kron<10, 6>(p, s);
    case 7 * 16 + 8: return kron<8, 7>(p, s);
    case 7 * 16 + 9: return kron<9, 7>(p, s);
    case 7 * 16 + 10: return kron<10, 7>(p, s);
    case 8 * 16 + 8: return kron<8, 8>(p, s);
    case 8 * 16 + 9: return kron<9, 8>(p, s);
    case 8 * 16 + 10: return kron<10, 8>(p, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace bfly
