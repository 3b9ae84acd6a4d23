// Backward rows launchers for fp16 activations (plain and residual-gradient
// forms). The kernel template is in bwd_kernel.hpp.
#include "bwd_kernel.hpp"

namespace rmsn {

int launch_bwd_rows_f16(const BwdArgs& a, void* stream) {
  const RowGeom g = bwd_geom(a.D);
  const bwd_detail::RowsLaunch f = a.gres != nullptr ? bwd_detail::pick<kBwdGres, kF16>(g)
                                                     : bwd_detail::pick<kBwdPlain, kF16>(g);
  if (f == nullptr) return static_cast<int>(hipErrorInvalidValue);
  return f(a, stream);
}

}  // namespace rmsn
