// Gated backward launchers: dx, dz and the dgamma partials of the gated norm
// (the gate's forward is in RL-Kernel PR "C1: zero-centred RMSNorm references
// and CUDA kernel"; its backward is the chain rule, spelled out in
// bwd_kernel.hpp).
#include "bwd_kernel.hpp"

namespace rmsn {

int launch_bwd_rows_gated(const BwdArgs& a, void* stream) {
  if (a.dt == kF16) return launch_bwd_rows_gated_f16(a, stream);
  if (a.D % 8 != 0) return launch_bwd_rows_gated_elem(a, stream);
  const RowGeom g = bwd_geom(a.D);
  bwd_detail::RowsLaunch f = nullptr;
  if (a.act == kGateSilu) f = bwd_detail::pick<kBwdGatedSilu>(g);
  else if (a.act == kGateSigmoid) f = bwd_detail::pick<kBwdGatedSigmoid>(g);
  if (f == nullptr) return static_cast<int>(hipErrorInvalidValue);
  return f(a, stream);
}

}  // namespace rmsn
