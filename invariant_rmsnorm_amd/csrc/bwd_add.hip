// Fused add-norm backward launchers: dh (the gradient of both x and the
// residual input, plus the gradient arriving at the updated residual) and
// the dgamma partials, with h = x + residual recomputed in fp32 (RL-Kernel PR
// "C1: zero-centred RMSNorm references and CUDA kernel", decoder-norm note).
// The kernel template is in bwd_kernel.hpp.
#include "bwd_kernel.hpp"

namespace rmsn {

int launch_bwd_rows_add(const BwdArgs& a, void* stream) {
  if (a.dt == kF16) return launch_bwd_rows_add_f16(a, stream);
  if (a.D % 8 != 0) return launch_bwd_rows_add_elem(a, stream);
  const RowGeom g = bwd_geom(a.D);
  const bwd_detail::RowsLaunch f =
      a.gres != nullptr ? bwd_detail::pick<kBwdAddGres>(g) : bwd_detail::pick<kBwdAdd>(g);
  if (f == nullptr) return static_cast<int>(hipErrorInvalidValue);
  return f(a, stream);
}

}  // namespace rmsn
