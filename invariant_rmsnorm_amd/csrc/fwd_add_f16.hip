// Fused add-norm forward launchers for fp16 activations, rows of any length:
// the norm of h = x + residual (fp32 sum) with the updated residual fp16(h).
// The kernel is in fwd_kernel.hpp.
#include "fwd_kernel.hpp"

namespace rmsn {

int launch_fwd_add_f16(const FwdArgs& a, void* stream) {
  const RowGeom g = fwd_geom(a.D);
  const fwd_detail::FwdLaunch f = a.D % 8 != 0 ? fwd_detail::pick<kFwdAdd, kF16E>(g)
                                               : fwd_detail::pick<kFwdAdd, kF16>(g);
  if (f == nullptr) return static_cast<int>(hipErrorInvalidValue);
  return f(a, stream);
}

}  // namespace rmsn
