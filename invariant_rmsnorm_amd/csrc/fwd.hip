// Forward launchers: the plain and residual-copy forms here, the gated forms
// in fwd_gated.hip, the fused add-norm in fwd_add.hip, fp16 activations in
// fwd_f16.hip. The kernel itself is in fwd_kernel.hpp.
#include "fwd_kernel.hpp"

namespace rmsn {

int launch_fwd(const FwdArgs& a, void* stream) {
  if (a.T == 0) return 0;
  if (a.z != nullptr) return launch_fwd_gated(a, stream);
  if (a.rin != nullptr) return launch_fwd_add(a, stream);
  if (a.D % 8 != 0) return launch_fwd_elem(a, stream);
  if (a.dt == kF16) return launch_fwd_f16(a, stream);
  const fwd_detail::FwdLaunch f = fwd_detail::pick<0>(fwd_geom(a.D));
  if (f == nullptr) return static_cast<int>(hipErrorInvalidValue);
  return f(a, stream);
}

}  // namespace rmsn
