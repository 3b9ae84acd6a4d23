// Fused add-norm forward launchers: the norm of h = x + residual (fp32 sum),
// with the updated residual bf16(h) (RL-Kernel PR "C1: zero-centred RMSNorm
// references and CUDA kernel", decoder-norm note: the fused add normalises
// the fp32 sum). The kernel is in fwd_kernel.hpp.
#include "fwd_kernel.hpp"

namespace rmsn {

int launch_fwd_add(const FwdArgs& a, void* stream) {
  if (a.dt == kF16) return launch_fwd_add_f16(a, stream);
  if (a.D % 8 != 0) return launch_fwd_add_elem(a, stream);
  const fwd_detail::FwdLaunch f = fwd_detail::pick<kFwdAdd>(fwd_geom(a.D));
  if (f == nullptr) return static_cast<int>(hipErrorInvalidValue);
  return f(a, stream);
}

}  // namespace rmsn
