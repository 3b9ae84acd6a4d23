// Forward launchers for fp16 activations (plain and residual-copy forms; the
// contract of RL-Kernel PR "C1: zero-centred RMSNorm references and CUDA
// kernel" checks fp16 beside bf16). The kernel is in fwd_kernel.hpp.
#include "fwd_kernel.hpp"

namespace rmsn {

int launch_fwd_f16(const FwdArgs& a, void* stream) {
  const fwd_detail::FwdLaunch f = fwd_detail::pick<0, kF16>(fwd_geom(a.D));
  if (f == nullptr) return static_cast<int>(hipErrorInvalidValue);
  return f(a, stream);
}

}  // namespace rmsn
