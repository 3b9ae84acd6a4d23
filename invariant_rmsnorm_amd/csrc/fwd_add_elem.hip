// Fused add-norm forward launcher for rows whose length D is not a multiple
// of 8: the kernel of fwd_kernel.hpp with rows of any alignment (bf16).
#include "fwd_kernel.hpp"

namespace rmsn {

int launch_fwd_add_elem(const FwdArgs& a, void* stream) {
  const fwd_detail::FwdLaunch f = fwd_detail::pick<kFwdAdd, kBf16E>(fwd_geom(a.D));
  if (f == nullptr) return static_cast<int>(hipErrorInvalidValue);
  return f(a, stream);
}

}  // namespace rmsn
