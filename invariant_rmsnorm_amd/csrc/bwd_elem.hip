// Backward rows launchers for rows whose length D is not a multiple of 8,
// bf16 activations (plain and residual-gradient forms): the kernel of
// bwd_kernel.hpp with rows of any alignment (fp16 in bwd_elem_f16.hip).
#include "bwd_kernel.hpp"

namespace rmsn {

int launch_bwd_rows_elem(const BwdArgs& a, void* stream) {
  if (a.dt == kF16) return launch_bwd_rows_elem_f16(a, stream);
  const RowGeom g = bwd_geom(a.D);
  const bwd_detail::RowsLaunch f = a.gres != nullptr ? bwd_detail::pick<kBwdGres, kBf16E>(g)
                                                     : bwd_detail::pick<kBwdPlain, kBf16E>(g);
  if (f == nullptr) return static_cast<int>(hipErrorInvalidValue);
  return f(a, stream);
}

}  // namespace rmsn
