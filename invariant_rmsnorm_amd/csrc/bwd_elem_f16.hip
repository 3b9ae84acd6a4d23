// Backward rows launchers for rows whose length D is not a multiple of 8,
// fp16 activations (plain and residual-gradient forms).
#include "bwd_kernel.hpp"

namespace rmsn {

int launch_bwd_rows_elem_f16(const BwdArgs& a, void* stream) {
  const RowGeom g = bwd_geom(a.D);
  const bwd_detail::RowsLaunch f = a.gres != nullptr ? bwd_detail::pick<kBwdGres, kF16E>(g)
                                                     : bwd_detail::pick<kBwdPlain, kF16E>(g);
  if (f == nullptr) return static_cast<int>(hipErrorInvalidValue);
  return f(a, stream);
}

}  // namespace rmsn
