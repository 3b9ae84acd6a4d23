// Fused add-norm backward rows launchers for fp16 activations, rows of any
// length (h = x + residual recomputed in fp32; bwd_kernel.hpp).
#include "bwd_kernel.hpp"

namespace rmsn {

int launch_bwd_rows_add_f16(const BwdArgs& a, void* stream) {
  const RowGeom g = bwd_geom(a.D);
  bwd_detail::RowsLaunch f = nullptr;
  if (a.D % 8 != 0)
    f = a.gres != nullptr ? bwd_detail::pick<kBwdAddGres, kF16E>(g) : bwd_detail::pick<kBwdAdd, kF16E>(g);
  else
    f = a.gres != nullptr ? bwd_detail::pick<kBwdAddGres, kF16>(g) : bwd_detail::pick<kBwdAdd, kF16>(g);
  if (f == nullptr) return static_cast<int>(hipErrorInvalidValue);
  return f(a, stream);
}

}  // namespace rmsn
