// Fused add-norm backward rows launchers for rows whose length D is not a
// multiple of 8: the kernel of bwd_kernel.hpp with rows of any alignment
// (bf16).
#include "bwd_kernel.hpp"

namespace rmsn {

int launch_bwd_rows_add_elem(const BwdArgs& a, void* stream) {
  const RowGeom g = bwd_geom(a.D);
  const bwd_detail::RowsLaunch f = a.gres != nullptr ? bwd_detail::pick<kBwdAddGres, kBf16E>(g)
                                                     : bwd_detail::pick<kBwdAdd, kBf16E>(g);
  if (f == nullptr) return static_cast<int>(hipErrorInvalidValue);
  return f(a, stream);
}

}  // namespace rmsn
