// Gated backward launchers for fp16 activations in rows whose length D is not
// a multiple of 8 (rows of any alignment).
#include "bwd_kernel.hpp"

namespace rmsn {

int launch_bwd_rows_gated_elem_f16(const BwdArgs& a, void* stream) {
  const RowGeom g = bwd_geom(a.D);
  bwd_detail::RowsLaunch f = nullptr;
  if (a.act == kGateSilu) f = bwd_detail::pick<kBwdGatedSilu, kF16E>(g);
  else if (a.act == kGateSigmoid) f = bwd_detail::pick<kBwdGatedSigmoid, kF16E>(g);
  if (f == nullptr) return static_cast<int>(hipErrorInvalidValue);
  return f(a, stream);
}

}  // namespace rmsn
