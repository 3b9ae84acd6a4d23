// Gated backward launchers for fp16 activations, rows whose length is a
// multiple of 8 (the chain rule of the gated forward is spelled out in
// bwd_kernel.hpp).
#include "bwd_kernel.hpp"

namespace rmsn {

int launch_bwd_rows_gated_f16(const BwdArgs& a, void* stream) {
  if (a.D % 8 != 0) return launch_bwd_rows_gated_elem_f16(a, stream);
  const RowGeom g = bwd_geom(a.D);
  bwd_detail::RowsLaunch f = nullptr;
  if (a.act == kGateSilu) f = bwd_detail::pick<kBwdGatedSilu, kF16>(g);
  else if (a.act == kGateSigmoid) f = bwd_detail::pick<kBwdGatedSigmoid, kF16>(g);
  if (f == nullptr) return static_cast<int>(hipErrorInvalidValue);
  return f(a, stream);
}

}  // namespace rmsn
