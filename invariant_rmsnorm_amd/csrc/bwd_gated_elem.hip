// Gated backward launchers for rows whose length D is not a multiple of 8:
// the kernel of bwd_kernel.hpp (gated modes, the chain rule of the gated
// forward spelled out there) with rows of any alignment (bf16).
#include "bwd_kernel.hpp"

namespace rmsn {

int launch_bwd_rows_gated_elem(const BwdArgs& a, void* stream) {
  const RowGeom g = bwd_geom(a.D);
  bwd_detail::RowsLaunch f = nullptr;
  if (a.act == kGateSilu) f = bwd_detail::pick<kBwdGatedSilu, kBf16E>(g);
  else if (a.act == kGateSigmoid) f = bwd_detail::pick<kBwdGatedSigmoid, kBf16E>(g);
  if (f == nullptr) return static_cast<int>(hipErrorInvalidValue);
  return f(a, stream);
}

}  // namespace rmsn
