// Forward launchers for rows whose length D is not a multiple of 8 (plain
// and residual-copy forms, bf16 or fp16 activations): the kernel of
// fwd_kernel.hpp with rows of any alignment (unaligned 16-byte accesses, the
// partial last group element by element). The arithmetic and the reduction
// tree are those of 16-byte rows of ceil(D/8) groups.
#include "fwd_kernel.hpp"

namespace rmsn {

int launch_fwd_elem(const FwdArgs& a, void* stream) {
  const RowGeom g = fwd_geom(a.D);
  const fwd_detail::FwdLaunch f =
      a.dt == kF16 ? fwd_detail::pick<0, kF16E>(g) : fwd_detail::pick<0, kBf16E>(g);
  if (f == nullptr) return static_cast<int>(hipErrorInvalidValue);
  return f(a, stream);
}

}  // namespace rmsn
