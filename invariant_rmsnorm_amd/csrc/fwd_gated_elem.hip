// Gated forward launchers for rows whose length D is not a multiple of 8:
// the kernel of fwd_kernel.hpp with rows of any alignment (bf16).
#include "fwd_kernel.hpp"

namespace rmsn {

int launch_fwd_gated_elem(const FwdArgs& a, void* stream) {
  using namespace fwd_detail;
  const RowGeom g = fwd_geom(a.D);
  FwdLaunch f = nullptr;
  switch (fwd_gate_code(true, a.act, a.cast != 0)) {
    case fwd_gate_code(true, kGateSilu, false):
      f = pick<fwd_gate_code(true, kGateSilu, false), kBf16E>(g);
      break;
    case fwd_gate_code(true, kGateSigmoid, false):
      f = pick<fwd_gate_code(true, kGateSigmoid, false), kBf16E>(g);
      break;
    case fwd_gate_code(true, kGateSilu, true):
      f = pick<fwd_gate_code(true, kGateSilu, true), kBf16E>(g);
      break;
    case fwd_gate_code(true, kGateSigmoid, true):
      f = pick<fwd_gate_code(true, kGateSigmoid, true), kBf16E>(g);
      break;
    default: break;
  }
  if (f == nullptr) return static_cast<int>(hipErrorInvalidValue);
  return f(a, stream);
}

}  // namespace rmsn
