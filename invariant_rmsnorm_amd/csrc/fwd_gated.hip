// Gated forward launchers (RL-Kernel PR "C1: zero-centred RMSNorm references
// and CUDA kernel": silu or sigmoid gate; weight multiply in fp32, or the
// cast-to-input-dtype rounding convention).
#include "fwd_kernel.hpp"

namespace rmsn {

int launch_fwd_gated(const FwdArgs& a, void* stream) {
  if (a.dt == kF16) return launch_fwd_gated_f16(a, stream);
  if (a.D % 8 != 0) return launch_fwd_gated_elem(a, stream);
  using namespace fwd_detail;
  const RowGeom g = fwd_geom(a.D);
  FwdLaunch f = nullptr;
  switch (fwd_gate_code(true, a.act, a.cast != 0)) {
    case fwd_gate_code(true, kGateSilu, false): f = pick<fwd_gate_code(true, kGateSilu, false)>(g); break;
    case fwd_gate_code(true, kGateSigmoid, false): f = pick<fwd_gate_code(true, kGateSigmoid, false)>(g); break;
    case fwd_gate_code(true, kGateSilu, true): f = pick<fwd_gate_code(true, kGateSilu, true)>(g); break;
    case fwd_gate_code(true, kGateSigmoid, true): f = pick<fwd_gate_code(true, kGateSigmoid, true)>(g); break;
    default: break;
  }
  if (f == nullptr) return static_cast<int>(hipErrorInvalidValue);
  return f(a, stream);
}

}  // namespace rmsn
