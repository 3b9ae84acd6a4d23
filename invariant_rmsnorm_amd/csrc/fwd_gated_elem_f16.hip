// Gated forward launchers for fp16 activations in rows whose length D is not
// a multiple of 8, rows of any alignment (the
// contract of RL-Kernel PR "C1: zero-centred RMSNorm references and CUDA
// kernel" checks fp16 beside bf16; the cast convention rounds to fp16 there).
// The kernel is in fwd_kernel.hpp.
#include "fwd_kernel.hpp"

namespace rmsn {

namespace {

template <int DT>
fwd_detail::FwdLaunch pick_gated(const FwdArgs& a, const RowGeom& g) {
  using namespace fwd_detail;
  switch (fwd_gate_code(true, a.act, a.cast != 0)) {
    case fwd_gate_code(true, kGateSilu, false): return pick<fwd_gate_code(true, kGateSilu, false), DT>(g);
    case fwd_gate_code(true, kGateSigmoid, false): return pick<fwd_gate_code(true, kGateSigmoid, false), DT>(g);
    case fwd_gate_code(true, kGateSilu, true): return pick<fwd_gate_code(true, kGateSilu, true), DT>(g);
    case fwd_gate_code(true, kGateSigmoid, true): return pick<fwd_gate_code(true, kGateSigmoid, true), DT>(g);
    default: return nullptr;
  }
}

}  // namespace

int launch_fwd_gated_elem_f16(const FwdArgs& a, void* stream) {
  const fwd_detail::FwdLaunch f = pick_gated<kF16E>(a, fwd_geom(a.D));
  if (f == nullptr) return static_cast<int>(hipErrorInvalidValue);
  return f(a, stream);
}

}  // namespace rmsn
